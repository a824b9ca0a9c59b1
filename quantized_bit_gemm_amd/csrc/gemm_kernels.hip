// gemm_kernels.hip -- the decode-sized 8-bit scaled GEMM family for gfx950.
//
// One kernel template covers the three formats and the algorithmic variants
// that the pages fold into a single GEMM implementation with tunable
// parameters ("Helion DSL added to vLLM to autotune linear inference
// backends", signaltitans.com, "Unified GEMM Architecture"; "Helion nel
// backend vLLM", ai-radar.it, paragraphs 2-3):
//   - FP8 Dynamic: E4M3 x E4M3 on the matrix cores, fp32 accumulation,
//     per-token x per-channel dequantization in the epilogue;
//   - W8A8 INT8: int8 x int8, exact int32 accumulation, same epilogue;
//   - Block FP8: every 128-wide K step is one 16x16x128 MFMA whose result is
//     scaled by a_scale[m,g] * w_scale[n/128,g] and added to the accumulator;
//   - Standard vs Swap-AB (A@B computed as (B^T A^T)^T): which operand fills
//     the matrix core's row slot; Swap-AB puts the weight rows there and the
//     tokens in the column slot, and the epilogue writes the transpose;
//   - Split-K: grid.y cuts K into split_k equal chunks; partial results go to
//     a workspace and the last workgroup of each tile to arrive sums them in
//     chunk order (deterministic) and applies the epilogue, so no second
//     launch is needed.  The arrival counter is reset by that workgroup.
//
// Why this shape on MI355X.  At M <= 32 the GEMM reads N*K weight bytes once
// and does ~2M flops per byte, far below the matrix-core ridge, so it is
// bound by HBM bandwidth: the design goal is to keep enough 16-byte weight
// loads in flight on all 256 CUs.  Each lane streams 2 x 16 contiguous bytes
// of one weight row per 128-wide K step straight into the MFMA operand
// registers (the K positions inside a step are assigned identically for both
// operands, so any assignment gives the same dot product; the chosen one
// makes every load instruction read 16 rows x 64 contiguous bytes).  A wave
// keeps KU steps of NT 16-row sub-tiles in flight; WK waves of a workgroup
// split the K chunk and are reduced through LDS; WN waves sit side by side
// along N.  The activation rows (<= 32 x K bytes) are re-read from L2 by
// every wave.  Weights are never staged through LDS: each weight byte is
// used by exactly one lane, so LDS would add a copy without reuse.
#include "qbg_device.h"
#include "qbg_launch.h"

namespace qbg {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

template <int OP>
struct Acc;
template <>
struct Acc<OP_FP8> { using vec = v4f; using scalar = float; };
template <>
struct Acc<OP_INT8> { using vec = v4i; using scalar = int; };
template <>
struct Acc<OP_BLOCK_F32> { using vec = v4f; using scalar = float; };
template <>
struct Acc<OP_BLOCK_UE8M0> { using vec = v4f; using scalar = float; };

__device__ __forceinline__ uint4 ld16(const uint8_t* p) {
    return *reinterpret_cast<const uint4*>(p);
}

// One 128-wide K step: D += X * Y^T over 128 K positions, X supplying the
// 16 rows of D and Y its 16 columns.  Each operand is two 16-byte chunks per
// lane (lane l: row/column l % 16, K positions 16*(l/16) + [0,16) and
// 64 + 16*(l/16) + [0,16) of the step).
template <int OP>
__device__ __forceinline__ typename Acc<OP>::vec mma_step(const uint4& xl, const uint4& xh,
                                                          const uint4& yl, const uint4& yh,
                                                          typename Acc<OP>::vec c) {
    if constexpr (OP == OP_INT8) {
        const v4i x0 = {(int)xl.x, (int)xl.y, (int)xl.z, (int)xl.w};
        const v4i x1 = {(int)xh.x, (int)xh.y, (int)xh.z, (int)xh.w};
        const v4i y0 = {(int)yl.x, (int)yl.y, (int)yl.z, (int)yl.w};
        const v4i y1 = {(int)yh.x, (int)yh.y, (int)yh.z, (int)yh.w};
        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(x0, y0, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(x1, y1, c, 0, 0, 0);
        return c;
    } else {
        const v8i x = {(int)xl.x, (int)xl.y, (int)xl.z, (int)xl.w,
                       (int)xh.x, (int)xh.y, (int)xh.z, (int)xh.w};
        const v8i y = {(int)yl.x, (int)yl.y, (int)yl.z, (int)yl.w,
                       (int)yh.x, (int)yh.y, (int)yh.z, (int)yh.w};
        // operand formats 0/0 = E4M3 x E4M3; zero scale operands select the unscaled MFMA
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, c, 0, 0, 0, 0, 0, 0);
    }
}

template <int OP>
__device__ __forceinline__ float block_scale(const void* s, int64_t idx) {
    if constexpr (OP == OP_BLOCK_UE8M0)
        return ue8m0_value(reinterpret_cast<const uint8_t*>(s)[idx]);
    else
        return reinterpret_cast<const float*>(s)[idx];
}

template <int OP>
__device__ __forceinline__ void store_out(const GemmArgs& p, int t, int n,
                                          typename Acc<OP>::scalar v) {
    const int64_t o = (int64_t)t * p.N + n;
    if constexpr (OP == OP_INT8) {
        if (p.raw_i32) {
            reinterpret_cast<int*>(p.out)[o] = v;
            return;
        }
    }
    float f = (float)v;
    if constexpr (OP == OP_FP8 || OP == OP_INT8)
        f = f * reinterpret_cast<const float*>(p.a_scale)[t] *
            reinterpret_cast<const float*>(p.w_scale)[n];
    reinterpret_cast<uint16_t*>(p.out)[o] = (uint16_t)f32_to_bf16(f);
}

template <int OP, bool SWAP, int NT, int MT, int WN, int WK, int KU>
__global__ __launch_bounds__(64 * WN * WK) void gemm_kernel(const GemmArgs p) {
    using AccV = typename Acc<OP>::vec;
    using AccS = typename Acc<OP>::scalar;
    constexpr bool BLOCK = (OP == OP_BLOCK_F32 || OP == OP_BLOCK_UE8M0);
    constexpr int TN = 16 * NT * WN;  // weight rows per workgroup
    constexpr int TNP = TN + 1;       // padded LDS row

    extern __shared__ char smem_raw[];
    AccS* red = reinterpret_cast<AccS*>(smem_raw);  // [WK][M][TNP]
    __shared__ int s_last;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wn = wave % WN, wk = wave / WN;
    const int r16 = lane & 15, g4 = lane >> 4;
    const int tile = blockIdx.x, split = blockIdx.y;
    const int M = p.M, N = p.N;
    const int64_t K = p.K;
    const int n_wave = tile * TN + wn * 16 * NT;
    const int64_t k_begin = (int64_t)split * p.k_chunk;
    const int chunk = p.k_chunk;
    const int nsteps = (chunk + 127) / 128;
    const int full_steps = chunk / 128;

    AccV acc[NT][MT];
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[j][mt] = AccV{0, 0, 0, 0};

    const uint8_t* wp[NT];
    bool wlive[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int n = n_wave + 16 * j;
        wlive[j] = n < N;  // uniform across the wave (N % 16 == 0)
        wp[j] = p.w + (int64_t)(wlive[j] ? n + r16 : 0) * K + k_begin + g4 * 16;
    }
    const uint8_t* ap[MT];
    bool alive[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int t = 16 * mt + r16;
        alive[mt] = t < M;
        ap[mt] = p.a + (int64_t)(alive[mt] ? t : 0) * K + k_begin + g4 * 16;
    }
    const uint4 z4 = {0u, 0u, 0u, 0u};

    // Scale factors of one block step for each (sub-tile, token slot, acc element).
    auto apply_block = [&](int step, AccV (&tmp)[NT][MT]) __attribute__((always_inline)) {
        if constexpr (BLOCK) {
            const int64_t g = (k_begin >> 7) + step;
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                if (!wlive[j]) continue;
                const float ws = block_scale<OP>(p.w_scale, (int64_t)((n_wave + 16 * j) >> 7) * p.kgroups + g);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    if constexpr (SWAP) {
                        const int t = 16 * mt + r16;
                        const float f = t < M ? block_scale<OP>(p.a_scale, (int64_t)t * p.kgroups + g) * ws : 0.0f;
#pragma unroll
                        for (int v = 0; v < 4; ++v) acc[j][mt][v] = __builtin_fmaf(tmp[j][mt][v], f, acc[j][mt][v]);
                    } else {
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int t = 16 * mt + 4 * g4 + v;
                            const float f = t < M ? block_scale<OP>(p.a_scale, (int64_t)t * p.kgroups + g) * ws : 0.0f;
                            acc[j][mt][v] = __builtin_fmaf(tmp[j][mt][v], f, acc[j][mt][v]);
                        }
                    }
                }
            }
        }
    };

    auto compute = [&](int step, const uint4 (&wl)[NT], const uint4 (&wh)[NT],
                       const uint4 (&al)[MT], const uint4 (&ah)[MT]) __attribute__((always_inline)) {
        if constexpr (BLOCK) {
            AccV tmp[NT][MT];
#pragma unroll
            for (int j = 0; j < NT; ++j)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const AccV zero = {0, 0, 0, 0};
                    tmp[j][mt] = SWAP ? mma_step<OP>(wl[j], wh[j], al[mt], ah[mt], zero)
                                      : mma_step<OP>(al[mt], ah[mt], wl[j], wh[j], zero);
                }
            apply_block(step, tmp);
        } else {
#pragma unroll
            for (int j = 0; j < NT; ++j)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[j][mt] = SWAP ? mma_step<OP>(wl[j], wh[j], al[mt], ah[mt], acc[j][mt])
                                      : mma_step<OP>(al[mt], ah[mt], wl[j], wh[j], acc[j][mt]);
        }
    };

    // Main loop: groups of KU whole steps; this wave takes steps
    // s0 .. s0+KU-1 with s0 = wk*KU + it*WK*KU.  Two register buffers
    // alternate: the loads of the next group are issued before the current
    // group is multiplied, so every wave keeps a group of loads in flight.
#define QBG_LOAD_GROUP(SG, WL, WH, AL, AH)                                        \
    _Pragma("unroll") for (int u = 0; u < KU; ++u) {                              \
        const int off = ((SG) + u) * 128;                                         \
        _Pragma("unroll") for (int j = 0; j < NT; ++j) {                          \
            WL[u][j] = wlive[j] ? ld16(wp[j] + off) : z4;                         \
            WH[u][j] = wlive[j] ? ld16(wp[j] + off + 64) : z4;                    \
        }                                                                         \
        _Pragma("unroll") for (int mt = 0; mt < MT; ++mt) {                       \
            AL[u][mt] = alive[mt] ? ld16(ap[mt] + off) : z4;                      \
            AH[u][mt] = alive[mt] ? ld16(ap[mt] + off + 64) : z4;                 \
        }                                                                         \
    }
#define QBG_COMPUTE_GROUP(SG, WL, WH, AL, AH)                                     \
    _Pragma("unroll") for (int u = 0; u < KU; ++u) compute((SG) + u, WL[u], WH[u], AL[u], AH[u]);

    constexpr int kStride = WK * KU;
    int s0 = wk * KU;
    if (s0 + KU <= full_steps) {
        uint4 wl0[KU][NT], wh0[KU][NT], wl1[KU][NT], wh1[KU][NT];
        uint4 al0[KU][MT], ah0[KU][MT], al1[KU][MT], ah1[KU][MT];
        QBG_LOAD_GROUP(s0, wl0, wh0, al0, ah0)
        while (true) {
            int s1 = s0 + kStride;
            const bool more1 = s1 + KU <= full_steps;
            if (more1) { QBG_LOAD_GROUP(s1, wl1, wh1, al1, ah1) }
            QBG_COMPUTE_GROUP(s0, wl0, wh0, al0, ah0)
            s0 = s1;
            if (!more1) break;
            s1 = s0 + kStride;
            const bool more0 = s1 + KU <= full_steps;
            if (more0) { QBG_LOAD_GROUP(s1, wl0, wh0, al0, ah0) }
            QBG_COMPUTE_GROUP(s0, wl1, wh1, al1, ah1)
            s0 = s1;
            if (!more0) break;
        }
    }
#undef QBG_LOAD_GROUP
#undef QBG_COMPUTE_GROUP
    // Tail: the remaining steps of this wave (at most KU), each masked per
    // 16-byte chunk against the end of the K chunk.
    if (s0 < nsteps) {
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int s = s0 + u;
            if (s >= nsteps) continue;
            const int off = s * 128;
            const bool lo_ok = off + g4 * 16 < chunk;
            const bool hi_ok = off + 64 + g4 * 16 < chunk;
            uint4 wl[NT], wh[NT], al[MT], ah[MT];
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                wl[j] = (wlive[j] && lo_ok) ? ld16(wp[j] + off) : z4;
                wh[j] = (wlive[j] && hi_ok) ? ld16(wp[j] + off + 64) : z4;
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                al[mt] = (alive[mt] && lo_ok) ? ld16(ap[mt] + off) : z4;
                ah[mt] = (alive[mt] && hi_ok) ? ld16(ap[mt] + off + 64) : z4;
            }
            compute(s, wl, wh, al, ah);
        }
    }

    // Reduce the WK partial tiles through LDS: red[wk][t][n_local].
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = SWAP ? 16 * mt + r16 : 16 * mt + 4 * g4 + v;
                const int nl = wn * 16 * NT + 16 * j + (SWAP ? 4 * g4 + v : r16);
                if (t < M) red[(wk * M + t) * TNP + nl] = acc[j][mt][v];
            }
    __syncthreads();

    const int elems = M * TN;
    const int n_tile0 = tile * TN;
    if (p.split_k == 1) {
        for (int e = threadIdx.x; e < elems; e += blockDim.x) {
            const int t = e / TN, nl = e - t * TN, n = n_tile0 + nl;
            if (n >= N) continue;
            AccS sum = red[t * TNP + nl];
#pragma unroll
            for (int w = 1; w < WK; ++w) sum += red[(w * M + t) * TNP + nl];
            store_out<OP>(p, t, n, sum);
        }
        return;
    }

    // Split-K: publish this chunk's partial, then the last arrival reduces.
    // The partials are written through to memory (system-scope stores bypass
    // the XCD-private L2s) and read back with cache-bypassing loads, so the
    // hand-off needs no L2 writeback or invalidate: each wave waits for its
    // stores to be acknowledged, the workgroup synchronizes, and one thread
    // takes a ticket from the tile's arrival counter.
    AccS* part = reinterpret_cast<AccS*>(p.partial);
    for (int e = threadIdx.x; e < elems; e += blockDim.x) {
        const int t = e / TN, nl = e - t * TN, n = n_tile0 + nl;
        if (n >= N) continue;
        AccS sum = red[t * TNP + nl];
#pragma unroll
        for (int w = 1; w < WK; ++w) sum += red[(w * M + t) * TNP + nl];
        __hip_atomic_store(&part[((int64_t)split * M + t) * N + n], sum, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_SYSTEM);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev = __hip_atomic_fetch_add(&p.counters[tile], 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == (unsigned)(p.split_k - 1));
    }
    __syncthreads();
    if (!s_last) return;
    for (int e = threadIdx.x; e < elems; e += blockDim.x) {
        const int t = e / TN, nl = e - t * TN, n = n_tile0 + nl;
        if (n >= N) continue;
        AccS sum = 0;
        for (int sp = 0; sp < p.split_k; ++sp)
            sum += __hip_atomic_load(&part[((int64_t)sp * M + t) * N + n], __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_SYSTEM);
        store_out<OP>(p, t, n, sum);
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(&p.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void fill_zero_kernel(uint32_t* p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// Compiled tile variants: {nt, wn, wk, ku}.
constexpr TileShape kTiles[] = {
    {1, 1, 4, 2},  // 0: 16 rows, 256 threads
    {1, 1, 8, 2},  // 1: 16 rows, 512 threads
    {1, 1, 4, 4},  // 2
    {1, 1, 8, 4},  // 3
    {2, 1, 4, 2},  // 4: 32 rows
    {2, 1, 8, 2},  // 5
    {2, 1, 4, 4},  // 6
    {1, 2, 4, 2},  // 7: 32 rows, 512 threads
    {2, 2, 2, 4},  // 8: 64 rows
    {2, 2, 4, 2},  // 9: 64 rows, 512 threads
    {1, 4, 1, 4},  // 10: 64 rows, no K split inside the workgroup
    {1, 1, 16, 1}, // 11: 16 rows, 1024 threads
};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

template <int OP, bool SWAP, int MT, int KID>
hipError_t launch_one(const GemmArgs& p, hipStream_t stream) {
    constexpr TileShape T = kTiles[KID];
    using AccS = typename Acc<OP>::scalar;
    const int tn = 16 * T.nt * T.wn;
    const dim3 grid((unsigned)((p.N + tn - 1) / tn), (unsigned)p.split_k);
    const dim3 block(64 * T.wn * T.wk);
    const size_t lds = (size_t)T.wk * p.M * (tn + 1) * sizeof(AccS);
    hipLaunchKernelGGL((gemm_kernel<OP, SWAP, T.nt, MT, T.wn, T.wk, T.ku>), grid, block, lds,
                       stream, p);
    return hipGetLastError();
}

template <int OP, bool SWAP, int MT, int KID = 0>
hipError_t launch_kid(int kid, const GemmArgs& p, hipStream_t stream) {
    if constexpr (KID < kNumTiles) {
        if (kid == KID) return launch_one<OP, SWAP, MT, KID>(p, stream);
        return launch_kid<OP, SWAP, MT, KID + 1>(kid, p, stream);
    } else {
        return hipErrorInvalidValue;
    }
}

template <int OP>
hipError_t launch_op(const GemmArgs& p, int kid, int swap_ab, hipStream_t stream) {
    const int mt = p.M <= 16 ? 1 : 2;
    if (swap_ab)
        return mt == 1 ? launch_kid<OP, true, 1>(kid, p, stream) : launch_kid<OP, true, 2>(kid, p, stream);
    return mt == 1 ? launch_kid<OP, false, 1>(kid, p, stream) : launch_kid<OP, false, 2>(kid, p, stream);
}

}  // namespace

int gemm_kernel_count() { return kNumTiles; }

TileShape gemm_tile(int kernel_id) {
    if (kernel_id < 0 || kernel_id >= kNumTiles) return TileShape{0, 0, 0, 0};
    return kTiles[kernel_id];
}

hipError_t launch_gemm(int op, const GemmArgs& args, int kernel_id, int swap_ab,
                       hipStream_t stream) {
    switch (op) {
        case OP_FP8: return launch_op<OP_FP8>(args, kernel_id, swap_ab, stream);
        case OP_INT8: return launch_op<OP_INT8>(args, kernel_id, swap_ab, stream);
        case OP_BLOCK_F32: return launch_op<OP_BLOCK_F32>(args, kernel_id, swap_ab, stream);
        case OP_BLOCK_UE8M0: return launch_op<OP_BLOCK_UE8M0>(args, kernel_id, swap_ab, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fill_zero(void* p, size_t n, hipStream_t stream) {
    const int64_t words = (int64_t)(n / 4);
    if (words == 0) return hipSuccess;
    const dim3 grid((unsigned)((words + 255) / 256));
    hipLaunchKernelGGL(fill_zero_kernel, grid, dim3(256), 0, stream, static_cast<uint32_t*>(p), words);
    return hipGetLastError();
}

}  // namespace qbg
