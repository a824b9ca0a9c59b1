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
//   - Block FP8 with fp32 scales: every 128-wide K step is one 16x16x128 MFMA
//     whose result is scaled by a_scale[m,g] * w_scale[n/128,g] and added to
//     the accumulator;
//   - Block FP8 with UE8M0 (power-of-two) scales: the scales are exactly the
//     E8M0 operand scales of gfx950's scaled MFMA, so each step hands the
//     matrix core the code of every operand row and the products are scaled
//     inside the MFMA, accumulating across steps like the per-channel op;
//   - Standard vs Swap-AB (A@B computed as (B^T A^T)^T): which operand fills
//     the matrix core's row slot; Swap-AB puts the weight rows there and the
//     tokens in the column slot, and the epilogue writes the transpose;
//   - Split-K: grid.y cuts K into split_k equal chunks; partial results go to
//     a workspace and the last workgroup of each tile to arrive sums them in
//     chunk order (deterministic) and applies the epilogue, so no second
//     launch is needed.  The arrival counter is reset by that workgroup.
//   - Fused per-token quantization (LDS-staged variants): the launch takes the
//     bf16 activations, a few workgroups quantize them and publish the codes,
//     and every workgroup streams its first weight stages while it waits
//     for them, so the quantizer costs no launch of its own.
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
// every wave.  In this register-streaming kernel each weight byte goes
// straight from memory to the one lane that uses it; the LDS-staged variant
// further down trades that copy for fully contiguous 1 KB loads and a deeper
// pipeline that costs no registers.
#include <type_traits>

#include "qbg_device.h"
#include "qbg_launch.h"

// The launchers of the (op, mode) families are compiled as separate objects
// (QBG_GEMM_PART = 0..7, one family each; part 0 also holds the dispatcher and
// the host helpers) so that the build compiles them in parallel; without
// QBG_GEMM_PART one object holds everything.
#ifndef QBG_GEMM_PART
#define QBG_GEMM_PART -1
#endif
#define QBG_PART(n) (QBG_GEMM_PART < 0 || QBG_GEMM_PART == (n))
#if QBG_GEMM_PART >= 0
// a part instantiates some families only, so helpers of the others go unused
#pragma clang diagnostic ignored "-Wunused-function"
#pragma clang diagnostic ignored "-Wunneeded-internal-declaration"
#endif

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

// Passes x through an empty volatile asm statement: uses of x (and the wait for
// the load that produced it) cannot move ahead of the statement.
__device__ __forceinline__ void pin16(uint4& x) {
    v4i t = {(int)x.x, (int)x.y, (int)x.z, (int)x.w};
    asm volatile("" : "+v"(t));
    x = uint4{(uint32_t)t.x, (uint32_t)t.y, (uint32_t)t.z, (uint32_t)t.w};
}

// E4M3 products run on the BF16 matrix cores.  Measured on MI355X, every FP8
// matrix-core instruction of gfx950 (16x16x128 and 32x32x64 of the f8f6f4
// family, and 16x16x32 fp8) returns the same, lossy sum: products much smaller
// than the largest one of their K block lose their low bits, so a dot product
// whose terms cancel (a token row with an outlier) can be off by several
// percent.  The BF16 instructions sum the same products as accurately as fp32
// fused multiply-adds.  Every E4M3 value is a bf16 value (4 significant bits,
// exponents 2^-9 .. 2^8), and v_cvt_scalef32_pk_bf16_fp8 converts two codes at a
// time exactly (checked on the device for all 256 codes), multiplying by a
// power-of-two scale, which is exact too: so a BF16 product of converted codes
// is the exact E4M3 product, and the UE8M0 block scales fold into the
// conversion.  At decode sizes the GEMM is bound by the weight stream, not by
// the matrix cores, so the halved matrix rate costs nothing there.
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Eight E4M3 codes (two dwords) as eight bf16 values times `scale` (a power of two).
__device__ __forceinline__ v8bf e4m3x8_bf16(uint32_t lo, uint32_t hi, float scale) {
    const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, false);
    const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, true);
    const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, false);
    const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, true);
    return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// D += X * Y^T over the 32 E4M3 codes each lane holds of its X row and Y column
// (16x16 output; four 16x16x32 BF16 products, each pairing the same code
// positions of both operands, so the 128 products are each taken once).
__device__ __forceinline__ v4f mma16_e4m3(const uint4& xl, const uint4& xh, const uint4& yl,
                                          const uint4& yh, v4f c, float sx = 1.0f,
                                          float sy = 1.0f) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_bf16(xl.x, xl.y, sx), e4m3x8_bf16(yl.x, yl.y, sy), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_bf16(xl.z, xl.w, sx), e4m3x8_bf16(yl.z, yl.w, sy), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_bf16(xh.x, xh.y, sx), e4m3x8_bf16(yh.x, yh.y, sy), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_bf16(xh.z, xh.w, sx), e4m3x8_bf16(yh.z, yh.w, sy), c, 0, 0, 0);
    return c;
}

// The same for a 32x32 output tile: 32 codes per lane (x, y) over 64 K
// positions, four 32x32x16 BF16 products.
__device__ __forceinline__ v16f mma32_e4m3(const v8i& x, const v8i& y, v16f c, float sx = 1.0f,
                                           float sy = 1.0f) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(e4m3x8_bf16(x[2 * q], x[2 * q + 1], sx),
                                                    e4m3x8_bf16(y[2 * q], y[2 * q + 1], sy), c, 0, 0, 0);
    return c;
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
        return mma16_e4m3(xl, xh, yl, yh, c);
    }
}

// One 128-wide K step of E4M3 x E4M3 with UE8M0 scales: every product
// X[r,k] * Y[c,k] is multiplied by 2^(sx - 127) * 2^(sy - 127), sx being the
// code of this lane's X row and sy that of its Y column; the scales are applied
// exactly while the codes are converted.
__device__ __forceinline__ v4f mma_step_e8m0(const uint4& xl, const uint4& xh, const uint4& yl,
                                             const uint4& yh, v4f c, int sx, int sy) {
    return mma16_e4m3(xl, xh, yl, yh, c, ue8m0_value((uint32_t)sx), ue8m0_value((uint32_t)sy));
}

template <int OP>
__device__ __forceinline__ float block_scale(const void* s, int64_t idx) {
    if constexpr (OP == OP_BLOCK_UE8M0)
        return ue8m0_value(reinterpret_cast<const uint8_t*>(s)[idx]);
    else
        return reinterpret_cast<const float*>(s)[idx];
}

// Writes one output element.  `factor` is a_scale[t] * w_scale[n] for the
// per-channel ops (prefetched), unused otherwise.
template <int OP>
__device__ __forceinline__ void store_out(const GemmArgs& p, int t, int n,
                                          typename Acc<OP>::scalar v, float factor) {
    const int64_t o = (int64_t)t * p.N + n;
    if constexpr (OP == OP_INT8) {
        if (p.raw_i32) {
            reinterpret_cast<int*>(p.out)[o] = v;
            return;
        }
    }
    float f = (float)v;
    if constexpr (OP == OP_FP8 || OP == OP_INT8) f = f * factor;
    reinterpret_cast<uint16_t*>(p.out)[o] = (uint16_t)f32_to_bf16(f);
}

// The per-channel scale products a_scale[t] * w_scale[n] of the output
// elements this thread writes at the end of the tile (elements
// e = threadIdx.x + i * NTHR of the M x TN tile, M <= TMAX).  The two factors
// are loaded when the kernel starts and multiplied only at the end: a product
// taken at once would make the kernel wait for the loads (a full memory round
// trip) before it issues its first weight load.
template <int OP, int TN, int NTHR, int TMAX = kMaxTokensPerLaunch, int RT = 0>
struct EpiScales {
    // RT > 0: the workgroup owns weight rows [RT * tile, RT * tile + RT) only
    // (RT < TN); element columns RT .. TN-1 hold no output.
    static constexpr int kRows = RT > 0 ? RT : TN;
    static constexpr bool kUsed = (OP == OP_FP8 || OP == OP_INT8);
    static constexpr int kPer = (TMAX * TN + NTHR - 1) / NTHR;
    float a[kUsed ? kPer : 1];  // a_scale[t]
    float w[kUsed ? kPer : 1];  // w_scale[n]

    __device__ __forceinline__ void prefetch(const GemmArgs& p) {
        if constexpr (kUsed) {
            const bool raw = OP == OP_INT8 && p.raw_i32;
            const float* as = reinterpret_cast<const float*>(p.a_scale);
            const float* ws = reinterpret_cast<const float*>(p.w_scale);
            const int elems = p.M * TN, n0 = blockIdx.x * kRows;
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int e = threadIdx.x + i * NTHR;
                const int t = e / TN, nl = e - t * TN, n = n0 + nl;
                a[i] = 0.0f;
                w[i] = 0.0f;
                if (!raw && e < elems && nl < kRows && n < p.N) {
                    a[i] = as[t];
                    w[i] = ws[n];
                }
            }
        }
    }
    // Fused launch: w_scale first (the activation scales do not exist yet) ...
    __device__ __forceinline__ void prefetch_w(const GemmArgs& p) {
        if constexpr (kUsed) {
            const float* ws = reinterpret_cast<const float*>(p.w_scale);
            const int elems = p.M * TN, n0 = blockIdx.x * kRows;
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int e = threadIdx.x + i * NTHR;
                const int t = e / TN, nl = e - t * TN, n = n0 + nl;
                a[i] = 0.0f;
                w[i] = (e < elems && nl < kRows && n < p.N) ? ws[n] : 0.0f;
            }
        }
    }
    // ... then a_scale once it is published ...
    __device__ __forceinline__ void apply_a(const GemmArgs& p) {
        if constexpr (kUsed) {
            const float* as = reinterpret_cast<const float*>(p.a_scale);
            const int elems = p.M * TN;
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int e = threadIdx.x + i * NTHR;
                if (e < elems) a[i] = as[e / TN];
            }
        }
    }
    // ... or from the workgroup's own scales in LDS (LOCAL fused mode).
    __device__ __forceinline__ void apply_a_lds(const float* sc, int M) {
        if constexpr (kUsed) {
            const int elems = M * TN;
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int e = threadIdx.x + i * NTHR;
                if (e < elems) a[i] = sc[e / TN];
            }
        }
    }
    __device__ __forceinline__ float get(int i) const {
        if constexpr (kUsed) return a[i] * w[i];
        return 0.0f;
    }
};

// Fused launch: per-token quantization of activation row r by the whole
// workgroup, the standalone quantizer's arithmetic (amax, token_scale,
// quant8), stored with write-through (system-scope) stores so that
// workgroups on every XCD read the codes from memory, not from a stale cache
// line.  NTHR == blockDim.x; `red` holds NTHR / 64 floats of LDS.
template <int QT, int NTHR>
__device__ __forceinline__ void publish_row(const GemmArgs& p, int r, float* red) {
    constexpr int CH = 8;  // 16-byte chunks a thread keeps in registers
    const int nchunks = p.K >> 3;
    const uint4* row = reinterpret_cast<const uint4*>(p.x + (int64_t)r * p.K);
    uint64_t* qrow = reinterpret_cast<uint64_t*>(const_cast<uint8_t*>(p.a) + (int64_t)r * p.K);
    float* scale = reinterpret_cast<float*>(const_cast<void*>(p.a_scale));
    float v[8];
    float amax = 0.0f;
    if (nchunks <= CH * NTHR) {
        uint4 c[CH];
        load_row_chunks<CH>(row, nchunks, threadIdx.x, NTHR, c);  // a repeated chunk: same max
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            unpack8(c[i], v);
#pragma unroll
            for (int j = 0; j < 8; ++j) amax = amax_fold(amax, v[j]);
        }
        const float s = token_scale<QT>(block_max(amax, red));
        if (threadIdx.x == 0)
            __hip_atomic_store(&scale[r], s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int idx = threadIdx.x + i * NTHR;
            if (idx >= nchunks) continue;
            unpack8(c[i], v);
            const uint2 q = quant8<QT>(v, s);
            __hip_atomic_store(&qrow[idx], (uint64_t)q.x | ((uint64_t)q.y << 32), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_SYSTEM);
        }
    } else {  // long rows: amax pass, then a quantize pass that re-reads the row from cache
        for (int idx = threadIdx.x; idx < nchunks; idx += NTHR) {
            unpack8(row[idx], v);
#pragma unroll
            for (int j = 0; j < 8; ++j) amax = amax_fold(amax, v[j]);
        }
        const float s = token_scale<QT>(block_max(amax, red));
        if (threadIdx.x == 0)
            __hip_atomic_store(&scale[r], s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        for (int idx = threadIdx.x; idx < nchunks; idx += NTHR) {
            unpack8(row[idx], v);
            const uint2 q = quant8<QT>(v, s);
            __hip_atomic_store(&qrow[idx], (uint64_t)q.x | ((uint64_t)q.y << 32), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_SYSTEM);
        }
    }
}

// End of a tile, shared by both kernel kinds: the WK partial tiles of each
// wave are reduced through LDS in a fixed order, then either the epilogue
// writes the outputs (split_k == 1) or the Split-K hand-off runs.
// `red` holds at least WK * M * (TN + 1) accumulators; the caller has finished
// every other use of that LDS.  A wave's accumulator token slots start at
// token t0 (waves side by side along M hold different tokens).
template <int OP, bool SWAP, int NT, int MT, int WN, int WK, int WM = 1,
          int TMAX = kMaxTokensPerLaunch, int RT = 0>
__device__ __forceinline__ void finish_tile(const GemmArgs& p, typename Acc<OP>::scalar* red,
                                            typename Acc<OP>::vec (&acc)[NT][MT], int wn, int wk,
                                            int* s_last_ptr,
                                            const EpiScales<OP, 16 * NT * WN, 64 * WN * WK * WM,
                                                            TMAX, RT>& es,
                                            int t0 = 0) {
    using AccS = typename Acc<OP>::scalar;
    constexpr int TN = 16 * NT * WN;
    // weight rows this workgroup owns: [R * tile, R * tile + R); local columns
    // R .. TN-1 of the accumulator tile hold duplicate rows and are dropped
    constexpr int R = RT > 0 ? RT : TN;
    constexpr int NTHR = 64 * WN * WK * WM;
    constexpr int EPT = EpiScales<OP, TN, NTHR, TMAX>::kPer;
    constexpr int TNP = TN + 1;
    int& s_last = *s_last_ptr;
    const int lane = threadIdx.x & 63;
    const int r16 = lane & 15, g4 = lane >> 4;
    const int tile = blockIdx.x, split = blockIdx.y;
    const int M = p.M, N = p.N;
    // Reduce the WK partial tiles through LDS: red[wk][t][n_local].
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = t0 + (SWAP ? 16 * mt + r16 : 16 * mt + 4 * g4 + v);
                const int nl = wn * 16 * NT + 16 * j + (SWAP ? 4 * g4 + v : r16);
                if (t < M) red[(wk * M + t) * TNP + nl] = acc[j][mt][v];
            }
    __syncthreads();

    const int elems = M * TN;
    const int n_tile0 = tile * R;
    if (p.split_k == 1) {
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int e = threadIdx.x + i * NTHR;
            const int t = e / TN, nl = e - t * TN, n = n_tile0 + nl;
            if (e >= elems || nl >= R || n >= N) continue;
            AccS sum = red[t * TNP + nl];
#pragma unroll
            for (int w = 1; w < WK; ++w) sum += red[(w * M + t) * TNP + nl];
            store_out<OP>(p, t, n, sum, es.get(i));
        }
        return;
    }

    // Split-K: publish this chunk's partial, then the last arrival reduces.
    // The partials are written through to memory (system-scope stores bypass
    // the XCD-private L2s) and read back with cache-bypassing loads, so the
    // hand-off needs no L2 writeback or invalidate: each wave waits for its
    // stores to be acknowledged, the workgroup synchronizes, and one thread
    // takes a ticket from the tile's arrival counter.
    //
    // Ordering this relies on (the hardware's, stated because the accesses are
    // relaxed atomics rather than a release/acquire pair, whose agent-scope
    // fences would write back and invalidate whole L2s):
    //  1. a system-scope store is performed at memory, past every cache, when
    //     the wave's vector-memory counter has drained (s_waitcnt 0), and the
    //     counter never drains before the store is acknowledged;
    //  2. s_waitcnt and the workgroup barrier are side-effecting for the
    //     compiler, so no memory access moves across them; the ticket's
    //     fetch_add is issued after every wave of the workgroup passed them;
    //  3. the ticket is an agent-scope read-modify-write performed at memory,
    //     in one order for all workgroups; a workgroup that draws the last
    //     ticket issues its loads only after the fetch_add has returned;
    //  4. those loads are system-scope (they bypass L1 and L2), so they read
    //     memory, which already holds every other chunk's partial by 1-3.
    AccS* part = reinterpret_cast<AccS*>(p.partial);
    for (int e = threadIdx.x; e < elems; e += blockDim.x) {
        const int t = e / TN, nl = e - t * TN, n = n_tile0 + nl;
        if (nl >= R || n >= N) continue;
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
    // Every partial this thread sums is loaded before the first is used: one
    // memory round trip per batch of SB chunks instead of one per chunk.  The
    // sums still run in chunk order, so the bits do not depend on which
    // workgroup arrives last.
    constexpr int SB = EPT <= 4 ? 8 : EPT <= 8 ? 4 : EPT <= 16 ? 2 : 1;  // chunks per batch
    AccS sum[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) sum[i] = 0;
    for (int sp0 = 0; sp0 < p.split_k; sp0 += SB) {
        AccS v[EPT][SB];
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int e = threadIdx.x + i * NTHR;
            const int t = e / TN, nl = e - t * TN, n = n_tile0 + nl;
            const bool live = e < elems && nl < R && n < N;
#pragma unroll
            for (int b = 0; b < SB; ++b)
                v[i][b] = (live && sp0 + b < p.split_k)
                              ? __hip_atomic_load(&part[((int64_t)(sp0 + b) * M + t) * N + n],
                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM)
                              : AccS(0);
        }
#pragma unroll
        for (int i = 0; i < EPT; ++i)
#pragma unroll
            for (int b = 0; b < SB; ++b) sum[i] += v[i][b];
    }
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = threadIdx.x + i * NTHR;
        const int t = e / TN, nl = e - t * TN, n = n_tile0 + nl;
        if (e >= elems || nl >= R || n >= N) continue;
        store_out<OP>(p, t, n, sum[i], es.get(i));
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(&p.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// LDS-staged variant (all four ops).
//
// The workgroup's weight rows [n0, n0+TN) and the AR activation rows stream
// through an NS-deep ring of LDS stages, each holding RB = 128*SK bytes of K
// for every row.  Stages are filled with direct global->LDS loads
// (global_load_lds_dwordx4): one instruction moves 1 KB of consecutive bytes
// (1024/RB whole row segments), so global reads are fully contiguous and cost
// no registers; the ring keeps NS-1 stages in flight per workgroup.  Within
// a row, 16-byte chunk c is stored at slot c ^ (row % 16), so the MFMA-layout
// reads (16 rows x the same chunk) hit 16 different bank groups.  The
// activation tile is loaded once per stage and shared by all waves.  Rows
// past M (activations) or N (weights) load a valid duplicate row whose
// results are never stored.
//
// Block ops: every workgroup's TN rows lie in one 128-row weight block, so
// the scales a step needs are one weight-block scale and one scale per token.
// They are staged once, for the whole K chunk, behind the stage ring: word
// g * AR + t holds a_scale[t,g] * w_scale[block,g] (fp32 scales) or the UE8M0
// codes of token t (bits 0-7) and of the block (bits 8-15), and each step
// reads its words together with its operands.
//
// Synchronization: each wave waits with s_waitcnt vmcnt for its own loads of
// the stage it is about to read, then s_barrier makes every wave's loads of
// that stage visible and guarantees the slot being refilled is no longer read.
// The LDS reads are issued in one asm block that also waits for them, so the
// compiler never sees an LDS read that could alias an in-flight load (which
// would make it drain all loads).
// ---------------------------------------------------------------------------
// CPOL is the load's cache policy: 0 for rows other workgroups read again
// (activations), kNonTemporal for the weight stream, which every workgroup
// reads exactly once.  Measured on MI355X with a plain streaming kernel, the
// non-temporal hint raises global->LDS streaming from HBM from 5.8 to 6.4 TB/s
// on 100 MB and from 3.9 to 4.2 TB/s on 16 MB per launch.
constexpr int kNonTemporal = 2;  // the nt bit of the gfx950 cache-policy field
template <int CPOL = 0>
__device__ __forceinline__ void lds_dma16(const uint8_t* g, char* lds) {
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(g),
                                     (__attribute__((address_space(3))) void*)(lds), 16, 0, CPOL);
}

__device__ __forceinline__ uint4 and4(const uint4& v, uint32_t m) {
    return uint4{v.x & m, v.y & m, v.z & m, v.w & m};
}

__device__ __forceinline__ uint32_t lds_addr(const char* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(p);
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until at most n vector-memory loads of this wave are outstanding.
template <int LPW, int NS>
__device__ __forceinline__ void wait_stages(int stages_after) {
    // n = stages_after * LPW, stages_after in [0, NS-2]; immediates must be constants
#define QBG_VMW(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))
    static_assert(NS <= 8 && LPW <= 63, "vmcnt range");
    // a count the 6-bit vmcnt field cannot hold waits for more loads: still correct
    constexpr int kMaxAfter = 63 / LPW;
    // (a count outside [0, NS-2] cannot occur; it would wait for every load)
    switch (stages_after < kMaxAfter ? stages_after : kMaxAfter) {
        case 1: if constexpr (NS > 2 && kMaxAfter >= 1) { QBG_VMW(1 * LPW); } else { QBG_VMW(0); } break;
        case 2: if constexpr (NS > 3 && kMaxAfter >= 2) { QBG_VMW(2 * LPW); } else { QBG_VMW(0); } break;
        case 3: if constexpr (NS > 4 && kMaxAfter >= 3) { QBG_VMW(3 * LPW); } else { QBG_VMW(0); } break;
        case 4: if constexpr (NS > 5 && kMaxAfter >= 4) { QBG_VMW(4 * LPW); } else { QBG_VMW(0); } break;
        case 5: if constexpr (NS > 6 && kMaxAfter >= 5) { QBG_VMW(5 * LPW); } else { QBG_VMW(0); } break;
        case 6: if constexpr (NS > 7 && kMaxAfter >= 6) { QBG_VMW(6 * LPW); } else { QBG_VMW(0); } break;
        default: QBG_VMW(0); break;
    }
#undef QBG_VMW
}

__device__ __forceinline__ void lds_read4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                          uint4& x0, uint4& x1, uint4& x2, uint4& x3) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3)
        : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
        : "memory");
}

__device__ __forceinline__ void lds_read2(uint32_t a0, uint32_t a1, uint4& x0, uint4& x1) {
    asm volatile(
        "ds_read_b128 %0, %2\n\t"
        "ds_read_b128 %1, %3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x0), "=&v"(x1)
        : "v"(a0), "v"(a1)
        : "memory");
}

// Four operand chunks plus one 32-bit scale word.
__device__ __forceinline__ void lds_read4w(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                           uint32_t as, uint4& x0, uint4& x1, uint4& x2,
                                           uint4& x3, uint32_t& w) {
    asm volatile(
        "ds_read_b128 %0, %5\n\t"
        "ds_read_b128 %1, %6\n\t"
        "ds_read_b128 %2, %7\n\t"
        "ds_read_b128 %3, %8\n\t"
        "ds_read_b32 %4, %9\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3), "=&v"(w)
        : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "v"(as)
        : "memory");
}

// Four operand chunks plus four consecutive 32-bit scale words.
__device__ __forceinline__ void lds_read5(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                          uint32_t a4, uint4& x0, uint4& x1, uint4& x2,
                                          uint4& x3, uint4& x4) {
    asm volatile(
        "ds_read_b128 %0, %5\n\t"
        "ds_read_b128 %1, %6\n\t"
        "ds_read_b128 %2, %7\n\t"
        "ds_read_b128 %3, %8\n\t"
        "ds_read_b128 %4, %9\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3), "=&v"(x4)
        : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "v"(a4)
        : "memory");
}

__device__ __forceinline__ void lds_read1(uint32_t a0, uint4& x0) {
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(x0) : "v"(a0) : "memory");
}

__device__ __forceinline__ void lds_read1w(uint32_t a0, uint32_t& w) {
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(w) : "v"(a0) : "memory");
}

// Six 16-byte LDS reads and one wait.
__device__ __forceinline__ void lds_read6(const uint32_t (&a)[6], uint4 (&x)[6]) {
    asm volatile(
        "ds_read_b128 %0, %6\n\t"
        "ds_read_b128 %1, %7\n\t"
        "ds_read_b128 %2, %8\n\t"
        "ds_read_b128 %3, %9\n\t"
        "ds_read_b128 %4, %10\n\t"
        "ds_read_b128 %5, %11\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5])
        : "memory");
}

// Eight 16-byte LDS reads and one wait.
__device__ __forceinline__ void lds_read8(const uint32_t (&a)[8], uint4 (&x)[8]) {
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %9\n\t"
        "ds_read_b128 %2, %10\n\t"
        "ds_read_b128 %3, %11\n\t"
        "ds_read_b128 %4, %12\n\t"
        "ds_read_b128 %5, %13\n\t"
        "ds_read_b128 %6, %14\n\t"
        "ds_read_b128 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
          "=&v"(x[6]), "=&v"(x[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
        : "memory");
}

// NP (lo, hi) chunk pairs of one operand, read in batches of at most eight
// reads per wait: lo[i] at a_lo[i], hi[i] at a_hi[i].
template <int NP>
__device__ __forceinline__ void lds_read_pairs(const uint32_t (&a_lo)[NP], const uint32_t (&a_hi)[NP],
                                               uint4 (&lo)[NP], uint4 (&hi)[NP]) {
    if constexpr (NP == 1) {
        lds_read2(a_lo[0], a_hi[0], lo[0], hi[0]);
    } else if constexpr (NP == 2) {
        lds_read4(a_lo[0], a_hi[0], a_lo[1], a_hi[1], lo[0], hi[0], lo[1], hi[1]);
    } else if constexpr (NP == 3) {
        lds_read4(a_lo[0], a_hi[0], a_lo[1], a_hi[1], lo[0], hi[0], lo[1], hi[1]);
        lds_read2(a_lo[2], a_hi[2], lo[2], hi[2]);
    } else {
        static_assert(NP % 4 == 0, "pairs in batches of four");
#pragma unroll
        for (int b = 0; b < NP; b += 4) {
            const uint32_t a[8] = {a_lo[b], a_hi[b], a_lo[b + 1], a_hi[b + 1],
                                   a_lo[b + 2], a_hi[b + 2], a_lo[b + 3], a_hi[b + 3]};
            uint4 x[8];
            lds_read8(a, x);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                lo[b + i] = x[2 * i];
                hi[b + i] = x[2 * i + 1];
            }
        }
    }
}

__device__ __forceinline__ uint32_t u4_at(const uint4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// LOCAL fused mode: the workgroup quantizes the M activation rows itself,
// from a copy of the rows in LDS.
//
// The caller loads the M bf16 rows (2MK contiguous bytes) into LDS at `xs` by
// LDS DMA before it issues its first weight stages, waits for its own row
// loads only (the weight stages stay in flight) and synchronizes the
// workgroup.  Every LDS access below is an inline-asm block that waits for
// itself: the compiler then never sees an LDS access next to the DMA loads in
// flight, which would make it wait for all of them.
//
// Pass 1 reduces each row's amax: item i of a thread is 16-byte chunk
// (i % cpr) * NTHR + threadIdx.x of row i / cpr (cpr items per row; chunks past
// the row end read the row's last chunk again, which leaves the max as it
// is); thread r then forms row r's scale.  Pass 2 writes the codes of the
// workgroup's K range [k_begin, k_begin + chunk) to LDS: byte k of that range
// of row r at act + r * RS + (((k / 16) ^ (r % 16)) * 16) + k % 16, the
// swizzle of the stage ring.  The arithmetic is the standalone quantizer's
// (amax, token_scale, quant8), so codes and scales are the same bytes.  `red`
// holds M * NW floats, `sc` M; all four regions are LDS byte addresses.
__device__ __forceinline__ void lds_write_b32(uint32_t a, uint32_t v) {
    asm volatile("ds_write_b32 %0, %1" : : "v"(a), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_write_b64(uint32_t a, uint64_t v) {
    asm volatile("ds_write_b64 %0, %1" : : "v"(a), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Eight 16-byte reads and eight 32-bit reads, one wait.
__device__ __forceinline__ void lds_read8s(const uint32_t (&a)[8], const uint32_t (&as)[8],
                                           uint4 (&x)[8], uint32_t (&w)[8]) {
    asm volatile(
        "ds_read_b128 %0, %16\n\t"
        "ds_read_b128 %1, %17\n\t"
        "ds_read_b128 %2, %18\n\t"
        "ds_read_b128 %3, %19\n\t"
        "ds_read_b128 %4, %20\n\t"
        "ds_read_b128 %5, %21\n\t"
        "ds_read_b128 %6, %22\n\t"
        "ds_read_b128 %7, %23\n\t"
        "ds_read_b32 %8, %24\n\t"
        "ds_read_b32 %9, %25\n\t"
        "ds_read_b32 %10, %26\n\t"
        "ds_read_b32 %11, %27\n\t"
        "ds_read_b32 %12, %28\n\t"
        "ds_read_b32 %13, %29\n\t"
        "ds_read_b32 %14, %30\n\t"
        "ds_read_b32 %15, %31\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
          "=&v"(x[6]), "=&v"(x[7]), "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3]),
          "=&v"(w[4]), "=&v"(w[5]), "=&v"(w[6]), "=&v"(w[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]),
          "v"(as[0]), "v"(as[1]), "v"(as[2]), "v"(as[3]), "v"(as[4]), "v"(as[5]), "v"(as[6]),
          "v"(as[7])
        : "memory");
}

template <int QT, int NTHR>
__device__ __forceinline__ void local_quantize(const GemmArgs& p, int64_t k_begin, int chunk,
                                               uint32_t xs, uint32_t act, int RS, uint32_t red,
                                               uint32_t sc) {
    constexpr int NW = NTHR / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int M = p.M;
    const int K = p.K;
    const int rc = K >> 3;                       // 16-byte chunks of a bf16 row
    const int cpr = (rc + NTHR - 1) / NTHR;      // items per row and thread
    const int ni = M * cpr;
    // pass 1: row amax
    {
        float run = 0.0f;
        int r = 0, j = 0;  // row and item of the next item to reduce (uniform)
        for (int i0 = 0; i0 < ni; i0 += 8) {
            uint32_t a[8];
            int rr = r, jj = j;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int idx = min(jj * NTHR + (int)threadIdx.x, rc - 1);
                a[u] = xs + (uint32_t)(min(rr, M - 1) * 2 * K + idx * 16);
                if (++jj == cpr) { jj = 0; ++rr; }
            }
            uint4 v[8];
            lds_read8(a, v);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (i0 + u < ni) {
                    float f[8];
                    unpack8(v[u], f);
#pragma unroll
                    for (int e = 0; e < 8; ++e) run = amax_fold(run, f[e]);
                    if (++j == cpr) {
                        const float m = wave_max(run);
                        if (lane == 0) lds_write_b32(red + 4u * (uint32_t)(r * NW + wave), __float_as_uint(m));
                        run = 0.0f;
                        j = 0;
                        ++r;
                    }
                }
            }
        }
    }
    lds_wait();
    __builtin_amdgcn_s_barrier();
    if ((int)threadIdx.x < M) {
        float a = 0.0f;
        for (int w = 0; w < NW; ++w) {
            uint32_t v;
            lds_read1w(red + 4u * (uint32_t)(threadIdx.x * NW + w), v);
            a = max_nan(a, __uint_as_float(v));
        }
        lds_write_b32(sc + 4u * threadIdx.x, __float_as_uint(token_scale<QT>(a)));
        lds_wait();
    }
    __builtin_amdgcn_s_barrier();
    // pass 2: codes of this workgroup's K range
    const int kb = (int)(k_begin >> 3), cq = chunk >> 3;  // first chunk of the range, chunks
    const int cpq = (cq + NTHR - 1) / NTHR;
    const int nq = M * cpq;
    int r = 0, j = 0;
    for (int i0 = 0; i0 < nq; i0 += 8) {
        uint32_t a[8], as[8];
        int rr = r, jj = j;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int l = min(jj * NTHR + (int)threadIdx.x, cq - 1);
            const int row = min(rr, M - 1);
            a[u] = xs + (uint32_t)(row * 2 * K + (kb + l) * 16);
            as[u] = sc + 4u * (uint32_t)row;
            if (++jj == cpq) { jj = 0; ++rr; }
        }
        uint4 v[8];
        uint32_t sv[8];
        lds_read8s(a, as, v, sv);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (i0 + u < nq) {
                const int l = j * NTHR + (int)threadIdx.x;  // 8-byte code group within the range
                if (l < cq) {
                    float f[8];
                    unpack8(v[u], f);
                    const uint2 q = quant8<QT>(f, __uint_as_float(sv[u]));
                    lds_write_b64(act + (uint32_t)(r * RS + (((l >> 1) ^ (r & 15)) << 4) + ((l & 1) << 3)),
                                  (uint64_t)q.x | ((uint64_t)q.y << 32));
                }
                if (++j == cpq) { j = 0; ++r; }
            }
        }
    }
    lds_wait();
}

// Row quantization for the register kernel's LOCAL mode (at most 16 rows):
// the same result as local_quantize (the standalone quantizer's amax,
// token_scale and quant8 on the same bf16 values, so the same bytes), in
// fewer steps.  Every thread reads its 16-byte chunks of all M rows in one
// pass and folds them, each wave writes one partial per row, and after the one
// barrier every wave reduces a row's partials itself (the maximum does not
// depend on the order), so no thread waits on another's sum.  The codes of the
// K range [k_begin, k_begin + chunk) go to act with the stage ring's swizzle;
// the scales to sc (thread 0).  All four are LDS byte addresses; the caller synchronizes the
// workgroup before the codes are read.
__device__ __forceinline__ uint4 lds_read_b128w(uint32_t a) {
    uint4 x;
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(x) : "v"(a) : "memory");
    return x;
}
template <int QT, int NTHR>
__device__ __forceinline__ void local_quantize_rows(int M, int K, int64_t k_begin, int chunk,
                                                    uint32_t xs, uint32_t act, int RS,
                                                    uint32_t red, uint32_t sc) {
    constexpr int NW = NTHR / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rc = K >> 3;  // 16-byte chunks (8 bf16 values) of a row
    // Rows go four at a time while four remain (four reads, one wait), then one
    // at a time.
    int r0 = 0;
    for (; r0 + 4 <= M; r0 += 4) {
        uint32_t rb[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) rb[u] = xs + (uint32_t)((r0 + u) * 2 * K);
        float run[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int c = threadIdx.x; c < rc; c += NTHR) {
            uint4 x[4];
            lds_read4(rb[0] + c * 16, rb[1] + c * 16, rb[2] + c * 16, rb[3] + c * 16, x[0], x[1],
                      x[2], x[3]);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float f[8];
                unpack8(x[u], f);
#pragma unroll
                for (int e = 0; e < 8; ++e) run[u] = amax_fold(run[u], f[e]);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float m = wave_max(run[u]);
            if (lane == 0) lds_write_b32(red + 4u * (uint32_t)((r0 + u) * NW + wave), __float_as_uint(m));
        }
    }
    for (int r = r0; r < M; ++r) {
        float run = 0.0f;
        for (int c = threadIdx.x; c < rc; c += NTHR) {
            float f[8];
            unpack8(lds_read_b128w(xs + (uint32_t)(r * 2 * K + c * 16)), f);
#pragma unroll
            for (int e = 0; e < 8; ++e) run = amax_fold(run, f[e]);
        }
        const float m = wave_max(run);
        if (lane == 0) lds_write_b32(red + 4u * (uint32_t)(r * NW + wave), __float_as_uint(m));
    }
    lds_wait();
    __builtin_amdgcn_s_barrier();
    const int kb = (int)(k_begin >> 3), cq = chunk >> 3;  // first 8-code group of the range, groups
    auto row_scale = [&](int r) {
        uint32_t pv = 0;  // +0.0f: the partials are non-negative or NaN
        if (lane < NW) lds_read1w(red + 4u * (uint32_t)(r * NW + lane), pv);
        const float s = token_scale<QT>(wave_max(__uint_as_float(pv)));
        if (threadIdx.x == 0) lds_write_b32(sc + 4u * (uint32_t)r, __float_as_uint(s));
        return s;
    };
    auto put = [&](int r, int l, const uint4& x, float s) {
        float f[8];  // code group l: the 8 bf16 values at byte (kb + l) * 16 of the row
        unpack8(x, f);
        const uint2 q = quant8<QT>(f, s);
        lds_write_b64(act + (uint32_t)(r * RS + (((l >> 1) ^ (r & 15)) << 4) + ((l & 1) << 3)),
                      (uint64_t)q.x | ((uint64_t)q.y << 32));
    };
    r0 = 0;
    for (; r0 + 4 <= M; r0 += 4) {
        uint32_t rb[4];
        float s[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            rb[u] = xs + (uint32_t)((r0 + u) * 2 * K + kb * 16);
            s[u] = row_scale(r0 + u);
        }
        for (int l = threadIdx.x; l < cq; l += NTHR) {
            uint4 x[4];
            lds_read4(rb[0] + l * 16, rb[1] + l * 16, rb[2] + l * 16, rb[3] + l * 16, x[0], x[1],
                      x[2], x[3]);
#pragma unroll
            for (int u = 0; u < 4; ++u) put(r0 + u, l, x[u], s[u]);
        }
    }
    for (int r = r0; r < M; ++r) {
        const float s = row_scale(r);
        for (int l = threadIdx.x; l < cq; l += NTHR)
            put(r, l, lds_read_b128w(xs + (uint32_t)(r * 2 * K + (kb + l) * 16)), s);
    }
    lds_wait();
}

// ---------------------------------------------------------------------------
// Register-streaming kernel (all four ops).
// ---------------------------------------------------------------------------
// RT > 0: the workgroup owns RT < TN weight rows (per-channel ops), so that a
// row count that is no multiple of 16 * NT * WN still splits evenly over the
// CUs (6144 rows = 256 workgroups of 24).
//
// LOC: the fused one-launch mode (LOCAL) on this kernel, per-channel ops, at
// most 16 tokens.  Each wave owns exactly two load groups of the K chunk
// (checked on the host), so every weight load of the workgroup is issued at
// once, before anything else waits; the workgroup meanwhile loads the M bf16
// rows into LDS, quantizes them there (the standalone quantizer's arithmetic,
// local_quantize) and then reads its activation operands from the codes in
// LDS.  The quantization runs while the weights are in flight.
template <int OP, bool SWAP, int NT, int MT, int WN, int WK, int KU, int RT = 0, bool LOC = false>
__global__ __launch_bounds__(64 * WN * WK) void gemm_kernel(const GemmArgs p) {
    using AccV = typename Acc<OP>::vec;
    using AccS = typename Acc<OP>::scalar;
    constexpr bool BLOCK = (OP == OP_BLOCK_F32 || OP == OP_BLOCK_UE8M0);
    constexpr int TN = 16 * NT * WN;       // weight rows the accumulators hold
    constexpr int R = RT > 0 ? RT : TN;  // weight rows the workgroup owns
    static_assert(RT == 0 || (!BLOCK && RT >= 8 && RT < TN && RT % 4 == 0), "owned rows: per-channel ops");

    extern __shared__ char smem_raw[];
    AccS* red = reinterpret_cast<AccS*>(smem_raw);  // [WK][M][TNP]
    __shared__ int s_last;

    // the wave index is the same in every lane: readfirstlane tells the compiler,
    // so values derived from it live in scalar registers and branch uniformly
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wn = wave % WN, wk = wave / WN;
    const int r16 = lane & 15, g4 = lane >> 4;
    const int tile = blockIdx.x, split = blockIdx.y;
    const int M = p.M, N = p.N;
    const int64_t K = p.K;
    const int n_wave = tile * R + wn * 16 * NT;
    const int64_t k_begin = (int64_t)split * p.k_chunk;
    const int chunk = p.k_chunk;
    const int nsteps = (chunk + 127) / 128;
    const int full_steps = chunk / 128;

    static_assert(!LOC || ((OP == OP_FP8 || OP == OP_INT8) && MT == 1), "LOCAL: per-channel ops, 16 tokens");
    EpiScales<OP, TN, 64 * WN * WK, kMaxTokensPerLaunch, RT> es;
    if constexpr (LOC) es.prefetch_w(p);  // the activation scales do not exist yet
    else es.prefetch(p);

    AccV acc[NT][MT];
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[j][mt] = AccV{0, 0, 0, 0};

    // A lane's operand bytes of a step sit at a uniform base (the tensor, the
    // chunk start and the step's offset) plus a fixed 32-bit lane offset (its
    // row times K plus its 16-byte slot), so a step's addresses cost scalar
    // arithmetic only: no vector temporaries that could land on registers a
    // load in flight still owns.  Dead token rows (past M) read row 0.  The
    // workgroup owns weight rows [R * tile, R * tile + R) clipped at N (at least
    // one: the grid has ceil(N / R) workgroups); a lane whose row of sub-tile j
    // is not owned reads an owned row of the same sub-tile (the same segments as
    // another lane of that load: no extra traffic), or row 0 when the sub-tile
    // owns none.  Products of rows not owned are never stored.
    const int owned = min(R, N - tile * R);
    uint32_t wo[NT];
    bool wlive[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int live_rows = min(max(owned - (wn * 16 * NT + 16 * j), 0), 16);  // uniform
        wlive[j] = live_rows > 0;
        const int r = r16 < live_rows ? r16 : (live_rows > 0 ? r16 % live_rows : 0);
        wo[j] = (uint32_t)((wlive[j] ? n_wave + 16 * j + r : 0) * K) + (uint32_t)(g4 * 16);
    }
    uint32_t ao[MT];
    bool alive[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int t = 16 * mt + r16;
        alive[mt] = t < M;
        ao[mt] = (uint32_t)((alive[mt] ? t : 0) * K) + (uint32_t)(g4 * 16);
    }
    const uint8_t* const wbase = p.w + k_begin;
    const uint8_t* const abase = p.a + k_begin;
    const uint4 z4 = {0u, 0u, 0u, 0u};

    // Block scales of every 128-wide step, loaded together with the step's
    // operands so the step never waits on them.  fp32 scales: w_scale per
    // weight sub-tile (one 128-row block) and a_scale per token of the
    // accumulator rows this lane holds.  UE8M0: the E8M0 codes of this lane's
    // operand rows (weight sub-tile block, token 16*mt + r16).  Rows past N or
    // M read the last block's or token's scales (their results are never
    // stored): every load of a group is unconditional, so the compiler counts
    // the loads in flight exactly and the next group stays in flight while
    // this one is multiplied (a load under a branch makes it wait for all).
    [[maybe_unused]] const int last_blk = (N - 1) >> 7;
    constexpr bool E8M0 = (OP == OP_BLOCK_UE8M0);
    using ScT = typename std::conditional<E8M0, int, float>::type;
    constexpr int NSA = (SWAP || E8M0) ? 1 : 4;
    constexpr int SCU = BLOCK ? KU : 1;  // scale buffers exist only for block ops
    constexpr int SCN = BLOCK ? NT : 1;
    constexpr int SCM = BLOCK ? MT : 1;
#define QBG_LOAD_SCALES(STEP, SWV, SAV)                                                   \
    if constexpr (E8M0) {                                                                 \
        const int64_t g_ = (k_begin >> 7) + (STEP);                                       \
        const uint8_t* wc_ = reinterpret_cast<const uint8_t*>(p.w_scale);                 \
        const uint8_t* ac_ = reinterpret_cast<const uint8_t*>(p.a_scale);                 \
        _Pragma("unroll") for (int j = 0; j < NT; ++j)                                    \
            SWV[j] = (int)wc_[(int64_t)min((n_wave + 16 * j) >> 7, last_blk) * p.kgroups + g_]; \
        _Pragma("unroll") for (int mt = 0; mt < MT; ++mt)                                 \
            SAV[mt][0] = (int)ac_[(int64_t)min(16 * mt + r16, M - 1) * p.kgroups + g_];   \
    } else if constexpr (BLOCK) {                                                         \
        const int64_t g_ = (k_begin >> 7) + (STEP);                                       \
        _Pragma("unroll") for (int j = 0; j < NT; ++j)                                    \
            SWV[j] = block_scale<OP>(p.w_scale,                                           \
                         (int64_t)min((n_wave + 16 * j) >> 7, last_blk) * p.kgroups + g_); \
        _Pragma("unroll") for (int mt = 0; mt < MT; ++mt)                                 \
            _Pragma("unroll") for (int v = 0; v < NSA; ++v) {                             \
                const int t_ = SWAP ? 16 * mt + r16 : 16 * mt + 4 * g4 + v;               \
                SAV[mt][v] = block_scale<OP>(p.a_scale, (int64_t)min(t_, M - 1) * p.kgroups + g_); \
            }                                                                             \
    }

    auto compute = [&](const uint4 (&wl)[NT], const uint4 (&wh)[NT], const uint4 (&al)[MT],
                       const uint4 (&ah)[MT], const ScT (&sw)[SCN],
                       const ScT (&sa)[SCM][NSA]) __attribute__((always_inline)) {
        if constexpr (E8M0) {
#pragma unroll
            for (int j = 0; j < NT; ++j)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[j][mt] = SWAP ? mma_step_e8m0(wl[j], wh[j], al[mt], ah[mt], acc[j][mt],
                                                      sw[j], sa[mt][0])
                                      : mma_step_e8m0(al[mt], ah[mt], wl[j], wh[j], acc[j][mt],
                                                      sa[mt][0], sw[j]);
        } else if constexpr (BLOCK) {
#pragma unroll
            for (int j = 0; j < NT; ++j)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const AccV zero = {0, 0, 0, 0};
                    const AccV tmp = SWAP ? mma_step<OP>(wl[j], wh[j], al[mt], ah[mt], zero)
                                          : mma_step<OP>(al[mt], ah[mt], wl[j], wh[j], zero);
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        acc[j][mt][v] = __builtin_fmaf(tmp[v], sa[mt][SWAP ? 0 : v] * sw[j],
                                                       acc[j][mt][v]);
                }
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
    // Workgroups start at different load groups of K and wrap around (when K
    // splits into whole groups), so side-by-side workgroups do not read the same
    // K offset of rows a power-of-two stride apart.  PHYS maps a loop step to
    // the K step it reads; a group's steps stay contiguous.
    constexpr int kStride = WK * KU;
    const int n_groups = full_steps / kStride;
    const int rot = (p.rotate && nsteps == full_steps && full_steps % kStride == 0 && n_groups > 1)
                        ? (int)(blockIdx.x % (unsigned)n_groups) * kStride : 0;
#define QBG_PHYS(S) ((S) + rot < full_steps ? (S) + rot : (S) + rot - full_steps)
#define QBG_LOAD_GROUP(SG, WL, WH, AL, AH, SW, SA)                                \
    _Pragma("unroll") for (int u = 0; u < KU; ++u) {                              \
        const int off = (QBG_PHYS(SG) + u) * 128;                                 \
        QBG_LOAD_SCALES(QBG_PHYS(SG) + u, SW[u], SA[u])                           \
        const uint8_t* const wb_ = wbase + off;                                   \
        const uint8_t* const ab_ = abase + off;                                   \
        _Pragma("unroll") for (int j = 0; j < NT; ++j) {                          \
            WL[u][j] = ld16(wb_ + wo[j]);                                         \
            WH[u][j] = ld16(wb_ + wo[j] + 64);                                    \
        }                                                                         \
        _Pragma("unroll") for (int mt = 0; mt < MT; ++mt) {                       \
            AL[u][mt] = ld16(ab_ + ao[mt]);                                       \
            AH[u][mt] = ld16(ab_ + ao[mt] + 64);                                  \
        }                                                                         \
    }
#define QBG_COMPUTE_GROUP(WL, WH, AL, AH, SW, SA)                                 \
    _Pragma("unroll") for (int u = 0; u < KU; ++u)                                \
        compute(WL[u], WH[u], AL[u], AH[u], SW[u], SA[u]);
    // Keeps a group's multiply behind the loads issued before it: the operands
    // pass through empty volatile asm placed after those loads, so the wait for
    // them (and the multiply) cannot be scheduled ahead of the next group's
    // loads, which would leave that group unissued while this one lands.
#define QBG_AFTER_LOADS(WL, WH, AL, AH, SW, SA)                                   \
    asm volatile("" ::: "memory");                                                \
    _Pragma("unroll") for (int u = 0; u < KU; ++u) {                              \
        _Pragma("unroll") for (int j = 0; j < NT; ++j) {                          \
            pin16(WL[u][j]);                                                      \
            pin16(WH[u][j]);                                                      \
        }                                                                         \
        _Pragma("unroll") for (int mt = 0; mt < MT; ++mt) {                       \
            pin16(AL[u][mt]);                                                     \
            pin16(AH[u][mt]);                                                     \
        }                                                                         \
    }

    if constexpr (LOC) {
        constexpr int NTHR = 64 * WN * WK;
        constexpr int NWV = WN * WK;
        constexpr int QT = OP == OP_INT8 ? 1 : 0;
        // LDS: the chunk's codes [M][RS] (RS whole 256-byte groups, so the
        // chunk swizzle stays inside a row), the amax partials [M][NWV] and the
        // scales [M] (fp32), then the M bf16 rows (2MK bytes, whole 1 KB loads).
        const int RS = (chunk + 255) & ~255;
        char* act = smem_raw;
        float* l_red = reinterpret_cast<float*>(act + M * RS);
        float* l_sc = l_red + M * NWV;
        char* xs = reinterpret_cast<char*>(l_sc) + ((M * 4 + 15) & ~15);
        const int xbytes = 2 * M * (int)K;
        for (int i = wave; i * 1024 < xbytes; i += NWV) {
            const int off = min(i * 1024 + lane * 16, xbytes - 16);
            lds_dma16(reinterpret_cast<const uint8_t*>(p.x) + off, xs + i * 1024);
        }
        // Then both load groups of this wave.  Loads complete in issue order, so
        // once at most these 4 * KU * NT weight loads are in flight the wave's row
        // loads have landed; the barrier covers every wave's.  The empty asm
        // statements keep the compiler from moving the weight loads ahead of the
        // row loads.
        asm volatile("" ::: "memory");
        uint4 wlg[2][KU][NT], whg[2][KU][NT];
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int u = 0; u < KU; ++u) {
                const uint8_t* const wb_ = wbase + (wk * KU + g * WK * KU + u) * 128;
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    wlg[g][u][j] = ld16(wb_ + wo[j]);
                    whg[g][u][j] = ld16(wb_ + wo[j] + 64);
                }
            }
        asm volatile("" ::: "memory");
        wait_vmcnt<4 * KU * NT>();
        __builtin_amdgcn_s_barrier();
        local_quantize_rows<QT, NTHR>(M, (int)K, k_begin, chunk, lds_addr(xs), lds_addr(act), RS,
                                      lds_addr(reinterpret_cast<char*>(l_red)),
                                      lds_addr(reinterpret_cast<char*>(l_sc)));
        __builtin_amdgcn_s_barrier();
        // Products: lane (r16, g4) takes 16-byte chunks g4 and g4 + 4 of its
        // token row (dead token slots read row 0) for each of its steps.
        ScT swd[SCN] = {};
        ScT sad[SCM][NSA] = {};
        const int arow = alive[0] ? r16 : 0;
        const uint32_t abs_ = lds_addr(act) + (uint32_t)(arow * RS);
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int u = 0; u < KU; ++u) {
                const int c = (wk * KU + g * WK * KU + u) * 8 + g4;
                uint4 al[1], ah[1];
                lds_read2(abs_ + (uint32_t)((c ^ (arow & 15)) << 4),
                          abs_ + (uint32_t)(((c + 4) ^ (arow & 15)) << 4), al[0], ah[0]);
                compute(wlg[g][u], whg[g][u], al, ah, swd, sad);
            }
        // a_q and a_scale: the chunk's codes leave LDS once, 16 bytes per thread
        // and pass, spread over the workgroups of the K chunk.
        const int cu = chunk >> 4;
        const int units = M * cu;
        for (int e = (int)(blockIdx.x * NTHR + threadIdx.x); e < units;
             e += (int)(gridDim.x * NTHR)) {
            const int r = e / cu, col = e - r * cu;
            const uint4 v = *reinterpret_cast<const uint4*>(act + r * RS + ((col ^ (r & 15)) << 4));
            *reinterpret_cast<uint4*>(p.a_out + (int64_t)r * K + k_begin + col * 16) = v;
        }
        if (split == 0 && blockIdx.x == 0 && (int)threadIdx.x < M)
            p.a_scale_out[threadIdx.x] = l_sc[threadIdx.x];
        es.apply_a_lds(l_sc, M);
        __syncthreads();  // the reduction below reuses this LDS
    } else {
    // The end test comes before a group's prefetch, never around it: on
    // every path into a multiply the same loads are in flight, so the
    // compiler waits for the current group only (a prefetch under a branch
    // would make it wait for the next group too).
    int s0 = wk * KU;
    if (s0 + KU <= full_steps) {
        uint4 wl0[KU][NT], wh0[KU][NT], wl1[KU][NT], wh1[KU][NT];
        uint4 al0[KU][MT], ah0[KU][MT], al1[KU][MT], ah1[KU][MT];
        ScT sw0[SCU][SCN], sw1[SCU][SCN], sa0[SCU][SCM][NSA], sa1[SCU][SCM][NSA];
        QBG_LOAD_GROUP(s0, wl0, wh0, al0, ah0, sw0, sa0)
        while (true) {
            const int s1 = s0 + kStride;
            if (s1 + KU > full_steps) {
                QBG_COMPUTE_GROUP(wl0, wh0, al0, ah0, sw0, sa0)
                s0 = s1;
                break;
            }
            QBG_LOAD_GROUP(s1, wl1, wh1, al1, ah1, sw1, sa1)
            QBG_AFTER_LOADS(wl0, wh0, al0, ah0, sw0, sa0)
            QBG_COMPUTE_GROUP(wl0, wh0, al0, ah0, sw0, sa0)
            const int s2 = s1 + kStride;
            if (s2 + KU > full_steps) {
                QBG_COMPUTE_GROUP(wl1, wh1, al1, ah1, sw1, sa1)
                s0 = s2;
                break;
            }
            QBG_LOAD_GROUP(s2, wl0, wh0, al0, ah0, sw0, sa0)
            QBG_AFTER_LOADS(wl1, wh1, al1, ah1, sw1, sa1)
            QBG_COMPUTE_GROUP(wl1, wh1, al1, ah1, sw1, sa1)
            s0 = s2;
        }
    }
#undef QBG_LOAD_GROUP
#undef QBG_COMPUTE_GROUP
#undef QBG_AFTER_LOADS
#undef QBG_PHYS
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
                wl[j] = (wlive[j] && lo_ok) ? ld16(wbase + off + wo[j]) : z4;
                wh[j] = (wlive[j] && hi_ok) ? ld16(wbase + off + wo[j] + 64) : z4;
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                al[mt] = (alive[mt] && lo_ok) ? ld16(abase + off + ao[mt]) : z4;
                ah[mt] = (alive[mt] && hi_ok) ? ld16(abase + off + ao[mt] + 64) : z4;
            }
            ScT swt[SCN], sat[SCM][NSA];
            QBG_LOAD_SCALES(s, swt, sat)
            compute(wl, wh, al, ah, swt, sat);
        }
    }

    }
#undef QBG_LOAD_SCALES
    finish_tile<OP, SWAP, NT, MT, WN, WK, 1, kMaxTokensPerLaunch, RT>(p, red, acc, wn, wk, &s_last,
                                                                     es);
}

// ---------------------------------------------------------------------------
// Prefill tile: past the matrix-core ridge (hundreds of tokens and more) the
// GEMM is bound by the matrix cores, so the tile maximizes reuse instead of
// weight bytes in flight.  A workgroup computes BM tokens x BN weight rows
// with WM x WN waves; each wave owns (BM/WM) x (BN/WN) outputs as 32x32
// matrix-core tiles (the scaled 32x32x64 MFMA, unscaled; its accumulator
// holds row 8*(v/4) + 4*(lane/32) + v%4 and column lane%32 in element v of
// lane `lane`).  Token and weight rows stream through an NS-deep LDS ring of
// BK-byte K stages (BK / 64 MFMA K steps each), filled with direct
// global->LDS loads; 128-byte stages make every row read one whole cache line.
// A lane supplies, for step s, the 16-byte chunks (BK/32) (lane/32) + 2 s and
// the next one of its row for both operands (the same K positions, so any
// assignment gives the same sums); chunks are swizzled per row (pf_slot) so
// those reads spread over the LDS banks.  Workgroups run in groups of 8 token
// tiles sweeping the weight tiles, so those in flight share weight tiles in
// the caches.  split_k is 1; K % BK == 0.
// ---------------------------------------------------------------------------
typedef int v16i __attribute__((ext_vector_type(16)));

// A 16-byte-per-lane global->LDS load written in asm: the compiler does not
// count it, so the LDS reads it schedules are not held back until every such
// load has landed; the kernel waits for them itself with vmcnt.  The address
// is a wave-uniform base plus a 32-bit per-lane offset; m0 holds the wave's
// LDS destination (lane l writes bytes 16 l .. 16 l + 15 from there).
__device__ __forceinline__ void lds_dma16_untracked(uint32_t voff, const uint8_t* sbase,
                                                    uint32_t lds_wave_dst) {
    asm volatile("global_load_lds_dwordx4 %0, %1" :: "v"(voff), "s"(sbase), "{m0}"(lds_wave_dst)
                 : "memory");
}
// The same with 4 bytes per lane (lane l writes bytes 4 l .. 4 l + 3).
__device__ __forceinline__ void lds_dma4_untracked(const void* g, uint32_t lds_wave_dst) {
    asm volatile("global_load_lds_dword %0, off" :: "v"(g), "{m0}"(lds_wave_dst) : "memory");
}
// Wait until this wave's LDS accesses have completed (a waitcnt the compiler
// sees, so it does not wait again before using their results).
__device__ __forceinline__ void wait_lgkm0() {
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// Scheduling groups for the compiler: up to two LDS reads, then one product,
// NM times; reads left over go last.
template <int NR, int NM, int K = 0>
__device__ __forceinline__ void sched_reads_products() {
    if constexpr (K < NM) {
        constexpr int r = 2 * K < NR ? (2 * K + 1 < NR ? 2 : 1) : 0;
        if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        sched_reads_products<NR, NM, K + 1>();
    } else if constexpr (NR > 2 * NM) {
        __builtin_amdgcn_sched_group_barrier(0x100, NR - 2 * NM, 0);
    }
}

// Wait until at most n stages of LPW loads each are outstanding, n in [0, NS-1].
template <int LPW, int NS>
__device__ __forceinline__ void wait_prefill(int n) {
#define QBG_VMW(c) __builtin_amdgcn_s_waitcnt(((c) & 15) | (7 << 4) | (15 << 8) | (((c) >> 4) << 14))
    static_assert((NS - 1) * LPW <= 63 && NS <= 6, "vmcnt range");
    switch (n) {
        case 0: QBG_VMW(0); break;
        case 1: QBG_VMW(1 * LPW); break;
        case 2: if constexpr (NS > 2) { QBG_VMW(2 * LPW); } break;
        case 3: if constexpr (NS > 3) { QBG_VMW(3 * LPW); } break;
        case 4: if constexpr (NS > 4) { QBG_VMW(4 * LPW); } break;
        default: if constexpr (NS > 5) { QBG_VMW(5 * LPW); } break;
    }
#undef QBG_VMW
}

// Slot of 16-byte chunk c of stage row r (an involution in c).  For the reads
// above (lane l: row l % 32, chunks (BK/32) (l / 32) + 2 s + h) the 16-byte
// reads of a wave hit distinct banks within every 8 consecutive lanes on a
// 128-byte bank line, and within every 16 consecutive lanes and every lanes
// {8 j .. 8 j + 7} + {32 + 8 j .. 32 + 8 j + 7} on a 256-byte line; rows 32
// apart share the swizzle.
template <int BK>
__device__ __forceinline__ int pf_slot(int c, int r) {
    if constexpr (BK == 64)
        return c ^ (((r >> 2) & 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 1));
    else
        return c ^ (((r >> 1) & 7) ^ ((r & 1) << 2));
}

// Two floats to two bf16 (round to nearest even) in one word, low = a.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// Grouped form of the prefill tiles: the token tiles of all experts form one
// list, expert after expert, each expert's routed rows offsets[e] ..
// offsets[e+1]-1 (clamped to [0, rows], as in the grouped LDS launch) cut
// into ceil(rows_e / BM) tiles.  Every wave scans the device offsets itself,
// 64 experts per pass, so the tile's expert is known without a barrier.
__device__ __forceinline__ void grouped_rows(const GemmArgs& p, int e, int& r0, int& r1) {
    r0 = min(max(p.offsets[e], 0), p.rows);
    r1 = min(max(p.offsets[e + 1], r0), p.rows);
}

// Token tiles over all experts, capped at ceil(rows / BM) + min(experts, rows),
// the most that well-formed offsets give (each expert adds at most one partial
// tile) and the count the host sizes the grid for.
template <int BM>
__device__ int grouped_token_tiles(const GemmArgs& p, int lane) {
    int total = 0;
    for (int c = 0; c < p.experts; c += 64) {
        int cnt = 0;
        if (c + lane < p.experts) {
            int r0, r1;
            grouped_rows(p, c + lane, r0, r1);
            cnt = (r1 - r0 + BM - 1) / BM;
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
        total += cnt;
    }
    return __builtin_amdgcn_readfirstlane(min(total, (p.rows + BM - 1) / BM + min(p.experts, p.rows)));
}

// The expert of token tile mt of that list, its rows [r0, r1) and its first
// tile's index in the list (uniform across the wave).
template <int BM>
__device__ void grouped_find_tile(const GemmArgs& p, int lane, int mt, int& e_out, int& r0_out,
                                  int& r1_out, int& first_out) {
    int base = 0;
    e_out = 0, r0_out = 0, r1_out = 0, first_out = 0;
    for (int c = 0; c < p.experts; c += 64) {
        const int e = c + lane;
        int r0 = 0, r1 = 0, cnt = 0;
        if (e < p.experts) {
            grouped_rows(p, e, r0, r1);
            cnt = (r1 - r0 + BM - 1) / BM;
        }
        int inc = cnt;  // inclusive prefix over the lanes
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(inc, d, 64);
            if (lane >= d) inc += y;
        }
        const unsigned long long hit = __ballot(base + inc > mt);
        if (hit) {  // the first lane whose tiles reach past mt holds it
            const int l = __builtin_ctzll(hit);
            e_out = __builtin_amdgcn_readfirstlane(__shfl(e, l, 64));
            r0_out = __builtin_amdgcn_readfirstlane(__shfl(r0, l, 64));
            r1_out = __builtin_amdgcn_readfirstlane(__shfl(r1, l, 64));
            first_out = __builtin_amdgcn_readfirstlane(base + __shfl(inc - cnt, l, 64));
            return;
        }
        base += __shfl(inc, 63, 64);
    }
}

template <int OP, int BM, int BN, int WM, int WN, int NS, int BK, bool GRP = false>
__global__ __launch_bounds__(64 * WM * WN)
__attribute__((amdgpu_waves_per_eu((BM / WM / 32) * (BN / WN / 32) > 8 ? 1 : 2)))
void gemm_prefill_kernel(const GemmArgs p) {
    constexpr int NW = WM * WN;
    constexpr int TMW = BM / WM / 32, TNW = BN / WN / 32;  // 32x32 tiles per wave
    constexpr int SPS = BK / 64;                           // MFMA K steps per stage
    constexpr int STAGE = (BM + BN) * BK;
    constexpr int RPI = 1024 / BK, LPR = BK / 16;  // rows per 1 KB load, lanes per row
    constexpr int LI = STAGE / 1024;               // 1 KB loads per stage
    constexpr int LPW = LI / NW;
    constexpr int QA = BM / RPI / NW;              // loads of a wave that bring token rows
    constexpr bool BF = OP == OP_BLOCK_F32;        // fp32 block scales ride in each slot
    constexpr int SLOT = STAGE + (BF ? NW * 256 : 0);
    constexpr int LPS = LPW + (BF ? 1 : 0);        // loads per wave per stage
    static_assert(BK == 64 || BK == 128, "stage width");
    static_assert(LI % NW == 0 && (BM / RPI) % NW == 0 && TMW >= 1 && TNW >= 1 &&
                  BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "prefill tile shape");
    static_assert(OP == OP_FP8 || OP == OP_INT8 || OP == OP_BLOCK_UE8M0 || OP == OP_BLOCK_F32,
                  "prefill tile: FP8, INT8 or Block-FP8");
    static_assert(!BF || (BK == 128 && NW > BM / 64), "fp32 Block-FP8: a scale load per wave");
    constexpr bool I8 = OP == OP_INT8;
    constexpr bool BU = OP == OP_BLOCK_UE8M0;  // one 128-wide scale group per stage
    static_assert(!BU || BK == 128, "Block-FP8: 128-byte stages");
    static_assert(!GRP || OP == OP_FP8 || OP == OP_INT8, "grouped prefill tiles: per-channel ops");
    using AccT = std::conditional_t<I8, v16i, v16f>;
    const bool raw = I8 && p.raw_i32;  // INT8: write the int32 sums (no scales given)
    extern __shared__ __attribute__((aligned(16))) char smem_lds[];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
    // Grouped: M becomes the tile's expert's row end (rows are global routed
    // rows), the weights and their scales that expert's.
    int M = p.M;
    const int N = p.N;
    const int64_t K = p.K;
    const uint8_t* w_base = p.w;
    const float* w_sc = reinterpret_cast<const float*>(p.w_scale);
    const int GM = GRP ? grouped_token_tiles<BM>(p, lane) : (M + BM - 1) / BM;
    const int GN = (N + BN - 1) / BN, tiles = GM * GN;
    const int T = p.k_chunk / BK;  // stages (of this workgroup's K chunk)
    // This workgroup's tile, as a position in the tile order (groups of GT
    // token tiles sweeping the weight tiles).  Workgroups are dealt to the 8
    // XCDs in turn; XCD x takes the x-th contiguous run of the order, so the
    // tiles that share its L2 are neighbours (a few token tiles by a few
    // weight tiles).  The grid is rounded up to a multiple of 8.
    // Split-K: the order runs chunk by chunk (chunk ks of every tile, then
    // chunk ks + 1), so an XCD still sweeps neighbouring tiles of one chunk.
    constexpr int GT = 8;  // token tiles per group of the tile order
    const int SK = p.split_k, work = tiles * SK;
    const int per = (work + 7) / 8;
    const int cur = ((int)blockIdx.x & 7) * per + ((int)blockIdx.x >> 3);
    if (cur >= min(((int)blockIdx.x & 7) * per + per, work)) return;
    const int ks = cur / tiles, tcur = cur - ks * tiles;
    const int64_t kbase = (int64_t)ks * p.k_chunk;
    const int gbase = ks * T;  // Block-FP8: the chunk's first 128-wide scale group
    auto coords = [&](int t, int& m0, int& n0) {
        const int group = t / (GT * GN), first = group * GT, gsz = min(GT, GM - first);
        const int local = t - group * GT * GN;
        m0 = (first + local % gsz) * BM;
        n0 = (local / gsz) * BN;
    };

    // Load q of a wave (instruction i = wave + q * NW of a stage) covers stage
    // rows RPI i .. RPI i + RPI - 1 (tokens first, then weight rows); lane l
    // brings row RPI i + l / LPR into slot l % LPR, i.e. source chunk
    // pf_slot(l % LPR, row).  Rows past M or N repeat the last row (never
    // stored).  Offsets are from the tile's first row.
    const uint8_t* a_tile;
    const uint8_t* w_tile;
    uint32_t voff[LPW];
    auto setup = [&](int m0, int n0) {
        a_tile = p.a + (int64_t)m0 * K + kbase;
        w_tile = w_base + (int64_t)n0 * K + kbase;
#pragma unroll
        for (int q = 0; q < LPW; ++q) {
            const int R = RPI * (wave + q * NW) + lane / LPR;
            const uint32_t cg = (uint32_t)pf_slot<BK>(lane % LPR, R) * 16u;
            if (q < QA)
                voff[q] = (uint32_t)(min(m0 + R, M - 1) - m0) * (uint32_t)K + cg;
            else
                voff[q] = (uint32_t)(min(n0 + R - BM, N - 1) - n0) * (uint32_t)K + cg;
        }
    };
    const uint32_t lds_wave = lds_addr(smem_lds) + 1024u * (uint32_t)__builtin_amdgcn_readfirstlane(wave);
    // fp32 Block-FP8: the scales of the chunk's stage g (group gbase + g) behind
    // the stage's operands,
    // one 4-byte load per wave: waves below BM/64 bring 64 token rows' a_scale each
    // (slot offset STAGE + 4 r), the next wave the tile's weight-block w_scale
    // (offset STAGE + 4 BM + 4 b), the rest repeat that (their areas go unread).
    int sm0 = 0, sn0 = 0;  // the tile's first token row and weight row
    auto issue_group_scales = [&](int g) {
        const int Gs = (int)(K / 128);
        const float* src;
        if (wave < BM / 64) {
            src = reinterpret_cast<const float*>(p.a_scale) + (int64_t)min(sm0 + 64 * wave + lane, M - 1) * Gs + gbase + g;
        } else {
            const int nb = (N + 127) / 128;
            src = reinterpret_cast<const float*>(p.w_scale) + (int64_t)min(sn0 / 128 + lane, nb - 1) * Gs + gbase + g;
        }
        lds_dma4_untracked(src, lds_addr(smem_lds) + (uint32_t)((g % NS) * SLOT + STAGE) +
                                    256u * (uint32_t)__builtin_amdgcn_readfirstlane(wave));
    };
#define QBG_PF_ISSUE(ST)                                                                  \
    {                                                                                     \
        const uint32_t slot_ = lds_wave + (uint32_t)(((ST) % NS) * SLOT);                 \
        const int64_t koff_ = (int64_t)(ST) * BK;                                         \
        _Pragma("unroll") for (int q = 0; q < LPW; ++q)                                  \
            lds_dma16_untracked(voff[q], (q < QA ? a_tile : w_tile) + koff_,              \
                                slot_ + q * NW * 1024);                                   \
        if constexpr (BF) issue_group_scales(ST);                                        \
    }
    // The tile's token and weight scales (rows past M or N repeat the last
    // one) go behind the ring; they are loaded first, so the wait for stage 0
    // covers them.
    constexpr int SCI = (BM + BN) / 64;  // 64 scales per load instruction
    static_assert((BM + BN) % 64 == 0, "scale rows");
    auto issue_scales = [&](int m0, int n0) {
#pragma unroll
        for (int q = 0; q < (SCI + NW - 1) / NW; ++q) {
            const int si = wave + q * NW;
            if (si < SCI) {
                const int r = 64 * si + lane;
                const float* src = r < BM ? reinterpret_cast<const float*>(p.a_scale) + min(m0 + r, M - 1)
                                          : w_sc + min(n0 + r - BM, N - 1);
                lds_dma4_untracked(src, lds_addr(smem_lds) + (uint32_t)(NS * SLOT) +
                                            256u * (uint32_t)__builtin_amdgcn_readfirstlane(si));
            }
        }
    };
    // LDS offsets (within a stage) of this lane's chunks of its row in the
    // first 32x32 tile, per step and half; tile i lies 32 * i rows further,
    // with the same swizzle.
    const int ra = wm * (BM / WM) + (lane & 31), rb = BM + wn * (BN / WN) + (lane & 31);
    const int c0 = (BK / 32) * (lane >> 5);
    uint32_t oa[SPS][2], ob[SPS][2];
#pragma unroll
    for (int st = 0; st < SPS; ++st)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            oa[st][h] = ra * BK + (pf_slot<BK>(c0 + 2 * st + h, ra) << 4);
            ob[st][h] = rb * BK + (pf_slot<BK>(c0 + 2 * st + h, rb) << 4);
        }
    // The operands of step s of stage st: plain LDS reads, scheduled (and
    // waited for) by the compiler; the loads that fill LDS are invisible to it.
    // Read in the order the products use them (A0, every B, then A1, A2, ...),
    // so a step's first products wait only on the previous step's first reads.
    // Block-FP8 also reads the stage's UE8M0 codes: the lane's token row of each
    // A tile and the 128-row weight block of each B tile (codes staged behind
    // the ring: [BM][G] token codes, then [BN/128][G] weight-block codes).
    struct Ops {
        v8i xa[TMW], xb[TNW];
        int ca[BU ? TMW : 1], cb[BU ? TNW : 1];
        float4 sa[BF ? 4 * TMW : 1];  // fp32 blocks, second step of a stage: a_scale of
        float sw[BF ? TNW : 1];       // rows 8 g + 4 (lane / 32) + 0..3 of each A tile; w_scale
    };
    const int G = (int)(K / 128);
    const uint8_t* const codes = reinterpret_cast<const uint8_t*>(smem_lds + NS * SLOT);
    auto fetch = [&](int st, int s, Ops& o) {
        const char* sbase = smem_lds + (st % NS) * SLOT;
        auto rd = [&](uint32_t o0, uint32_t o1) {
            const uint4 lo = *reinterpret_cast<const uint4*>(sbase + o0);
            const uint4 hi = *reinterpret_cast<const uint4*>(sbase + o1);
            return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        };
        o.xa[0] = rd(oa[s][0], oa[s][1]);
#pragma unroll
        for (int j = 0; j < TNW; ++j) o.xb[j] = rd(ob[s][0] + 32 * BK * j, ob[s][1] + 32 * BK * j);
#pragma unroll
        for (int i = 1; i < TMW; ++i) o.xa[i] = rd(oa[s][0] + 32 * BK * i, oa[s][1] + 32 * BK * i);
        if constexpr (BF) {
            if (s == 1) {  // the stage's group scales, read before its slot is refilled
                const float* gs = reinterpret_cast<const float*>(sbase + STAGE);
#pragma unroll
                for (int i = 0; i < TMW; ++i)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4)
                        o.sa[4 * i + g4] = *reinterpret_cast<const float4*>(
                            gs + wm * (BM / WM) + 32 * i + 8 * g4 + 4 * (lane >> 5));
#pragma unroll
                for (int j = 0; j < TNW; ++j) o.sw[j] = gs[BM + (wn * (BN / WN) + 32 * j) / 128];
            }
        }
        if constexpr (BU) {
#pragma unroll
            for (int i = 0; i < TMW; ++i) o.ca[i] = codes[(ra + 32 * i) * G + gbase + st];
#pragma unroll
            for (int j = 0; j < TNW; ++j)
                o.cb[j] = codes[(BM + (wn * (BN / WN) + 32 * j) / 128) * G + gbase + st];
        }
    };
    AccT acc[TMW][TNW];
    // One 64-byte K step: FP8, the lane's 32 codes converted to bf16 and four
    // 32x32x16 BF16 products per output tile (exact E4M3 products, see
    // mma16_e4m3); INT8, two 32x32x32 products (the lane's first 16 bytes for
    // every tile, then its second 16 bytes, so a product never waits on the one
    // just before).
    AccT tmp[BF ? TMW : 1][BF ? TNW : 1];  // fp32 blocks: the current group's sums
    auto mma = [&](const Ops& o, int half) {
        const auto& xa = o.xa;
        const auto& xb = o.xb;
        if constexpr (BF) {
            // a stage is one 128-wide group: its two steps sum into tmp, which is then
            // added to the accumulator times a_scale[t, g] * w_scale[block, g]
#pragma unroll
            for (int i = 0; i < TMW; ++i)
#pragma unroll
                for (int j = 0; j < TNW; ++j)
                    tmp[i][j] = mma32_e4m3(xa[i], xb[j], half ? tmp[i][j] : v16f{});
            if (half) {
#pragma unroll
                for (int i = 0; i < TMW; ++i)
#pragma unroll
                    for (int j = 0; j < TNW; ++j)
#pragma unroll
                        for (int g4 = 0; g4 < 4; ++g4) {
                            const float4 a4 = o.sa[4 * i + g4];
                            const float f[4] = {a4.x * o.sw[j], a4.y * o.sw[j], a4.z * o.sw[j], a4.w * o.sw[j]};
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                acc[i][j][4 * g4 + e] = fmaf(tmp[i][j][4 * g4 + e], f[e], acc[i][j][4 * g4 + e]);
                        }
            }
        } else if constexpr (I8) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < TMW; ++i)
#pragma unroll
                    for (int j = 0; j < TNW; ++j) {
                        const v4i a = h ? xa[i].s4567 : xa[i].s0123;
                        const v4i b = h ? xb[j].s4567 : xb[j].s0123;
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[i][j], 0, 0, 0);
                    }
        } else if constexpr (BU) {
            // each lane's codes are scaled by 2^(ca-127) and 2^(cb-127) as they are converted
#pragma unroll
            for (int i = 0; i < TMW; ++i)
#pragma unroll
                for (int j = 0; j < TNW; ++j)
                    acc[i][j] = mma32_e4m3(xa[i], xb[j], acc[i][j], ue8m0_value((uint32_t)o.ca[i]),
                                           ue8m0_value((uint32_t)o.cb[j]));
        } else {
#pragma unroll
            for (int i = 0; i < TMW; ++i)
#pragma unroll
                for (int j = 0; j < TNW; ++j)
                    acc[i][j] = mma32_e4m3(xa[i], xb[j], acc[i][j]);
        }
    };
    // Issue order of one step: two LDS reads, one product, and so on, so the
    // reads of the next step overlap this step's products.
    auto interleave = [] { sched_reads_products<2 * (TMW + TNW), (I8 ? 2 : 4) * TMW * TNW>(); };
    // Step u + 1 is read into registers while step u's products run.  When
    // step u + 1 opens stage st, the wave waits for that stage's loads, then
    // at the barrier every wave has waited for its reads of stage st - 1, so
    // slot (st - 1) % NS is refilled with stage st - 1 + NS: the ring keeps
    // NS - 1 stages in flight beyond the one being read.  The loop runs steps
    // in pairs (a stage opens at the second of each pair when SPS is 2); the
    // last step is peeled off so that every step in the loop reads, and the
    // compiler's wait for the reads stays after the products.
#define QBG_PF_STEP(u, OPENS, CUR, NXT, HALF)                                             \
    {                                                                                     \
        const int nx_ = (u) + 1;                                                          \
        if (OPENS) {                                                                      \
            const int st_ = nx_ / SPS;                                                    \
            wait_prefill<LPS, NS>(min(NS - 2, T - 1 - st_));                              \
            wait_lgkm0();                                                                 \
            asm volatile("s_barrier" ::: "memory");                                       \
            if (st_ - 1 + NS < T) QBG_PF_ISSUE(st_ - 1 + NS)                              \
        }                                                                                 \
        fetch(nx_ / SPS, nx_ % SPS, NXT);                                                 \
        mma(CUR, HALF);                                                                   \
        interleave();                                                                     \
    }
    // Epilogue: out[t, n] = bf16(acc * (a_scale[t] * w_scale[n])), the scales
    // read from LDS (four consecutive tokens per read).  A lane holds four
    // consecutive tokens of one column per group and writes them as four 2-byte
    // stores (the 32 lanes of a half-wave cover 64 contiguous bytes of a token
    // row); INT8 writes the float of the sum times the scale product, or, raw,
    // the int32 sums.  FULL: the whole tile lies inside M x N (no checks).
    uint16_t* out = reinterpret_cast<uint16_t*>(p.out);
    auto epilogue = [&](auto full_tag, int m0, int n0) {
        constexpr bool FULL = decltype(full_tag)::value;
        const float* asl = reinterpret_cast<const float*>(smem_lds + NS * SLOT);
        const float* wsl = asl + BM;
#pragma unroll
        for (int j = 0; j < TNW; ++j) {
            const int nl = wn * (BN / WN) + 32 * j + (lane & 31);
            const int n = n0 + nl;
            const float wsc = (raw || BU || BF) ? 0.0f : wsl[nl];
#pragma unroll
            for (int i = 0; i < TMW; ++i) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int rl = wm * (BM / WM) + 32 * i + 8 * g + 4 * (lane >> 5);
                    const int64_t o = (int64_t)(m0 + rl) * N + n;  // element (token m0 + rl, column n)
                    __builtin_amdgcn_sched_barrier(0);  // keep the scale reads next to their stores
                    if (I8 && raw) {
                        int* c = reinterpret_cast<int*>(p.out) + o;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (FULL || (m0 + rl + e < M && n < N)) c[(int64_t)e * N] = (int)acc[i][j][4 * g + e];
                        continue;
                    }
                    float x[4];
                    if constexpr (BU || BF) {  // already scaled group by group
#pragma unroll
                        for (int e = 0; e < 4; ++e) x[e] = acc[i][j][4 * g + e];
                    } else {
                        const float4 a4 = *reinterpret_cast<const float4*>(asl + rl);
                        const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) x[e] = (float)acc[i][j][4 * g + e] * (av[e] * wsc);
                    }
                    const uint32_t p01 = pack_bf16x2(x[0], x[1]), p23 = pack_bf16x2(x[2], x[3]);
                    const uint16_t v[4] = {(uint16_t)p01, (uint16_t)(p01 >> 16), (uint16_t)p23,
                                           (uint16_t)(p23 >> 16)};
                    uint16_t* c = out + o;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (FULL || (m0 + rl + e < M && n < N)) c[(int64_t)e * N] = v[e];
                }
            }
        }
    };

    int m0, n0;
    coords(tcur, m0, n0);
    if constexpr (GRP) {
        int e, r0, first;
        grouped_find_tile<BM>(p, lane, m0 / BM, e, r0, M, first);
        m0 = r0 + (m0 / BM - first) * BM;
        w_base = p.w + (int64_t)e * N * K;
        w_sc += (int64_t)e * N;
    }
    setup(m0, n0);
    sm0 = m0;
    sn0 = n0;
    if constexpr (BU) {
        // The tile's UE8M0 codes (token rows m0.., weight blocks n0/128..; rows
        // past the operands repeat the last word) as 4-byte words, G % 4 == 0,
        // through registers before any load into the ring.
        const int na = BM * G / 4, nd = na + (BN / 128) * G / 4;
        const uint32_t* a32 = reinterpret_cast<const uint32_t*>(p.a_scale);
        const uint32_t* w32 = reinterpret_cast<const uint32_t*>(p.w_scale);
        const int alim = M * G / 4 - 1, wlim = ((N + 127) / 128) * G / 4 - 1;
        const int a0w = m0 * G / 4, w0w = (n0 / 128) * G / 4;
        uint32_t* lc32 = reinterpret_cast<uint32_t*>(smem_lds + NS * SLOT);
        constexpr int CPT = 16, NTHR = 64 * NW;
        for (int base = 0; base < nd; base += CPT * NTHR) {
            uint32_t v[CPT];
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                const int d = min(base + c * NTHR + (int)threadIdx.x, nd - 1);
                v[c] = d < na ? a32[min(a0w + d, alim)] : w32[min(w0w + d - na, wlim)];
            }
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                const int d = base + c * NTHR + (int)threadIdx.x;
                if (d < nd) lc32[d] = v[c];
            }
        }
    } else if (!raw && !BF) {
        issue_scales(m0, n0);  // raw int32 outputs take no scales
    }
#pragma unroll
    for (int st = 0; st < NS; ++st)
        if (st < T) QBG_PF_ISSUE(st)
    wait_prefill<LPS, NS>(min(NS - 1, T - 1));
    wait_lgkm0();  // the staged codes, written with plain LDS stores
    asm volatile("s_barrier" ::: "memory");
#pragma unroll
    for (int i = 0; i < TMW; ++i)
#pragma unroll
        for (int j = 0; j < TNW; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;
    Ops o0, o1;
    fetch(0, 0, o0);
    const int U = T * SPS;  // steps
    int u = 0;
    // (with 128-byte stages o0 carries a stage's first step, o1 its second)
    for (; u + 2 < U; u += 2) {
        QBG_PF_STEP(u, SPS == 1, o0, o1, 0)
        QBG_PF_STEP(u + 1, true, o1, o0, 1)
    }
    if constexpr (SPS == 2) {  // an even number of steps: the last pair is always left
        QBG_PF_STEP(u, false, o0, o1, 0)
        mma(o1, 1);
    } else if (u + 1 < U) {
        QBG_PF_STEP(u, SPS == 1, o0, o1, 0)
        mma(o1, 0);
    } else {
        mma(o0, 0);
    }
    if (SK > 1) {
        // Split-K hand-off.  Each workgroup writes its chunk's sums to its own
        // slot of the tile's partials, lane-major (store v of tile (i, j) puts
        // the wave's 64 lanes side by side), with write-through stores that
        // bypass the XCD-private L2s.  It waits for them, and one thread takes a
        // ticket from the tile's arrival counter.  The last of the tile's SK
        // workgroups reads its own lanes' elements of the other slots with
        // cache-bypassing loads, adds them in chunk order (the bits do not depend
        // on which workgroup arrives last), resets the counter and runs the
        // epilogue.  The flag lives in the ring, free once every wave is past its
        // last read.  Ordering relied on (the same as the decode tiles' split-K,
        // see finish_tile): system-scope stores are performed at memory once the
        // issuing wave's counter drains; s_waitcnt and the barrier keep every
        // access in program order; the agent-scope ticket is performed at memory
        // after all of them; the last workgroup's system-scope loads, issued after
        // its ticket returned, bypass the caches and read memory.
        using PS = std::conditional_t<I8, int, float>;
        PS* part = reinterpret_cast<PS*>(p.partial) + (int64_t)tcur * SK * (BM * BN) + 64 * wave + lane;
        constexpr int VS = 64 * NW;  // stride between a lane's elements
#pragma unroll
        for (int i = 0; i < TMW; ++i)
#pragma unroll
            for (int j = 0; j < TNW; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    __hip_atomic_store(part + (int64_t)ks * (BM * BN) + ((i * TNW + j) * 16 + v) * VS,
                                       (PS)acc[i][j][v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        volatile int* s_last = reinterpret_cast<volatile int*>(smem_lds);
        if (threadIdx.x == 0) {
            const unsigned prev = __hip_atomic_fetch_add(&p.counters[tcur], 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            *s_last = prev == (unsigned)(SK - 1);
        }
        __syncthreads();
        if (!*s_last) return;
#pragma unroll
        for (int i = 0; i < TMW; ++i)
#pragma unroll
            for (int j = 0; j < TNW; ++j) {
                AccT sum = {};
                for (int sp = 0; sp < SK; ++sp) {
                    if (sp == ks) {
                        sum += acc[i][j];
                    } else {
                        AccT x;
#pragma unroll
                        for (int v = 0; v < 16; ++v)
                            x[v] = __hip_atomic_load(part + (int64_t)sp * (BM * BN) + ((i * TNW + j) * 16 + v) * VS,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                        sum += x;
                    }
                }
                acc[i][j] = sum;
            }
        if (threadIdx.x == 0)
            __hip_atomic_store(&p.counters[tcur], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (m0 + BM <= M && n0 + BN <= N)
        epilogue(std::true_type{}, m0, n0);
    else
        epilogue(std::false_type{}, m0, n0);
#undef QBG_PF_STEP
#undef QBG_PF_ISSUE
}

// Epilogue of an unsplit decode tile straight from the matrix-core registers.
// Lane l holds element v of each 16 x 16 accumulator tile at row 4*(l/16) + v,
// column l % 16: tokens x weight rows (Standard) or weight rows x tokens
// (Swap-AB).  Waves that split K (wk > 0) hand their partial tiles to the wave
// with wk == 0 through LDS, one 16-byte write and read per lane and tile; that
// wave adds them in wk order (the bits do not depend on timing) and stores.
// The per-channel scale factors of the lane's elements are loaded early
// (prefetch) and multiplied only here.
template <int OP, bool SWAP, int NTW, int MTW, int WNW, int WKW, int RT = 0>
struct RegEpilogue {
    static constexpr bool kScaled = (OP == OP_FP8 || OP == OP_INT8);
    static constexpr int NA = SWAP ? 1 : 4;  // token rows per lane and tile
    static constexpr int NWS = SWAP ? 4 : 1;  // weight rows per lane and tile
    float a[kScaled ? MTW : 1][NA];
    float w[kScaled ? NTW : 1][NWS];

    __device__ __forceinline__ int token(int mt, int v) const {
        const int lane = threadIdx.x & 63;
        return 16 * mt + (SWAP ? (lane & 15) : 4 * (lane >> 4) + v);
    }
    __device__ __forceinline__ int col(int n0, int wn, int j, int v) const {
        const int lane = threadIdx.x & 63;
        return n0 + 16 * (wn * NTW + j) + (SWAP ? 4 * (lane >> 4) + v : (lane & 15));
    }
    __device__ __forceinline__ void prefetch(const GemmArgs& p, int n0, int wn) {
        if constexpr (kScaled) {
            if (OP == OP_INT8 && p.raw_i32) return;
            const float* as = reinterpret_cast<const float*>(p.a_scale);
            const float* ws = reinterpret_cast<const float*>(p.w_scale);
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
                for (int v = 0; v < NA; ++v) a[mt][v] = as[min(token(mt, v), p.M - 1)];
#pragma unroll
            for (int j = 0; j < NTW; ++j)
#pragma unroll
                for (int v = 0; v < NWS; ++v) w[j][v] = ws[min(col(n0, wn, j, v), p.N - 1)];
        }
    }
    template <class AccV>
    __device__ __forceinline__ void finish(const GemmArgs& p, AccV (&acc)[NTW][MTW], int n0, int wn,
                                           int wk, char* lds) const {
        const int lane = threadIdx.x & 63;
        if constexpr (WKW > 1) {
            // partial tiles of the waves with wk > 0: slot ((wk-1) * WNW + wn) * NTW * MTW + tile
            if (wk > 0) {
#pragma unroll
                for (int j = 0; j < NTW; ++j)
#pragma unroll
                    for (int mt = 0; mt < MTW; ++mt) {
                        const int slot = ((wk - 1) * WNW + wn) * NTW * MTW + j * MTW + mt;
                        *reinterpret_cast<AccV*>(lds + slot * 1024 + lane * 16) = acc[j][mt];
                    }
            }
            __syncthreads();
            if (wk > 0) return;
#pragma unroll
            for (int w2 = 1; w2 < WKW; ++w2)
#pragma unroll
                for (int j = 0; j < NTW; ++j)
#pragma unroll
                    for (int mt = 0; mt < MTW; ++mt) {
                        const int slot = ((w2 - 1) * WNW + wn) * NTW * MTW + j * MTW + mt;
                        acc[j][mt] += *reinterpret_cast<const AccV*>(lds + slot * 1024 + lane * 16);
                    }
        }
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int t = token(mt, v), n = col(n0, wn, j, v);
                    if (t >= p.M || n >= p.N || (RT > 0 && n - n0 >= RT)) continue;
                    float f = 1.0f;
                    if constexpr (kScaled) f = a[mt][SWAP ? 0 : v] * w[j][SWAP ? v : 0];
                    store_out<OP>(p, t, n, acc[j][mt][v], f);
                }
    }
};

// One output tile of the LDS-staged kernel over K chunk `split` (the body of
// gemm_lds_kernel; the grouped launch runs it once per expert slice).  FM:
// 0 = the activation codes are an input; 1 = fused, published by producer
// workgroups; 2 = fused, quantized by this workgroup (LOCAL: the stages carry
// weight rows only and the chunk's codes stay resident in LDS behind the ring).
// RT > 0 (plain per-channel launches): the workgroup owns RT < TN weight rows,
// [RT * tile, RT * tile + RT); the stage rows past RT read owned rows again and
// their products are never stored.
template <int OP, bool SWAP, int AR, int NTW, int WNW, int WKW, int SK, int NS, int FM,
          int WMW, int RT = 0>
__device__ __forceinline__ void gemm_lds_tile(const GemmArgs& p, int split) {
    constexpr bool FUSE = FM == 1;
    constexpr bool LOCAL = FM == 2;
    using AccV = typename Acc<OP>::vec;
    using AccS = typename Acc<OP>::scalar;
    constexpr int NW = WNW * WKW * WMW;
    constexpr int MT = (AR + 15) / 16;
    constexpr int MTW = MT / WMW;  // token slots per wave
    static_assert(MT % WMW == 0, "token slots split evenly over the waves along M");
    constexpr int TN = 16 * NTW * WNW;
    constexpr int RB = 128 * SK;
    constexpr int ROWS = TN + (LOCAL ? 0 : AR);
    constexpr int STAGE = ROWS * RB;
    constexpr int LI = STAGE / 1024;
    constexpr int LPW = LI / NW;
    constexpr int SPW = SK / WKW;
    static_assert(RB >= 256 && RB <= 1024 && STAGE % 1024 == 0 && LI % NW == 0, "stage shape");
    static_assert(SK % WKW == 0 && (AR == 4 || AR % 16 == 0) && NS >= 2, "wave split");
    constexpr bool BLOCK = (OP == OP_BLOCK_F32 || OP == OP_BLOCK_UE8M0);
    constexpr bool E8M0 = (OP == OP_BLOCK_UE8M0);
    // fp32 block scales, Standard layout: a lane's four accumulator rows are four
    // consecutive tokens, so their scale words are one 16-byte read
    constexpr bool SC128 = (OP == OP_BLOCK_F32 && !SWAP);
    static_assert(!BLOCK || 128 % TN == 0, "a block-op tile lies in one 128-row weight block");
    static_assert(!FUSE || OP == OP_FP8 || OP == OP_INT8, "fused quantization: per-channel ops");
    static_assert(WMW == 1 || (!BLOCK && !FUSE), "large-M tiles: per-channel ops");
    static_assert(!LOCAL || ((OP == OP_FP8 || OP == OP_INT8) && WMW == 1 && AR <= 32),
                  "local quantization: per-channel decode tiles");
    // large-M tiles read each operand's chunks in batches (one wait per batch)
    constexpr bool BATCHED = WMW > 1 || MTW > 2 || NTW > 2;

    extern __shared__ __attribute__((aligned(16))) char smem_lds[];
    __shared__ int s_last;
    __shared__ int s_timed_out;  // fused: the wait for the published rows ran out
    __shared__ float s_red[NW];  // fused: amax reduction

    // the wave index is the same in every lane: readfirstlane tells the compiler,
    // so values derived from it live in scalar registers and branch uniformly
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wn = wave % WNW, wm = (wave / WNW) % WMW, wk = wave / (WNW * WMW);
    const int mt0 = wm * MTW;  // this wave's first token slot
    const int r16 = lane & 15, g4 = lane >> 4;
    const int M = p.M, N = p.N;
    const int64_t K = p.K;
    static_assert(RT == 0 || (FM == 0 && !BLOCK && WMW == 1 && RT < TN && RT % 4 == 0),
                  "owned rows: plain per-channel decode tiles");
    constexpr int RW = RT > 0 ? RT : TN;  // weight rows the workgroup owns
    const int n0 = blockIdx.x * RW;
    const int64_t k_begin = (int64_t)split * p.k_chunk;
    const int chunk = p.k_chunk;
    const int T = (chunk + RB - 1) / RB;
    // Workgroups start at different stages of K and wrap around, so the
    // workgroups running side by side do not all read the same K offset of rows
    // that lie a power-of-two stride apart.  Only whole stages are rotated.
    const int rot = (p.rotate && chunk % RB == 0) ? (int)(blockIdx.x % (unsigned)T) : 0;

    // This wave's load instructions: i = wave + q * NW of every stage.  The
    // first WBLK 1 KB blocks of a stage hold weight rows; when they split evenly
    // over the waves, whether load q reads weights is known at compile time,
    // otherwise it is decided on the (wave-uniform) wave index.
    constexpr int WBLK = TN * RB / 1024;
    constexpr bool kWholeBlocks = WBLK % NW == 0;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const uint8_t* gsrc[LPW];
    int kin[LPW];
#pragma unroll
    for (int q = 0; q < LPW; ++q) {
        const int f = (wave + q * NW) * 1024 + lane * 16;
        const int R = f / RB;
        const int cg = ((f % RB) / 16) ^ (R & 15);
        kin[q] = cg * 16;
        if (R < TN) {
            const int row = min(n0 + (R < RW ? R : R % RW), N - 1);
            gsrc[q] = p.w + (int64_t)row * K + k_begin;
        } else {
            const int t = min(R - TN, M - 1);
            gsrc[q] = p.a + (int64_t)t * K + k_begin;
        }
    }
#define QBG_KSTAGE(ST) ((ST) + rot < T ? (ST) + rot : (ST) + rot - T)
    // PART 0: the whole stage; 1: its weight rows only; 2: its activation rows
    // only.  A 1 KB load block holds rows of one kind (TN * RB is a multiple of
    // 1 KB), so the choice is uniform across the wave.
#define QBG_ISSUE_PART(ST, PART)                                                          \
    {                                                                                     \
        char* slot_ = smem_lds + ((ST) % NS) * STAGE;                                     \
        _Pragma("unroll") for (int q = 0; q < LPW; ++q) {                                \
            const bool wrow_ = kWholeBlocks ? q * NW < WBLK : (wave_u + q * NW) < WBLK;   \
            if ((PART) == 0 || ((PART) == 1) == wrow_) {                                  \
                const int off_ = QBG_KSTAGE(ST) * RB + kin[q];                            \
                const uint8_t* g_ = gsrc[q] + (off_ < chunk ? off_ : 0);                  \
                char* l_ = slot_ + (wave + q * NW) * 1024;                                \
                if (wrow_) lds_dma16<kNonTemporal>(g_, l_); else lds_dma16(g_, l_);      \
            }                                                                             \
        }                                                                                 \
    }
#define QBG_ISSUE(ST) QBG_ISSUE_PART(ST, 0)
    // Whole stage ST's rows into ring slot SLOT % NS (LOCAL prologue).
#define QBG_ISSUE_SLOT(SLOT, ST)                                                          \
    {                                                                                     \
        char* slot_ = smem_lds + ((SLOT) % NS) * STAGE;                                   \
        _Pragma("unroll") for (int q = 0; q < LPW; ++q) {                                \
            const int off_ = QBG_KSTAGE(ST) * RB + kin[q];                                \
            lds_dma16<kNonTemporal>(gsrc[q] + (off_ < chunk ? off_ : 0),                  \
                                    slot_ + (wave + q * NW) * 1024);                      \
        }                                                                                 \
    }

    AccV acc[NTW][MTW];
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt) acc[j][mt] = AccV{0, 0, 0, 0};
    // LDS byte offset (within a stage) of this lane's chunk C of weight sub-tile J.
#define QBG_W_OFF(J, C) ((16 * (wn * NTW + (J)) + r16) * RB + (((C) ^ r16) * 16))
// Activation slot MTI's row of this lane (rows past AR-1 repeat the last one)
// and the LDS address of its chunk C: within the stage (abase = the stage's
// activation rows, stride RB) or, LOCAL, within the resident codes (abase =
// the stage's K offset in them, stride RS).
#define QBG_A_ROW(MTI) min(16 * (MTI) + r16, AR - 1)
#define QBG_A_ADDR(MTI, C) \
    (abase + (uint32_t)(QBG_A_ROW(MTI) * astride) + ((uint32_t)((C) ^ (QBG_A_ROW(MTI) & 15)) << 4))

    // The epilogue's scale loads go out before the first stage's loads: loads
    // complete in issue order, so the stage waits below also cover them.
    EpiScales<OP, TN, NW * 64, AR, RT> es;
    // Plain decode tiles without split-K end from the matrix-core registers.
    constexpr bool kRegEpi = FM == 0 && WMW == 1 && AR <= 32;
    static_assert(!kRegEpi || (WKW - 1) * WNW * NTW * MTW * 1024 <= NS * STAGE,
                  "the partial tiles fit in the stage ring's LDS");
    constexpr int QT = OP == OP_INT8 ? 1 : 0;
    // LOCAL: codes of the chunk [AR rows][RS bytes] behind the ring, then the
    // amax partials [AR][NW] and the scales [AR] (fp32).
    const int RS = T * RB;
    char* act = smem_lds + NS * STAGE;
    float* l_red = reinterpret_cast<float*>(act + AR * RS);
    float* l_sc = l_red + AR * NW;
    if constexpr (LOCAL) {
        es.prefetch_w(p);
        // The M bf16 rows (2MK contiguous bytes) into xs, then the first NS-1
        // weight stages (a stage past the chunk's last reloads the last one
        // into its own slot, which is never read, so every wave issues exactly
        // (NS-1) * LPW stage loads).  Loads of one kind complete in issue
        // order: once at most those stage loads are in flight, this wave's
        // row loads have landed, and the barrier covers every wave's.
        const int xbytes = 2 * M * (int)K;
        char* xs = act + AR * RS + AR * (NW + 1) * 4;
        for (int i = wave; i * 1024 < xbytes; i += NW) {
            const int off = min(i * 1024 + lane * 16, xbytes - 16);
            lds_dma16(reinterpret_cast<const uint8_t*>(p.x) + off, xs + i * 1024);
        }
#pragma unroll
        for (int st = 0; st < NS - 1; ++st) QBG_ISSUE_SLOT(st, st < T ? st : T - 1)
        wait_vmcnt<(NS - 1) * LPW>();
        __builtin_amdgcn_s_barrier();
        // up to 4 rows: the compact form (one read pass, every wave reduces the
        // partials itself); more rows: reads batched eight to a wait.  Same bytes.
        if (M <= 4)
            local_quantize_rows<QT, NW * 64>(M, (int)K, k_begin, chunk, lds_addr(xs), lds_addr(act),
                                             RS, lds_addr(reinterpret_cast<char*>(l_red)),
                                             lds_addr(reinterpret_cast<char*>(l_sc)));
        else
            local_quantize<QT, NW * 64>(p, k_begin, chunk, lds_addr(xs), lds_addr(act), RS,
                                        lds_addr(reinterpret_cast<char*>(l_red)),
                                        lds_addr(reinterpret_cast<char*>(l_sc)));
    } else if constexpr (FUSE) {
        // Producers: the first P workgroups of the first K chunk quantize the
        // rows (row r by workgroup r % P) before loading anything else, wait
        // until their stores are acknowledged, and add the row count to the
        // published-rows slot.
        //
        // Ordering relied on (relaxed atomics, not release/acquire, whose
        // agent-scope fences would write back and invalidate whole L2s):
        //  1. publish_row's codes and scales are system-scope stores, performed
        //     at memory when the producer's counter drains (s_waitcnt 0);
        //  2. s_waitcnt and the barrier are side-effecting for the compiler, so
        //     the count's fetch_add is issued after every producer store is
        //     performed;
        //  3. a consumer issues its activation-row loads only after its poll
        //     (an agent-scope read-modify-write performed at memory) returned
        //     a count of at least M, and the barrier after the poll orders every
        //     wave's loads after it;
        //  4. those loads cannot hit a stale cache line: the kernel's start
        //     invalidates L1 and L2 for the launch, and no workgroup of this
        //     launch touches the code lines before the count is complete
        //     (producers write them with stores that bypass the caches).
        const int P = min((int)gridDim.x, M);
        if (split == 0 && (int)blockIdx.x < P) {
            unsigned rows = 0;
            for (int r = blockIdx.x; r < M; r += P, ++rows) publish_row<QT, NW * 64>(p, r, s_red);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (threadIdx.x == 0)
                __hip_atomic_fetch_add(&p.sync[0], rows, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        es.prefetch_w(p);
    } else {
        if (!kRegEpi || p.split_k != 1) es.prefetch(p);
    }

    // First NS-1 stages; a fused launch loads only their weight rows before the wait.
    if constexpr (!LOCAL) {
#pragma unroll
        for (int st = 0; st < NS - 1; ++st)
            if (st < T) QBG_ISSUE_PART(st, FUSE ? 1 : 0)
    }
    // the register epilogue's scale factors go out behind the first stages
    RegEpilogue<OP, SWAP, NTW, MTW, WNW, WKW, RT> repi;
    if constexpr (kRegEpi) {
        if (p.split_k == 1) repi.prefetch(p, n0, wn);
    }

    if constexpr (FUSE) {
        // Wait (bounded) until all M rows are published.  The poll is an atomic
        // read-modify-write, so it sees the device-wide value.  On time-out the
        // workgroup quantizes every row itself: the same bytes the producers
        // write, so the overlapping stores are harmless and the launch always
        // finishes.
        if (threadIdx.x == 0) {
            int timed_out = 1;
            for (int i = 0; i < p.wait_limit; ++i) {
                if (__hip_atomic_fetch_add(&p.sync[0], 0u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT) >= (unsigned)M) {
                    timed_out = 0;
                    break;
                }
                __builtin_amdgcn_s_sleep(8);
            }
            s_timed_out = timed_out;
        }
        __syncthreads();
        if (s_timed_out) {
            for (int r = 0; r < M; ++r) publish_row<QT, NW * 64>(p, r, s_red);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        // Departure: the last workgroup past the wait clears both slots for the
        // next launch (every producer has counted its rows before departing).
        if (threadIdx.x == 0) {
            const unsigned total = gridDim.x * gridDim.y;
            const unsigned prev = __hip_atomic_fetch_add(&p.sync[1], 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            if (prev == total - 1) {
                __hip_atomic_store(&p.sync[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(&p.sync[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        asm volatile("" ::: "memory");
        es.apply_a(p);
#pragma unroll
        for (int st = 0; st < NS - 1; ++st)
            if (st < T) QBG_ISSUE_PART(st, 2)
    }

    // Block ops: stage the scale words of the chunk (while the first stages load).
    uint32_t scl_base = 0;
    if constexpr (BLOCK) {
        uint32_t* scl = reinterpret_cast<uint32_t*>(smem_lds + NS * STAGE);
        scl_base = lds_addr(smem_lds + NS * STAGE);
        const int64_t g0 = k_begin >> 7;
        const int64_t wrow = (int64_t)(n0 >> 7) * p.kgroups + g0;
        const int elems = (chunk >> 7) * AR;
        for (int e0 = 0; e0 < elems; e0 += 8 * NW * 64) {
            uint32_t v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int e = e0 + (int)threadIdx.x + i * NW * 64;
                v[i] = 0u;
                if (e < elems) {
                    const int g = e / AR, t = min(e - g * AR, M - 1);
                    const int64_t ai = (int64_t)t * p.kgroups + g0 + g;
                    if constexpr (E8M0)
                        v[i] = (uint32_t)reinterpret_cast<const uint8_t*>(p.a_scale)[ai] |
                               ((uint32_t)reinterpret_cast<const uint8_t*>(p.w_scale)[wrow + g] << 8);
                    else
                        v[i] = __float_as_uint(reinterpret_cast<const float*>(p.a_scale)[ai] *
                                               reinterpret_cast<const float*>(p.w_scale)[wrow + g]);
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int e = e0 + (int)threadIdx.x + i * NW * 64;
                if (e < elems) scl[e] = v[i];
            }
        }
        // the stage waits below count vector-memory loads only: finish these
        // LDS writes before the first barrier publishes them
        __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
    }
    // LDS byte offset of the scale word(s) of this lane's accumulator rows in
    // token slot MTI for chunk group GL.
#define QBG_S_OFF(MTI, GL) \
    (scl_base + 4u * (uint32_t)((GL) * AR + (SC128 ? min(16 * (MTI) + 4 * g4, AR - 4) \
                                                     : min(16 * (MTI) + r16, AR - 1))))

    const int astride = LOCAL ? RS : RB;
    for (int t = 0; t < T; ++t) {
        // Stage t + NS - 1 goes into the slot stage t - 1 held.  It is issued as
        // soon as every wave has finished reading that slot (the first barrier),
        // before the wait for stage t, so NS stages are in flight while stage t
        // lands; the second barrier makes stage t visible to every wave.
        if (t > 0) {
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        }
        if (t + NS - 1 < T) QBG_ISSUE(t + NS - 1)
        // (fused: the first stages' activation rows were issued last, so the
        // first wait takes everything)
        wait_stages<LPW, NS + 1>(FUSE && t == 0 ? 0 : min(NS - 1, T - 1 - t));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        const uint32_t base = lds_addr(smem_lds + (t % NS) * STAGE);
        const uint32_t abase = LOCAL ? lds_addr(act) + (uint32_t)(QBG_KSTAGE(t) * RB) : base + TN * RB;
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int s = wk + i * WKW;
            const int gk = (QBG_KSTAGE(t) * SK + s) * 128;  // byte offset of the step in the chunk
            if (gk >= chunk) continue;
            const int c = s * 8 + g4;
            const int gl = gk >> 7;  // 128-group of the step within the chunk
            uint4 wl[NTW], wh[NTW], al[MTW], ah[MTW];
            uint4 sc4[MTW];     // SC128: scale words of this lane's four accumulator rows
            uint32_t scw[MTW];  // other block ops: the scale word of this lane's operand row
            if constexpr (BATCHED) {
                uint32_t wa[NTW], wb[NTW], aa[MTW], ab[MTW];
#pragma unroll
                for (int j = 0; j < NTW; ++j) {
                    wa[j] = base + QBG_W_OFF(j, c);
                    wb[j] = base + QBG_W_OFF(j, c + 4);
                }
#pragma unroll
                for (int mt = 0; mt < MTW; ++mt) {
                    aa[mt] = QBG_A_ADDR(mt0 + mt, c);
                    ab[mt] = QBG_A_ADDR(mt0 + mt, c + 4);
                }
                lds_read_pairs<NTW>(wa, wb, wl, wh);
                lds_read_pairs<MTW>(aa, ab, al, ah);
                if constexpr (BLOCK) {  // (block ops run with one wave along M: mt0 == 0)
#pragma unroll
                    for (int mt = 0; mt < MTW; ++mt) {
                        if constexpr (SC128) lds_read1(QBG_S_OFF(mt0 + mt, gl), sc4[mt]);
                        else lds_read1w(QBG_S_OFF(mt0 + mt, gl), scw[mt]);
                    }
                }
            } else if constexpr (!BLOCK && NTW + MTW >= 3 && NTW + MTW <= 4) {
                // every operand chunk of the step in one batch of reads and one wait
                constexpr int NR = 2 * (NTW + MTW);
                uint32_t ra[NR];
                uint4 rx[NR];
#pragma unroll
                for (int j = 0; j < NTW; ++j) {
                    ra[2 * j] = base + QBG_W_OFF(j, c);
                    ra[2 * j + 1] = base + QBG_W_OFF(j, c + 4);
                }
#pragma unroll
                for (int mt = 0; mt < MTW; ++mt) {
                    ra[2 * NTW + 2 * mt] = QBG_A_ADDR(mt0 + mt, c);
                    ra[2 * NTW + 2 * mt + 1] = QBG_A_ADDR(mt0 + mt, c + 4);
                }
                if constexpr (NR == 6) lds_read6(ra, rx);
                else lds_read8(ra, rx);
#pragma unroll
                for (int j = 0; j < NTW; ++j) {
                    wl[j] = rx[2 * j];
                    wh[j] = rx[2 * j + 1];
                }
#pragma unroll
                for (int mt = 0; mt < MTW; ++mt) {
                    al[mt] = rx[2 * NTW + 2 * mt];
                    ah[mt] = rx[2 * NTW + 2 * mt + 1];
                }
            } else if constexpr (NTW == 1 && MTW == 1) {
                if constexpr (SC128)
                    lds_read5(base + QBG_W_OFF(0, c), base + QBG_W_OFF(0, c + 4),
                              QBG_A_ADDR(0, c), QBG_A_ADDR(0, c + 4),
                              QBG_S_OFF(0, gl), wl[0], wh[0], al[0], ah[0], sc4[0]);
                else if constexpr (BLOCK)
                    lds_read4w(base + QBG_W_OFF(0, c), base + QBG_W_OFF(0, c + 4),
                               QBG_A_ADDR(0, c), QBG_A_ADDR(0, c + 4),
                               QBG_S_OFF(0, gl), wl[0], wh[0], al[0], ah[0], scw[0]);
                else
                    lds_read4(base + QBG_W_OFF(0, c), base + QBG_W_OFF(0, c + 4),
                              QBG_A_ADDR(0, c), QBG_A_ADDR(0, c + 4), wl[0], wh[0],
                              al[0], ah[0]);
            } else {
#pragma unroll
                for (int j = 0; j < NTW; ++j)
                    lds_read2(base + QBG_W_OFF(j, c), base + QBG_W_OFF(j, c + 4), wl[j], wh[j]);
#pragma unroll
                for (int mt = 0; mt < MTW; ++mt)
                    lds_read2(QBG_A_ADDR(mt, c), QBG_A_ADDR(mt, c + 4), al[mt], ah[mt]);
                if constexpr (BLOCK) {
#pragma unroll
                    for (int mt = 0; mt < MTW; ++mt) {
                        if constexpr (SC128) lds_read1(QBG_S_OFF(mt, gl), sc4[mt]);
                        else lds_read1w(QBG_S_OFF(mt, gl), scw[mt]);
                    }
                }
            }
            if (gk + 128 > chunk) {  // partial step at the end of the chunk: zero the K
                                     // positions past it (integer masks keep the operands
                                     // in registers)
                const uint32_t lo_m = gk + g4 * 16 < chunk ? ~0u : 0u;
                const uint32_t hi_m = gk + 64 + g4 * 16 < chunk ? ~0u : 0u;
#pragma unroll
                for (int j = 0; j < NTW; ++j) {
                    wl[j] = and4(wl[j], lo_m);
                    wh[j] = and4(wh[j], hi_m);
                }
#pragma unroll
                for (int mt = 0; mt < MTW; ++mt) {
                    al[mt] = and4(al[mt], lo_m);
                    ah[mt] = and4(ah[mt], hi_m);
                }
            }
#pragma unroll
            for (int j = 0; j < NTW; ++j)
#pragma unroll
                for (int mt = 0; mt < MTW; ++mt) {
                    if constexpr (E8M0) {
                        const int ac = (int)(scw[mt] & 0xffu), wc = (int)((scw[mt] >> 8) & 0xffu);
                        acc[j][mt] = SWAP ? mma_step_e8m0(wl[j], wh[j], al[mt], ah[mt], acc[j][mt],
                                                          wc, ac)
                                          : mma_step_e8m0(al[mt], ah[mt], wl[j], wh[j], acc[j][mt],
                                                          ac, wc);
                    } else if constexpr (BLOCK) {
                        const AccV zero = {0, 0, 0, 0};
                        const AccV tmp = SWAP ? mma_step<OP>(wl[j], wh[j], al[mt], ah[mt], zero)
                                              : mma_step<OP>(al[mt], ah[mt], wl[j], wh[j], zero);
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const float f = __uint_as_float(SC128 ? u4_at(sc4[mt], v) : scw[mt]);
                            acc[j][mt][v] = __builtin_fmaf(tmp[v], f, acc[j][mt][v]);
                        }
                    } else {
                        acc[j][mt] = SWAP ? mma_step<OP>(wl[j], wh[j], al[mt], ah[mt], acc[j][mt])
                                          : mma_step<OP>(al[mt], ah[mt], wl[j], wh[j], acc[j][mt]);
                    }
                }
        }
    }
#undef QBG_S_OFF
    if constexpr (LOCAL) {
        // a_q and a_scale: the chunk's codes leave LDS once, 16 bytes per
        // thread and pass, spread over the workgroups of the K chunk.
        const int cu = chunk >> 4;  // 16-byte units of a row's range
        const int units = M * cu;
        for (int e = (int)(blockIdx.x * (NW * 64) + threadIdx.x); e < units;
             e += (int)(gridDim.x * (NW * 64))) {
            const int r = e / cu, col = e - r * cu;
            const uint4 v = *reinterpret_cast<const uint4*>(act + r * RS + ((col ^ (r & 15)) << 4));
            *reinterpret_cast<uint4*>(p.a_out + (int64_t)r * K + k_begin + col * 16) = v;
        }
        if (split == 0 && blockIdx.x == 0 && (int)threadIdx.x < M)
            p.a_scale_out[threadIdx.x] = l_sc[threadIdx.x];
        es.apply_a_lds(l_sc, M);
    }
    __syncthreads();  // every load has landed and every stage read is done: reuse LDS
    if constexpr (kRegEpi) {
        if (p.split_k == 1) {
            repi.finish(p, acc, n0, wn, wk, smem_lds);
            return;
        }
    }
    finish_tile<OP, SWAP, NTW, MTW, WNW, WKW, WMW, AR, RT>(p, reinterpret_cast<AccS*>(smem_lds), acc,
                                                      wn, wk, &s_last, es, 16 * mt0);
#undef QBG_ISSUE
#undef QBG_ISSUE_PART
#undef QBG_ISSUE_SLOT
#undef QBG_KSTAGE
#undef QBG_W_OFF
#undef QBG_A_ROW
#undef QBG_A_ADDR
}

// Large-M tiles (waves along M) take any number of tokens in one launch:
// grid.z runs over slices of AR tokens (split_k is 1 then; the split-K
// counters are per weight tile only).
template <int OP, bool SWAP, int AR, int NTW, int WNW, int WKW, int SK, int NS, int FM,
          int WMW, int RT = 0>
__global__ __launch_bounds__(64 * WNW * WKW * WMW) void gemm_lds_kernel(const GemmArgs p) {
    if constexpr (WMW > 1) {
        if (gridDim.z > 1) {
            GemmArgs q = p;
            const int m0 = (int)blockIdx.z * AR;
            q.M = min(AR, p.M - m0);
            q.a = p.a + (int64_t)m0 * p.K;
            q.a_scale = reinterpret_cast<const float*>(p.a_scale) + m0;
            q.out = reinterpret_cast<char*>(p.out) + (int64_t)m0 * p.N * (p.raw_i32 ? 4 : 2);
            gemm_lds_tile<OP, SWAP, AR, NTW, WNW, WKW, SK, NS, FM, WMW>(q, blockIdx.y);
            return;
        }
    }
    gemm_lds_tile<OP, SWAP, AR, NTW, WNW, WKW, SK, NS, FM, WMW, RT>(p, blockIdx.y);
}

// Grouped (mixture-of-experts) launch: grid.y runs over the experts.  Expert
// e owns the routed rows offsets[e] .. offsets[e+1]-1 (clamped to [0, M], so
// malformed offsets cannot address memory outside the tensors) and multiplies
// them with its weights w[e] [N,K] and scales w_scale[e] [N], AR rows at a time.
template <int OP, bool SWAP, int AR, int NTW, int WNW, int WKW, int SK, int NS>
__global__ __launch_bounds__(64 * WNW * WKW) void gemm_lds_grouped_kernel(const GemmArgs p) {
    const int e = blockIdx.y;
    const int total = p.rows;
    const int r0 = min(max(p.offsets[e], 0), total);
    const int r1 = min(max(p.offsets[e + 1], r0), total);
    GemmArgs q = p;
    q.w = p.w + (int64_t)e * p.N * p.K;
    q.w_scale = reinterpret_cast<const float*>(p.w_scale) + (int64_t)e * p.N;
    for (int s0 = r0; s0 < r1; s0 += AR) {
        q.M = min(AR, r1 - s0);
        q.a = p.a + (int64_t)s0 * p.K;
        q.a_scale = reinterpret_cast<const float*>(p.a_scale) + s0;
        q.out = reinterpret_cast<uint16_t*>(p.out) + (int64_t)s0 * p.N;
        gemm_lds_tile<OP, SWAP, AR, NTW, WNW, WKW, SK, NS, 0, 1>(q, 0);
        __syncthreads();  // the next slice reuses this tile's LDS
    }
}

#if QBG_PART(0)
__global__ void fill_zero_kernel(uint32_t* p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}
#endif

// Compiled tile variants.  Register-streaming kernel: {nt, wn, wk, ku, 0}.
constexpr TileShape kTiles[] = {
    {1, 1, 4, 2, 0},   // 0: 16 rows, 256 threads
    {1, 1, 8, 2, 0},   // 1: 16 rows, 512 threads
    {1, 1, 4, 4, 0},   // 2
    {1, 1, 8, 4, 0},   // 3
    {2, 1, 4, 2, 0},   // 4: 32 rows
    {2, 1, 8, 2, 0},   // 5
    {2, 1, 4, 4, 0},   // 6
    {1, 2, 4, 2, 0},   // 7: 32 rows, 512 threads
    {2, 2, 2, 4, 0},   // 8: 64 rows
    {2, 2, 4, 2, 0},   // 9: 64 rows, 512 threads
    {1, 4, 1, 4, 0},   // 10: 64 rows, no K split inside the workgroup
    {1, 1, 16, 1, 0},  // 11: 16 rows, 1024 threads
    // LDS-staged kernel: {ntw, wnw, wkw, sk (steps per stage), ns (stages)}
    {1, 4, 1, 2, 2},   // 12: 64 rows, 4 waves, 256-byte stages
    {1, 2, 2, 2, 3},   // 13: 32 rows
    {1, 2, 2, 2, 4},   // 14: 32 rows, 4 stages
    {1, 1, 4, 4, 2},   // 15: 16 rows, 512-byte stages
    {1, 1, 4, 4, 3},   // 16: 16 rows, 3 stages
    {2, 2, 1, 2, 2},   // 17: 64 rows, 2 waves
    {1, 1, 4, 8, 4},   // 18: 16 rows, 1 KB stage rows, 4 stages
    {1, 1, 4, 8, 3},   // 19: 16 rows, 1 KB stage rows, 3 stages
    {1, 2, 2, 8, 3},   // 20: 32 rows, 1 KB stage rows
    {1, 1, 2, 8, 4},   // 21: 16 rows, 2 waves, 1 KB stage rows
    // Large-M tiles (per-channel ops): {ntw, wnw, wkw, sk, ns, wmw, tokens per launch}.
    // Each wave holds ntw x (tokens / 16 / wmw) MFMA tiles of 16 x 16.
    {4, 2, 1, 2, 2, 2, 128},  // 22: 128 rows x 128 tokens, 64 KB stages
    {2, 2, 1, 2, 3, 2, 64},   // 23: 64 rows x 64 tokens
    {2, 1, 1, 2, 2, 4, 256},  // 24: 32 rows x 256 tokens, 72 KB stages
    {2, 2, 1, 2, 3, 2, 128},  // 25: 64 rows x 128 tokens, 48 KB stages
    {3, 2, 1, 2, 2, 2, 128},  // 26: 96 rows x 128 tokens (24576 rows = 256 workgroups)
    {3, 1, 1, 2, 2, 4, 256},  // 27: 48 rows x 256 tokens, 76 KB stages
    {2, 2, 1, 4, 2, 2, 64},   // 28: 64 rows x 64 tokens, 512-byte stage rows
    // Prefill tiles (FP8): {nt, wn, 1, 0, ns, wm, tokens, 1, K bytes per stage}:
    // 16*nt*wn weight rows x tokens, wm x wn waves of 32x32 matrix-core tiles.
    {4, 4, 1, 0, 2, 2, 256, 1, 128},  // 29: 256 rows x 256 tokens, 8 waves, 2 x 64 KB ring
    {8, 2, 1, 0, 2, 2, 256, 1, 128},  // 30: 256 rows x 256 tokens, 4 waves of 128 x 128
    {2, 4, 1, 0, 3, 2, 256, 1, 128},  // 31: 128 rows x 256 tokens, 3 stages
    {4, 4, 1, 0, 3, 2, 128, 1, 128},  // 32: 256 rows x 128 tokens, 3 stages
    {4, 2, 1, 0, 2, 2, 128, 1, 128},  // 33: 128 rows x 128 tokens, 4 waves, 66 KB (two per CU)
    // 64 tokens: mostly weight rows in each stage, for the token counts where
    // the weight stream still bounds the GEMM and bytes in flight set its speed
    {4, 4, 1, 0, 3, 2, 64, 1, 128},   // 34: 256 rows x 64 tokens, 8 waves, 3 x 40 KB ring
    {4, 2, 1, 0, 3, 2, 64, 1, 128},   // 35: 128 rows x 64 tokens, 4 waves, 74 KB (two per CU)
    // LDS-staged decode tiles with deeper rings ({ntw, wnw, wkw, sk, ns}): more weight
    // bytes in flight per CU next to 16-32 staged activation rows
    {1, 1, 4, 4, 6},   // 36: 16 rows, 512-byte stage rows, 6 stages
    {1, 1, 4, 8, 6},   // 37: 16 rows, 1 KB stage rows, 6 stages (up to 4 tokens)
    {2, 1, 4, 4, 4},   // 38: 32 rows (two sub-tiles per wave), 4 stages
    {1, 2, 2, 4, 4},   // 39: 32 rows, 2 x 2 waves, 4 stages
    {1, 4, 1, 2, 6},   // 40: 64 rows, 256-byte stage rows, 6 stages
    {4, 1, 4, 4, 3},   // 41: 64 rows (four sub-tiles per wave), 512-byte stage rows
    {3, 1, 4, 4, 3},   // 42: 48 rows (per-channel ops)
    {3, 2, 2, 2, 4},   // 43: 96 rows, 4 stages (per-channel ops)
    // eight waves (two per SIMD): one wave's conversions and products overlap
    // another's waits
    {1, 1, 8, 8, 3},   // 44: 16 rows, 1 KB stage rows, 3 stages
    {1, 2, 4, 4, 4},   // 45: 32 rows, 512-byte stage rows, 4 stages
    {2, 1, 8, 8, 3},   // 46: 32 rows (two sub-tiles per wave), 1 KB stage rows
    {1, 4, 2, 2, 4},   // 47: 64 rows, 256-byte stage rows, 4 stages
    {1, 1, 8, 8, 4},   // 48: 16 rows, 1 KB stage rows, 4 stages (up to 16 tokens)
    // 128 weight rows per workgroup: a quarter of the activation bytes per weight byte
    // that a 32-row tile streams at 32 tokens, where a launch still has enough
    // workgroups (N >= 32768)
    {2, 4, 1, 2, 3},   // 49: 128 rows, 4 waves of two sub-tiles, 256-byte stage rows
    {2, 4, 2, 2, 3},   // 50: 128 rows, 8 waves (K split in two)
    {1, 8, 1, 2, 3},   // 51: 128 rows, 8 waves of one sub-tile
    // Register kernel, per-channel ops: workgroups that own fewer rows than their
    // accumulators hold, so 6144 rows make 256 equal workgroups of 24 (with
    // 16-row tiles, 384 workgroups leave half the CUs with two and half with one)
    {1, 2, 4, 2, 0, 1, 0, 0, 64, 24},   // 52: 24 rows, two waves along N, 512 threads
    {2, 1, 8, 1, 0, 1, 0, 0, 64, 24},   // 53: 24 rows, two sub-tiles per wave, 512 threads
    {1, 2, 8, 1, 0, 1, 0, 0, 64, 24},   // 54: 24 rows, two waves along N, 1024 threads
    // one-launch (LOCAL) quantize + GEMM at up to 4 tokens: two load groups per wave
    {1, 1, 16, 3, 0},                   // 55: 16 rows, 1024 threads (K 12288)
    {2, 1, 16, 1, 0, 1, 0, 0, 64, 24},  // 56: 24 rows, 1024 threads (K 4096, 6144 rows)
    // An LDS-staged tile owning 24 of its 32 rows (plain per-channel ops): 6144 rows make
    // 256 workgroups where tile 45 makes 192 and tile 15 384
    {1, 2, 4, 4, 4, 1, 0, 0, 64, 24},   // 57: as tile 45
};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

// LDS of a prefill tile: the stage ring, then the tile's token and weight
// scales (fp32 each), or, Block-FP8 UE8M0, the tile's scale codes: one byte per
// (token row, group) and per (128-row weight block, group), K/128 groups.
constexpr size_t prefill_lds_bytes(const TileShape& t, int op = OP_FP8, int64_t K = 0) {
    const size_t bm = (size_t)t.tm, bn = (size_t)(16 * t.nt * t.wn);
    const size_t ring = (bm + bn) * (size_t)(t.ns * t.kb);
    if (op == OP_BLOCK_UE8M0) return ring + ((bm + bn / 128) * (size_t)(K / 128) + 15) / 16 * 16;
    if (op == OP_BLOCK_F32) return ring + (size_t)t.ns * t.wm * t.wn * 256;  // the group scales
    return ring + (bm + bn) * 4;
}

// Activation rows an LDS-staged tile stages (or, LOCAL, keeps resident) for
// M tokens: a large-M tile its token count; otherwise 4 when M <= 4 and the
// stage still splits evenly over the waves, else 16 or 32.  A LOCAL stage
// holds weight rows only.
constexpr int lds_rows_ok(const TileShape& t, int ar, bool local = false) {
    return ((16 * t.nt * t.wn + (local ? 0 : ar)) * 128 * t.ku) % (1024 * t.wn * t.wk * t.wm) == 0;
}
// -1 when no count of staged rows splits the stage into whole 1 KB loads per wave.
int lds_act_rows(const TileShape& t, int M, bool local = false) {
    if (t.tm > 0) return t.tm;
    if (M <= 4 && lds_rows_ok(t, 4, local)) return 4;
    if (M <= 16 && lds_rows_ok(t, 16, local)) return 16;
    return lds_rows_ok(t, 32, local) ? 32 : -1;
}
// LDS of an LDS-staged launch: the stage ring, then the block ops' scale
// words or the LOCAL mode's resident codes, amax partials, scales and bf16
// rows; at least the end-of-tile reduction's accumulators.
size_t lds_staged_bytes(const TileShape& t, int op, int ar, int M, int64_t K, int64_t k_chunk) {
    const size_t tn = 16 * t.nt * t.wn, rb = 128 * (size_t)t.ku;
    const bool local = op_is_local(op);
    const bool block = op == OP_BLOCK_F32 || op == OP_BLOCK_UE8M0;
    size_t bytes = (tn + (local ? 0 : ar)) * rb * t.ns;
    if (block) bytes += (size_t)(k_chunk / 128) * ar * 4;
    if (local) {
        const size_t stages = (size_t)((k_chunk + (int64_t)rb - 1) / (int64_t)rb);
        bytes += (size_t)ar * stages * rb + (size_t)ar * (t.wn * t.wk * t.wm + 1) * 4;
        bytes += (size_t)((2 * M * K + 1023) / 1024) * 1024;  // the bf16 rows
    }
    const size_t red = (size_t)t.wk * M * (tn + 1) * 4;
    return bytes > red ? bytes : red;
}
constexpr size_t kMaxLdsBytes = 160 * 1024;  // LDS of one CU

// Launch modes: plain GEMM, fused per-token quantization (published by
// producer workgroups), grouped (experts), fused with workgroup-local quantization.
enum LaunchMode { MODE_PLAIN = 0, MODE_FUSED = 1, MODE_GROUPED = 2, MODE_LOCAL = 3 };

template <int OP, bool SWAP, int MT, int AR, int KID, int MODE>
hipError_t launch_one(const GemmArgs& p, hipStream_t stream) {
    constexpr TileShape T = kTiles[KID];
    constexpr bool FUSE = MODE == MODE_FUSED;
    constexpr bool GROUPED = MODE == MODE_GROUPED;
    constexpr bool LOCAL = MODE == MODE_LOCAL;
    constexpr int FM = FUSE ? 1 : LOCAL ? 2 : 0;
    using AccS = typename Acc<OP>::scalar;
    const int tn = tile_n(T);  // weight rows per workgroup
    // a large-M tile without split-K covers all tokens in one launch (grid.z)
    const unsigned gz = (T.tm > 0 && p.split_k == 1) ? (unsigned)((p.M + AR - 1) / AR) : 1u;
    const dim3 grid((unsigned)((p.N + tn - 1) / tn), (unsigned)(GROUPED ? p.experts : p.split_k), gz);
    const dim3 block(64 * T.wn * T.wk * T.wm);
    constexpr bool kPerChannel = (OP == OP_FP8 || OP == OP_INT8);
    if constexpr (T.big > 0) {
        if constexpr ((MODE != MODE_PLAIN && !(GROUPED && kPerChannel)) ||
                      (OP != OP_FP8 && OP != OP_INT8 && OP != OP_BLOCK_UE8M0 && OP != OP_BLOCK_F32) ||
                      (OP == OP_BLOCK_F32 && (T.wm * T.wn <= T.tm / 64 || T.tm / T.wm > 64))) {
            return hipErrorInvalidValue;  // prefill tiles: plain and grouped per-channel GEMMs, Block-FP8
        } else {
            constexpr int BM = T.tm, BN = 16 * T.nt * T.wn;
            const size_t lds = prefill_lds_bytes(T, OP, p.K);
            if (lds > kMaxLdsBytes) return hipErrorInvalidConfiguration;
            const auto kern = gemm_prefill_kernel<OP, BM, BN, T.wm, T.wn, T.ns, T.kb, GROUPED>;
            static size_t raised = 0;
            if (lds > 65536 && lds > raised) {
                hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                                   (int)lds);
                if (e != hipSuccess) return e;
                raised = lds;
            }
            // grouped: the most token tiles the experts' row ranges can give
            const int64_t gm = GROUPED ? (int64_t)(p.rows + BM - 1) / BM + std::min(p.experts, p.rows)
                                       : (int64_t)(p.M + BM - 1) / BM;
            const int64_t tiles = gm * ((p.N + BN - 1) / BN) * p.split_k;  // x the K chunks
            if (tiles > 0x7fffffff) return hipErrorInvalidValue;
            const int64_t grid = (tiles + 7) / 8 * 8;  // whole rounds over the 8 XCDs
            hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * T.wm * T.wn), lds, stream, p);
            return hipGetLastError();
        }
    } else if constexpr (T.ns == 0 && (FUSE || GROUPED || (LOCAL && MT != 1))) {
        return hipErrorInvalidValue;  // PUBLISH and grouped launches: LDS-staged variants;
                                      // LOCAL on the register kernel: at most 16 tokens
    } else if constexpr (T.rows > 0 && (T.tm > 0 || !kPerChannel || (T.ns > 0 && MODE != MODE_PLAIN))) {
        return hipErrorInvalidValue;  // owned-row tiles: per-channel ops; LDS-staged ones plain only
    } else if constexpr (T.tm > 0 && (FUSE || GROUPED || LOCAL || !kPerChannel)) {
        return hipErrorInvalidValue;  // large-M tiles: plain per-channel GEMMs only
    } else if constexpr ((GROUPED || LOCAL) && !kPerChannel) {
        return hipErrorInvalidValue;  // grouped and LOCAL launches: per-channel GEMMs only
    } else if constexpr (!kPerChannel && T.ns > 0 && 128 % (16 * T.nt * T.wn) != 0) {
        return hipErrorInvalidValue;  // block ops: a tile's rows lie in one 128-row weight block
    } else if constexpr (T.ns == 0 && LOCAL) {
        // each wave owns exactly two load groups of the K chunk (checked on the host)
        if (p.k_chunk != 2 * 128 * T.wk * T.ku) return hipErrorInvalidValue;
        const size_t lds = gemm_lds_bytes(KID, OP == OP_INT8 ? OP_INT8_LOCAL : OP_FP8_LOCAL, p.M,
                                          p.K, p.k_chunk);
        if (lds > kMaxLdsBytes) return hipErrorInvalidConfiguration;
        const auto kern = gemm_kernel<OP, SWAP, T.nt, 1, T.wn, T.wk, T.ku, T.rows, true>;
        if (lds > 65536) {
            static size_t raised = 0;  // per instantiation: the largest size granted so far
            if (lds > raised) {
                hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                                   (int)lds);
                if (e != hipSuccess) return e;
                raised = lds;
            }
        }
        hipLaunchKernelGGL(kern, grid, block, lds, stream, p);
    } else if constexpr (T.ns == 0) {
        const size_t lds = (size_t)T.wk * p.M * (16 * T.nt * T.wn + 1) * sizeof(AccS);
        hipLaunchKernelGGL((gemm_kernel<OP, SWAP, T.nt, MT, T.wn, T.wk, T.ku, T.rows>), grid, block,
                           lds, stream, p);
    } else if constexpr (lds_rows_ok(T, AR, LOCAL)) {
        const int lop = LOCAL ? (OP == OP_INT8 ? OP_INT8_LOCAL : OP_FP8_LOCAL) : OP;
        const size_t lds = lds_staged_bytes(T, lop, AR, p.M < AR ? p.M : AR, p.K, p.k_chunk);
        if (lds > kMaxLdsBytes) return hipErrorInvalidConfiguration;
        auto kern = [] {
            if constexpr (GROUPED)
                return gemm_lds_grouped_kernel<OP, SWAP, AR, T.nt, T.wn, T.wk, T.ku, T.ns>;
            else
                return gemm_lds_kernel<OP, SWAP, AR, T.nt, T.wn, T.wk, T.ku, T.ns, FM, T.wm, T.rows>;
        }();
        if (lds > 65536) {
            static size_t raised = 0;  // per instantiation: the largest size granted so far
            if (lds > raised) {
                hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                                   (int)lds);
                if (e != hipSuccess) return e;
                raised = lds;
            }
        }
        hipLaunchKernelGGL(kern, grid, block, lds, stream, p);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int OP, bool SWAP, int MT, int MODE, int KID = 0>
hipError_t launch_kid(int kid, int ar, const GemmArgs& p, hipStream_t stream) {
    if constexpr (KID < kNumTiles) {
        if (kid == KID) {
            if constexpr (kTiles[KID].tm > 0) {
                return launch_one<OP, SWAP, 1, kTiles[KID].tm, KID, MODE>(p, stream);
            } else if constexpr (kTiles[KID].ns == 0) {
                return launch_one<OP, SWAP, MT, 16 * MT, KID, MODE>(p, stream);
            } else {
                if (ar == 4) return launch_one<OP, SWAP, 1, 4, KID, MODE>(p, stream);
                return launch_one<OP, SWAP, MT, 16 * MT, KID, MODE>(p, stream);
            }
        }
        return launch_kid<OP, SWAP, MT, MODE, KID + 1>(kid, ar, p, stream);
    } else {
        return hipErrorInvalidValue;
    }
}

template <int OP, int MODE = MODE_PLAIN>
hipError_t launch_op(const GemmArgs& p, int kid, int swap_ab, hipStream_t stream) {
    int mt = p.M <= 16 ? 1 : 2;
    const int ar = kTiles[kid].ns ? lds_act_rows(kTiles[kid], p.M, MODE == MODE_LOCAL) : 16 * mt;
    if (ar < 0) return hipErrorInvalidValue;
    if (kTiles[kid].ns && kTiles[kid].tm == 0) mt = ar > 16 ? 2 : 1;  // staged rows set the slots
    if (swap_ab)
        return mt == 1 ? launch_kid<OP, true, 1, MODE>(kid, ar, p, stream)
                       : launch_kid<OP, true, 2, MODE>(kid, ar, p, stream);
    return mt == 1 ? launch_kid<OP, false, 1, MODE>(kid, ar, p, stream)
                   : launch_kid<OP, false, 2, MODE>(kid, ar, p, stream);
}

}  // namespace

// One launcher per (op, mode) family, each in its own part.
hipError_t launch_gemm_fp8(const GemmArgs& p, int kid, int swap, hipStream_t s);
hipError_t launch_gemm_int8(const GemmArgs& p, int kid, int swap, hipStream_t s);
hipError_t launch_gemm_block_f32(const GemmArgs& p, int kid, int swap, hipStream_t s);
hipError_t launch_gemm_block_ue8m0(const GemmArgs& p, int kid, int swap, hipStream_t s);
hipError_t launch_gemm_fused(int op, const GemmArgs& p, int kid, int swap, hipStream_t s);
hipError_t launch_gemm_grouped(int op, const GemmArgs& p, int kid, int swap, hipStream_t s);
hipError_t launch_gemm_local_fp8(const GemmArgs& p, int kid, int swap, hipStream_t s);
hipError_t launch_gemm_local_int8(const GemmArgs& p, int kid, int swap, hipStream_t s);

#if QBG_PART(0)
hipError_t launch_gemm_fp8(const GemmArgs& p, int kid, int swap, hipStream_t s) {
    return launch_op<OP_FP8>(p, kid, swap, s);
}
#endif
#if QBG_PART(1)
hipError_t launch_gemm_int8(const GemmArgs& p, int kid, int swap, hipStream_t s) {
    return launch_op<OP_INT8>(p, kid, swap, s);
}
#endif
#if QBG_PART(2)
hipError_t launch_gemm_block_f32(const GemmArgs& p, int kid, int swap, hipStream_t s) {
    return launch_op<OP_BLOCK_F32>(p, kid, swap, s);
}
#endif
#if QBG_PART(3)
hipError_t launch_gemm_block_ue8m0(const GemmArgs& p, int kid, int swap, hipStream_t s) {
    return launch_op<OP_BLOCK_UE8M0>(p, kid, swap, s);
}
#endif
#if QBG_PART(4)
hipError_t launch_gemm_fused(int op, const GemmArgs& p, int kid, int swap, hipStream_t s) {
    return op == OP_FP8_FUSED ? launch_op<OP_FP8, MODE_FUSED>(p, kid, swap, s)
                              : launch_op<OP_INT8, MODE_FUSED>(p, kid, swap, s);
}
#endif
#if QBG_PART(5)
hipError_t launch_gemm_grouped(int op, const GemmArgs& p, int kid, int swap, hipStream_t s) {
    return op == OP_FP8_GROUPED ? launch_op<OP_FP8, MODE_GROUPED>(p, kid, swap, s)
                                : launch_op<OP_INT8, MODE_GROUPED>(p, kid, swap, s);
}
#endif
#if QBG_PART(6)
hipError_t launch_gemm_local_fp8(const GemmArgs& p, int kid, int swap, hipStream_t s) {
    return launch_op<OP_FP8, MODE_LOCAL>(p, kid, swap, s);
}
#endif
#if QBG_PART(7)
hipError_t launch_gemm_local_int8(const GemmArgs& p, int kid, int swap, hipStream_t s) {
    return launch_op<OP_INT8, MODE_LOCAL>(p, kid, swap, s);
}
#endif

#if QBG_PART(0)
int gemm_kernel_count() { return kNumTiles; }

TileShape gemm_tile(int kernel_id) {
    if (kernel_id < 0 || kernel_id >= kNumTiles) return TileShape{0, 0, 0, 0, 0};
    return kTiles[kernel_id];
}

bool gemm_kernel_supports(int kernel_id, int op) {
    if (kernel_id < 0 || kernel_id >= kNumTiles) return false;
    if (kTiles[kernel_id].big > 0) {
        const TileShape& t = kTiles[kernel_id];
        // fp32 blocks: a scale load per wave, and at most 64 token rows per wave (the
        // group sums and the wave's scales take registers of their own)
        return op == OP_FP8 || op == OP_INT8 || op_is_grouped(op) || op == OP_BLOCK_UE8M0 ||
               (op == OP_BLOCK_F32 && t.wm * t.wn > t.tm / 64 && t.tm / t.wm <= 64);
    }
    if (kTiles[kernel_id].tm > 0) return op == OP_FP8 || op == OP_INT8;
    if (kTiles[kernel_id].rows > 0)  // owned rows: per-channel ops (LOCAL on the register kernel)
        return op == OP_FP8 || op == OP_INT8 || (op_is_local(op) && kTiles[kernel_id].ns == 0);
    if (op_is_local(op)) return true;  // LDS-staged decode tiles and the register kernel
    if (op_is_fused(op) || op_is_grouped(op)) return kTiles[kernel_id].ns > 0;
    if ((op == OP_BLOCK_F32 || op == OP_BLOCK_UE8M0) && kTiles[kernel_id].ns > 0 &&
        128 % (16 * kTiles[kernel_id].nt * kTiles[kernel_id].wn) != 0)
        return false;  // block ops: a tile's rows lie in one 128-row weight block
    return op >= OP_FP8 && op <= OP_BLOCK_UE8M0;
}

size_t gemm_lds_bytes(int kernel_id, int op, int M, int64_t K, int64_t k_chunk) {
    if (kernel_id < 0 || kernel_id >= kNumTiles) return 0;
    const TileShape& t = kTiles[kernel_id];
    const int cap = tile_tokens(t);
    const int m = M < cap ? M : cap;
    const size_t tn = 16 * t.nt * t.wn;
    if (t.big > 0) return prefill_lds_bytes(t, op, K);
    if (t.ns == 0) {
        const size_t red = (size_t)t.wk * m * (tn + 1) * 4;
        if (!op_is_local(op)) return red;
        if (m > 16) return (size_t)-1;  // LOCAL on the register kernel: at most 16 tokens
        // the chunk's codes (whole 256-byte groups), amax partials, scales, bf16 rows
        const size_t rs = ((size_t)k_chunk + 255) / 256 * 256;
        const size_t loc = (size_t)m * rs + (size_t)m * t.wn * t.wk * 4 + ((size_t)m * 4 + 15) / 16 * 16 +
                           ((size_t)2 * m * K + 1023) / 1024 * 1024;
        return loc > red ? loc : red;
    }
    const int ar = lds_act_rows(t, m, op_is_local(op));
    if (ar < 0) return (size_t)-1;  // no feasible stage split: rejected like an LDS overflow
    return lds_staged_bytes(t, op, ar, m, K, k_chunk);
}

hipError_t launch_gemm(int op, const GemmArgs& args, int kernel_id, int swap_ab,
                       hipStream_t stream) {
    switch (op) {
        case OP_FP8: return launch_gemm_fp8(args, kernel_id, swap_ab, stream);
        case OP_INT8: return launch_gemm_int8(args, kernel_id, swap_ab, stream);
        case OP_BLOCK_F32: return launch_gemm_block_f32(args, kernel_id, swap_ab, stream);
        case OP_BLOCK_UE8M0: return launch_gemm_block_ue8m0(args, kernel_id, swap_ab, stream);
        case OP_FP8_FUSED:
        case OP_INT8_FUSED: return launch_gemm_fused(op, args, kernel_id, swap_ab, stream);
        case OP_FP8_GROUPED:
        case OP_INT8_GROUPED: return launch_gemm_grouped(op, args, kernel_id, swap_ab, stream);
        case OP_FP8_LOCAL: return launch_gemm_local_fp8(args, kernel_id, swap_ab, stream);
        case OP_INT8_LOCAL: return launch_gemm_local_int8(args, kernel_id, swap_ab, stream);
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
#endif

}  // namespace qbg
