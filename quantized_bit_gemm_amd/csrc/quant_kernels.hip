// quant_kernels.hip -- activation quantizers and fused producers for gfx950.
//
// Operations ("PyTorch integra Helion en vLLM para acelerar inferencia FP8",
// mechatronicstore.cl, sections "Patron de fusion del forward pass" and
// "Kernels Helion implementados"): dynamic per-token FP8 (and int8)
// quantization, per-token-group FP8 quantization with fp32 or UE8M0 scales,
// RMSNorm + per-token FP8 quantization and SiLU-and-mul + per-token FP8
// quantization, each in one launch, and their block-format forms
// ("rms_norm_per_block_quant", "silu_and_mul_per_block_quant": the same
// values quantized in 1 x 128 groups with fp32 or UE8M0 scales).  A 128x128
// block weight quantizer serves the offline weight side of Block FP8.
//
// Design: these kernels move a few hundred KB at decode sizes and are bound
// by launch and memory latency, not bandwidth.  One workgroup owns one row
// (or one 128x128 block): every thread loads its 16-byte chunks once into
// registers, the amax is reduced across the workgroup, and the same registers
// are quantized and written back, so each input byte is read exactly once.
#include "qbg_device.h"
#include "qbg_launch.h"

namespace qbg {
namespace {

constexpr int kQuantThreads = 256;
constexpr int kMaxThreads = 1024;
constexpr int kChunk = 8;  // bf16 values per 16-byte chunk

// The activation quantizers' codes and scales (per token, per 1 x 128 group,
// and those of the fused producers) are written through to memory
// (system-scope stores): the GEMM that reads them next runs on every XCD, and
// with write-through stores no dirty line of them is left in this kernel's L2
// when it ends.  Measured in the FP8 decode step: 0.3 % faster than plain
// stores (four alternations); non-temporal stores were 3.4 % slower.
template <class T>
__device__ __forceinline__ void store_through(T* p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ uint64_t pack64(uint2 r) { return (uint64_t)r.x | ((uint64_t)r.y << 32); }

// ---------------------------------------------------------------------------
// Per-token quantization: grid = M rows, CH register chunks per thread.
// ---------------------------------------------------------------------------
template <int QT, int CH>
__global__ __launch_bounds__(kMaxThreads) void quant_per_token_kernel(
    const uint16_t* __restrict__ x, int64_t K, uint8_t* __restrict__ q, float* __restrict__ scale) {
    __shared__ float red[kMaxThreads / kWave];
    const int64_t m = blockIdx.x;
    const uint4* row = reinterpret_cast<const uint4*>(x + m * K);
    const int nchunks = (int)(K / kChunk);
    uint4 xc[CH];
    load_row_chunks<CH>(row, nchunks, threadIdx.x, blockDim.x, xc);
    float v[CH][8];
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        unpack8(xc[c], v[c]);  // a chunk past the row repeats the last one: same max
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = amax_fold(amax, v[c][i]);
    }
    amax = block_max(amax, red);
    const float s = token_scale<QT>(amax);
    if (threadIdx.x == 0) store_through(&scale[m], s);
    uint64_t* qrow = reinterpret_cast<uint64_t*>(q + m * K);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int idx = threadIdx.x + c * blockDim.x;
        if (idx < nchunks) store_through(&qrow[idx], pack64(quant8<QT>(v[c], s)));
    }
}

// Rows longer than the register-resident variants: two passes over the row
// (the second pass reads from cache).
template <int QT>
__global__ __launch_bounds__(kQuantThreads) void quant_per_token_long_kernel(
    const uint16_t* __restrict__ x, int64_t K, uint8_t* __restrict__ q, float* __restrict__ scale) {
    __shared__ float red[kQuantThreads / kWave];
    const int64_t m = blockIdx.x;
    const uint4* row = reinterpret_cast<const uint4*>(x + m * K);
    const int64_t nchunks = K / kChunk;
    float amax = 0.0f;
    for (int64_t idx = threadIdx.x; idx < nchunks; idx += kQuantThreads) {
        float v[8];
        unpack8(row[idx], v);
        for (int i = 0; i < 8; ++i) amax = amax_fold(amax, v[i]);
    }
    amax = block_max(amax, red);
    const float s = token_scale<QT>(amax);
    if (threadIdx.x == 0) store_through(&scale[m], s);
    uint64_t* qrow = reinterpret_cast<uint64_t*>(q + m * K);
    for (int64_t idx = threadIdx.x; idx < nchunks; idx += kQuantThreads) {
        float v[8];
        unpack8(row[idx], v);
        store_through(&qrow[idx], pack64(quant8<QT>(v, s)));
    }
}

// ---------------------------------------------------------------------------
// 1 x 128 group quantization: 16 lanes own one group (8 values each); a
// 256-thread workgroup covers 16 groups.  Groups are numbered row-major over
// [M, K/128], which is also the scale layout.
// ---------------------------------------------------------------------------
template <bool UE8M0>
__global__ __launch_bounds__(kQuantThreads) void quant_group_kernel(
    const uint16_t* __restrict__ x, int64_t total_groups, uint8_t* __restrict__ q,
    void* __restrict__ scale) {
    const int64_t gid = (int64_t)blockIdx.x * (kQuantThreads / 16) + (threadIdx.x >> 4);
    const int sub = threadIdx.x & 15;
    const bool live = gid < total_groups;
    float v[8];
    float amax = 0.0f;
    if (live) {
        const uint4* src = reinterpret_cast<const uint4*>(x + gid * kGroup);
        unpack8(src[sub], v);
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = amax_fold(amax, v[i]);
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) amax = max_nan(amax, __shfl_xor(amax, off, 16));
    if (!live) return;
    float s = token_scale<0>(amax);
    if (UE8M0) {
        const uint32_t code = ue8m0_code(s);
        if (code != 0xFFu) s = ue8m0_value(code);  // 0xFF: s stays NaN
        if (sub == 0) store_through(reinterpret_cast<uint8_t*>(scale) + gid, (uint8_t)code);
    } else {
        if (sub == 0) store_through(reinterpret_cast<float*>(scale) + gid, s);
    }
    store_through(reinterpret_cast<uint64_t*>(q + gid * kGroup) + sub, pack64(quant8<0>(v, s)));
}

// ---------------------------------------------------------------------------
// 128 x 128 weight block quantization: one workgroup per block; each thread
// holds 8 chunks (a block is 2048 chunks).  Rows past N are skipped.
// ---------------------------------------------------------------------------
template <bool UE8M0>
__global__ __launch_bounds__(kQuantThreads) void quant_weight_block_kernel(
    const uint16_t* __restrict__ w, int64_t N, int64_t K, uint8_t* __restrict__ q,
    void* __restrict__ scale) {
    __shared__ float red[kQuantThreads / kWave];
    const int64_t bn = blockIdx.y, bk = blockIdx.x, kb = K / kGroup;
    constexpr int CH = kGroup * kGroup / kChunk / kQuantThreads;  // 8
    float v[CH][8];
    bool ok[CH];
    uint4 wc[CH];
    float amax = 0.0f;
    // all loads first (rows past N read row N-1, masked below), then the max
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int idx = threadIdx.x + c * kQuantThreads;  // chunk within the block
        const int64_t r = bn * kGroup + idx / (kGroup / kChunk);
        const int64_t col = bk * kGroup + (idx % (kGroup / kChunk)) * kChunk;
        ok[c] = r < N;
        wc[c] = *reinterpret_cast<const uint4*>(w + (r < N ? r : N - 1) * K + col);
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        unpack8(wc[c], v[c]);
        if (ok[c]) {
#pragma unroll
            for (int i = 0; i < 8; ++i) amax = amax_fold(amax, v[c][i]);
        }
    }
    amax = block_max(amax, red);
    float s = token_scale<0>(amax);
    if (UE8M0) {
        const uint32_t code = ue8m0_code(s);
        if (code != 0xFFu) s = ue8m0_value(code);  // 0xFF: s stays NaN
        if (threadIdx.x == 0) reinterpret_cast<uint8_t*>(scale)[bn * kb + bk] = (uint8_t)code;
    } else {
        if (threadIdx.x == 0) reinterpret_cast<float*>(scale)[bn * kb + bk] = s;
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        if (!ok[c]) continue;
        const int idx = threadIdx.x + c * kQuantThreads;
        const int64_t r = bn * kGroup + idx / (kGroup / kChunk);
        const int64_t col = bk * kGroup + (idx % (kGroup / kChunk)) * kChunk;
        *reinterpret_cast<uint2*>(q + r * K + col) = quant8<0>(v[c], s);
    }
}

// ---------------------------------------------------------------------------
// Fused producers' last step: quantize the row values this thread holds in
// registers (chunk idx = threadIdx.x + c * blockDim.x, 8 values each) to E4M3.
// SM 0: one fp32 scale per row (per token); SM 1 / SM 2: one scale per
// 1 x 128 group, fp32 / UE8M0.  A group is 16 consecutive chunks, held by 16
// consecutive lanes (blockDim.x is a multiple of 64), so its amax is a
// 16-lane shuffle reduction.  `scale_row` points at the row's scales.
// ---------------------------------------------------------------------------
enum ScaleMode { SM_TOKEN = 0, SM_GROUP_F32 = 1, SM_GROUP_UE8M0 = 2 };

template <int SM, int CH>
__device__ __forceinline__ void quant_row_fp8(float (&v)[CH][8], int nchunks, float thread_amax,
                                              uint8_t* qrow, void* scale_row, float* red) {
    uint64_t* q2 = reinterpret_cast<uint64_t*>(qrow);
    if constexpr (SM == SM_TOKEN) {
        const float s = token_scale<0>(block_max(thread_amax, red));
        if (threadIdx.x == 0) store_through(reinterpret_cast<float*>(scale_row), s);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int idx = threadIdx.x + c * blockDim.x;
            if (idx < nchunks) store_through(&q2[idx], pack64(quant8<0>(v[c], s)));
        }
    } else {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int idx = threadIdx.x + c * blockDim.x;
            float a = 0.0f;
            if (idx < nchunks) {
#pragma unroll
                for (int i = 0; i < 8; ++i) a = amax_fold(a, v[c][i]);
            }
#pragma unroll
            for (int off = 8; off >= 1; off >>= 1) a = max_nan(a, __shfl_xor(a, off, 16));
            float s = token_scale<0>(a);
            uint32_t code = 0;
            if constexpr (SM == SM_GROUP_UE8M0) {
                code = ue8m0_code(s);
                if (code != 0xFFu) s = ue8m0_value(code);  // 0xFF: s stays NaN
            }
            if (idx < nchunks) {
                if ((idx & 15) == 0) {
                    if constexpr (SM == SM_GROUP_UE8M0)
                        store_through(reinterpret_cast<uint8_t*>(scale_row) + (idx >> 4), (uint8_t)code);
                    else
                        store_through(reinterpret_cast<float*>(scale_row) + (idx >> 4), s);
                }
                store_through(&q2[idx], pack64(quant8<0>(v[c], s)));
            }
        }
    }
}

// Scales of row m: [M] per token, or [M, len/128] per group (fp32 or bytes).
template <int SM>
__device__ __forceinline__ void* scale_row_ptr(void* scale, int64_t m, int64_t len) {
    if constexpr (SM == SM_TOKEN) return reinterpret_cast<float*>(scale) + m;
    if constexpr (SM == SM_GROUP_F32) return reinterpret_cast<float*>(scale) + m * (len / kGroup);
    return reinterpret_cast<uint8_t*>(scale) + m * (len / kGroup);
}

// ---------------------------------------------------------------------------
// Fused RMSNorm + per-token FP8: y = fl32((x * r) * w) with
// r = 1/sqrt(sum(x^2)/H + eps) in fp64, then the per-token (or group) quantizer on y.
// ---------------------------------------------------------------------------
template <int SM, int CH>
__global__ __launch_bounds__(kMaxThreads) void rms_norm_quant_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, float eps, int64_t H,
    uint8_t* __restrict__ q, void* __restrict__ scale) {
    __shared__ double dred[kMaxThreads / kWave];
    __shared__ float red[kMaxThreads / kWave];
    const int64_t m = blockIdx.x;
    const uint4* row = reinterpret_cast<const uint4*>(x + m * H);
    const uint4* wrow = reinterpret_cast<const uint4*>(w);
    const int nchunks = (int)(H / kChunk);
    // the row and the norm weights in one round trip
    uint4 xc[CH], wc[CH];
    load_row_chunks<CH>(row, nchunks, threadIdx.x, blockDim.x, xc);
    load_row_chunks<CH>(wrow, nchunks, threadIdx.x, blockDim.x, wc);
    float v[CH][8];
    double ss = 0.0;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int idx = threadIdx.x + c * blockDim.x;
        if (idx < nchunks) {
            unpack8(xc[c], v[c]);
#pragma unroll
            for (int i = 0; i < 8; ++i) ss += (double)v[c][i] * (double)v[c][i];
        }
    }
    ss = block_sum(ss, dred);
    const double r = 1.0 / sqrt(ss / (double)H + (double)eps);
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int idx = threadIdx.x + c * blockDim.x;
        if (idx < nchunks) {
            float wv[8];
            unpack8(wc[c], wv);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                v[c][i] = (float)(((double)v[c][i] * r) * (double)wv[i]);
                amax = amax_fold(amax, v[c][i]);
            }
        }
    }
    quant_row_fp8<SM, CH>(v, nchunks, amax, q + m * H, scale_row_ptr<SM>(scale, m, H), red);
}

// ---------------------------------------------------------------------------
// Fused SiLU-and-mul + per-token FP8: y = fl32((g / (1 + exp(-g))) * u) in fp64,
// g = gate_up[m, k], u = gate_up[m, I + k]; then the per-token (or group) quantizer on y.
// ---------------------------------------------------------------------------
template <int SM, int CH>
__global__ __launch_bounds__(kMaxThreads) void silu_mul_quant_kernel(
    const uint16_t* __restrict__ gu, int64_t I, uint8_t* __restrict__ q, void* __restrict__ scale) {
    __shared__ float red[kMaxThreads / kWave];
    const int64_t m = blockIdx.x;
    const uint4* grow = reinterpret_cast<const uint4*>(gu + m * 2 * I);
    const uint4* urow = reinterpret_cast<const uint4*>(gu + m * 2 * I + I);
    const int nchunks = (int)(I / kChunk);
    uint4 gc[CH], uc[CH];
    load_row_chunks<CH>(grow, nchunks, threadIdx.x, blockDim.x, gc);
    load_row_chunks<CH>(urow, nchunks, threadIdx.x, blockDim.x, uc);
    float v[CH][8];
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int idx = threadIdx.x + c * blockDim.x;
        if (idx < nchunks) {
            float g[8], u[8];
            unpack8(gc[c], g);
            unpack8(uc[c], u);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const double gd = (double)g[i];
                v[c][i] = (float)((gd / (1.0 + exp(-gd))) * (double)u[i]);
                amax = amax_fold(amax, v[c][i]);
            }
        }
    }
    quant_row_fp8<SM, CH>(v, nchunks, amax, q + m * I, scale_row_ptr<SM>(scale, m, I), red);
}

__global__ void convert_e4m3_kernel(const float* __restrict__ in, uint8_t* __restrict__ out,
                                    int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = (uint8_t)(e4m3x2(in[i], 0.0f) & 0xFFu);
}

// Launch shape for a row of `len` bf16 values held in registers: the thread
// count grows with the row (a multiple of 64, at most 1024) so that each thread
// converts at most CH chunks; CH = 0 if the row is too long for that.
struct RowShape {
    int threads, ch;
};
RowShape row_shape(int64_t len) {
    const int64_t chunks = (len + kChunk - 1) / kChunk;
    for (int ch : {2, 4, 8}) {
        int64_t t = (chunks + ch - 1) / ch;
        t = ((t + kWave - 1) / kWave) * kWave;
        if (t <= kMaxThreads) return RowShape{(int)(t < kWave ? kWave : t), ch};
    }
    return RowShape{kQuantThreads, 0};
}

}  // namespace

// ---- launchers (host) -------------------------------------------------------

hipError_t launch_quant_per_token(int qtype, const void* x, int64_t M, int64_t K, void* q,
                                  float* scale, hipStream_t stream) {
    const dim3 grid((unsigned)M);
    const uint16_t* xs = static_cast<const uint16_t*>(x);
    uint8_t* qs = static_cast<uint8_t*>(q);
    const RowShape rs = row_shape(K);
    const dim3 blk(rs.threads);
#define QBG_PT(QT)                                                                              \
    switch (rs.ch) {                                                                            \
        case 2: hipLaunchKernelGGL((quant_per_token_kernel<QT, 2>), grid, blk, 0, stream, xs, K, qs, scale); break; \
        case 4: hipLaunchKernelGGL((quant_per_token_kernel<QT, 4>), grid, blk, 0, stream, xs, K, qs, scale); break; \
        case 8: hipLaunchKernelGGL((quant_per_token_kernel<QT, 8>), grid, blk, 0, stream, xs, K, qs, scale); break; \
        default: hipLaunchKernelGGL((quant_per_token_long_kernel<QT>), grid, dim3(kQuantThreads), 0, stream, xs, K, qs, scale); break; \
    }
    if (qtype == 0) {
        QBG_PT(0)
    } else {
        QBG_PT(1)
    }
#undef QBG_PT
    return hipGetLastError();
}

hipError_t launch_quant_group(const void* x, int64_t M, int64_t K, int ue8m0, void* q, void* scale,
                              hipStream_t stream) {
    const int64_t total = M * (K / kGroup);
    const int per_block = kQuantThreads / 16;
    const dim3 grid((unsigned)((total + per_block - 1) / per_block));
    const uint16_t* xs = static_cast<const uint16_t*>(x);
    uint8_t* qs = static_cast<uint8_t*>(q);
    if (ue8m0)
        hipLaunchKernelGGL((quant_group_kernel<true>), grid, dim3(kQuantThreads), 0, stream, xs, total, qs, scale);
    else
        hipLaunchKernelGGL((quant_group_kernel<false>), grid, dim3(kQuantThreads), 0, stream, xs, total, qs, scale);
    return hipGetLastError();
}

hipError_t launch_quant_weight_block(const void* w, int64_t N, int64_t K, int ue8m0, void* q,
                                     void* scale, hipStream_t stream) {
    const dim3 grid((unsigned)(K / kGroup), (unsigned)((N + kGroup - 1) / kGroup));
    const uint16_t* ws = static_cast<const uint16_t*>(w);
    uint8_t* qs = static_cast<uint8_t*>(q);
    if (ue8m0)
        hipLaunchKernelGGL((quant_weight_block_kernel<true>), grid, dim3(kQuantThreads), 0, stream, ws, N, K, qs, scale);
    else
        hipLaunchKernelGGL((quant_weight_block_kernel<false>), grid, dim3(kQuantThreads), 0, stream, ws, N, K, qs, scale);
    return hipGetLastError();
}

bool rows_fit_registers(int64_t len) { return row_shape(len).ch != 0; }

hipError_t launch_rms_norm_quant(const void* x, const void* w, float eps, int64_t M, int64_t H,
                                 int scale_mode, void* q, void* scale, hipStream_t stream) {
    const dim3 grid((unsigned)M);
    const uint16_t* xs = static_cast<const uint16_t*>(x);
    const uint16_t* wsp = static_cast<const uint16_t*>(w);
    uint8_t* qs = static_cast<uint8_t*>(q);
    const RowShape rs = row_shape(H);
    const dim3 blk(rs.threads);
#define QBG_RMS(SM)                                                                                 \
    switch (rs.ch) {                                                                                \
        case 2: hipLaunchKernelGGL((rms_norm_quant_kernel<SM, 2>), grid, blk, 0, stream, xs, wsp, eps, H, qs, scale); break; \
        case 4: hipLaunchKernelGGL((rms_norm_quant_kernel<SM, 4>), grid, blk, 0, stream, xs, wsp, eps, H, qs, scale); break; \
        case 8: hipLaunchKernelGGL((rms_norm_quant_kernel<SM, 8>), grid, blk, 0, stream, xs, wsp, eps, H, qs, scale); break; \
        default: return hipErrorInvalidValue;                                                       \
    }
    switch (scale_mode) {
        case SM_TOKEN: QBG_RMS(SM_TOKEN) break;
        case SM_GROUP_F32: QBG_RMS(SM_GROUP_F32) break;
        case SM_GROUP_UE8M0: QBG_RMS(SM_GROUP_UE8M0) break;
        default: return hipErrorInvalidValue;
    }
#undef QBG_RMS
    return hipGetLastError();
}

hipError_t launch_silu_mul_quant(const void* gate_up, int64_t M, int64_t I, int scale_mode, void* q,
                                 void* scale, hipStream_t stream) {
    const dim3 grid((unsigned)M);
    const uint16_t* g = static_cast<const uint16_t*>(gate_up);
    uint8_t* qs = static_cast<uint8_t*>(q);
    const RowShape rs = row_shape(I);
    const dim3 blk(rs.threads);
#define QBG_SILU(SM)                                                                                \
    switch (rs.ch) {                                                                                \
        case 2: hipLaunchKernelGGL((silu_mul_quant_kernel<SM, 2>), grid, blk, 0, stream, g, I, qs, scale); break; \
        case 4: hipLaunchKernelGGL((silu_mul_quant_kernel<SM, 4>), grid, blk, 0, stream, g, I, qs, scale); break; \
        case 8: hipLaunchKernelGGL((silu_mul_quant_kernel<SM, 8>), grid, blk, 0, stream, g, I, qs, scale); break; \
        default: return hipErrorInvalidValue;                                                       \
    }
    switch (scale_mode) {
        case SM_TOKEN: QBG_SILU(SM_TOKEN) break;
        case SM_GROUP_F32: QBG_SILU(SM_GROUP_F32) break;
        case SM_GROUP_UE8M0: QBG_SILU(SM_GROUP_UE8M0) break;
        default: return hipErrorInvalidValue;
    }
#undef QBG_SILU
    return hipGetLastError();
}

hipError_t launch_convert_e4m3(const float* in, uint8_t* out, int64_t n, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const dim3 grid((unsigned)((n + 255) / 256));
    hipLaunchKernelGGL(convert_e4m3_kernel, grid, dim3(256), 0, stream, in, out, n);
    return hipGetLastError();
}

}  // namespace qbg
