// qbg_device.h -- device helpers shared by the gfx950 kernels: bf16 and
// E4M3/int8 conversions, wave and workgroup reductions.
//
// Numeric rules (as fixed in include/qbg.h): E4M3 is the OCP "FN" variant
// (bias 7, largest finite 448); conversions round to nearest even after a
// clamp to the format's range; bf16 outputs round to nearest even.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qbg {

constexpr int kWave = 64;
constexpr int kGroup = 128;  // activation group width = weight block edge = one MFMA K step

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Low and high bf16 halves of a 32-bit word.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even; a NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    return f != f ? 0x7FC0u : r;  // a select: no branch on the common path
}

// Clamp then convert two floats to E4M3 with the matrix-core conversion unit
// (round to nearest even); returns the two codes in the low 16 bits.
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
    a = fminf(fmaxf(a, -448.0f), 448.0f);
    b = fminf(fmaxf(b, -448.0f), 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// Four floats -> four E4M3 codes packed little-endian in a 32-bit word.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    return e4m3x2(a, b) | (e4m3x2(c, d) << 16);
}

// fp32 -> symmetric int8: round half to even, clamp to [-127, 127].
__device__ __forceinline__ uint32_t i8_byte(float v) {
    float r = __builtin_rintf(v);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (uint32_t)((int)r) & 0xFFu;
}

__device__ __forceinline__ uint32_t i8x4(float a, float b, float c, float d) {
    return i8_byte(a) | (i8_byte(b) << 8) | (i8_byte(c) << 16) | (i8_byte(d) << 24);
}

// The eight bf16 values of a 16-byte chunk as fp32.
__device__ __forceinline__ void unpack8(const uint4& c, float* v) {
    v[0] = bf16_lo(c.x); v[1] = bf16_hi(c.x);
    v[2] = bf16_lo(c.y); v[3] = bf16_hi(c.y);
    v[4] = bf16_lo(c.z); v[5] = bf16_hi(c.z);
    v[6] = bf16_lo(c.w); v[7] = bf16_hi(c.w);
}

// Loads chunks first + i * stride (i < CH) of a row of nchunks 16-byte chunks
// into c, every load issued before any is used; an index past the row reads
// the row's last chunk instead, which the caller masks (or, for a max,
// ignores: a repeated value leaves it unchanged).  Loads under a branch would
// each wait for the one before, one memory round trip per chunk.
template <int CH>
__device__ __forceinline__ void load_row_chunks(const uint4* row, int nchunks, int first,
                                                int stride, uint4 (&c)[CH]) {
#pragma unroll
    for (int i = 0; i < CH; ++i) c[i] = row[min(first + i * stride, nchunks - 1)];
}

// Quantize 8 fp32 values with scale s (IEEE division), clamped to the type's
// range; QT 0 = E4M3, 1 = int8.  Returns the 8 bytes.  Every per-token
// quantizer (standalone or fused into a GEMM launch) goes through this.
template <int QT>
__device__ __forceinline__ uint2 quant8(const float* v, float s) {
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = v[i] / s;
    uint2 r;
    if (QT == 0) {
        r.x = e4m3x4(t[0], t[1], t[2], t[3]);
        r.y = e4m3x4(t[4], t[5], t[6], t[7]);
    } else {
        r.x = i8x4(t[0], t[1], t[2], t[3]);
        r.y = i8x4(t[4], t[5], t[6], t[7]);
    }
    // a non-finite unit (NaN scale): the NaN code everywhere (int8 has none: 0),
    // chosen by a select so the common path takes no branch
    const bool bad = s != s;
    const uint32_t c = QT == 0 ? 0x7F7F7F7Fu : 0u;
    r.x = bad ? c : r.x;
    r.y = bad ? c : r.y;
    return r;
}

// The maximum of IEEE 754-2019 (gfx950: v_maximum3_f32), which propagates a
// NaN where fmaxf drops it: every amax and its reductions use it, so a unit
// holding a NaN ends with amax NaN and one holding an infinity with +inf.
__device__ __forceinline__ float max_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// |v| folded into a running amax.
__device__ __forceinline__ float amax_fold(float run, float v) { return max_nan(run, fabsf(v)); }

// The scale of a unit (a token row or a group) from its amax: amax / qmax
// (IEEE), 1 for an all-zero unit, and NaN for a unit holding a NaN or an
// infinity (amax NaN or +inf), whose codes are then all the NaN code (quant8).
// Inputs are finite in the contract; this rule makes a non-finite one visible
// (every output of that token becomes NaN) instead of encoding it as +-448.
template <int QT>
__device__ __forceinline__ float token_scale(float amax) {
    const float qmax = QT == 0 ? 448.0f : 127.0f;
    if (!(amax <= 3.40282347e38f)) return __uint_as_float(0x7FC00000u);
    return amax > 0.0f ? amax / qmax : 1.0f;
}

// Smallest power of two >= s (s > 0, finite) as a UE8M0 code, clamped to
// [0, 254]; a NaN scale (a non-finite unit) gives 0xFF, the format's NaN.
__device__ __forceinline__ uint32_t ue8m0_code(float s) {
    if (s != s) return 0xFFu;
    uint32_t u = __float_as_uint(s);
    int e = (int)((u >> 23) & 0xFF);
    uint32_t mant = u & 0x7FFFFFu;
    int code;
    if (e == 0) {
        // subnormal s = mant * 2^-149: smallest 2^p >= s
        int msb = 31 - __clz(mant);                  // s in [2^(msb-149), 2^(msb-148))
        code = (mant == (1u << msb)) ? msb - 149 + 127 : msb - 148 + 127;
    } else {
        code = (mant == 0) ? e : e + 1;              // exponent field already carries the bias
    }
    return (uint32_t)max(0, min(254, code));
}

__device__ __forceinline__ float ue8m0_value(uint32_t code) {
    // 2^(code-127); code 0 is 2^-127, a subnormal fp32
    return code == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(code << 23);
}

// Max over the wave and the workgroup: NaN-propagating (amax reductions).
// The wave's maximum with data-parallel-primitive (DPP) lane moves, which run
// on the vector ALU instead of the LDS crossbar a lane shuffle takes: pairs and
// quads of lanes (quad permutations), halves and whole rows of 16 lanes
// (mirrors), then the row maxima through lanes 15 and 31 (row broadcasts into
// the rows above), so lane 63 holds the maximum of all 64, which every lane
// then reads.  A maximum does not depend on the order it is taken in (NaN
// propagates either way), so this equals any other reduction order bit for bit.
// Lanes a step does not write keep their value (old operand = the value).
#define QBG_DPP_MAX_STEP(V, CTRL, ROWS)                                                    \
    V = max_nan(V, __int_as_float(__builtin_amdgcn_update_dpp(                             \
                       __float_as_int(V), __float_as_int(V), CTRL, ROWS, 0xF, false)))
__device__ __forceinline__ float wave_max(float v) {
    QBG_DPP_MAX_STEP(v, 0xB1, 0xF);   // quad_perm [1,0,3,2]: lane pairs
    QBG_DPP_MAX_STEP(v, 0x4E, 0xF);   // quad_perm [2,3,0,1]: quads
    QBG_DPP_MAX_STEP(v, 0x141, 0xF);  // row_half_mirror: halves of a row
    QBG_DPP_MAX_STEP(v, 0x140, 0xF);  // row_mirror: rows of 16
    QBG_DPP_MAX_STEP(v, 0x142, 0xA);  // row_bcast15: rows 1 and 3 take rows 0 and 2
    QBG_DPP_MAX_STEP(v, 0x143, 0xC);  // row_bcast31: rows 2 and 3 take rows 0-1
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
#undef QBG_DPP_MAX_STEP

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// Max over the whole workgroup (blockDim.x a multiple of 64, <= 1024).
// `red` is a workgroup-shared scratch of at least blockDim.x/64 floats.
__device__ __forceinline__ float block_max(float v, float* red) {
    v = wave_max(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < nw; ++i) r = max_nan(r, red[i]);
    return r;
}

// Sum over the workgroup in a fixed order (waves summed 0..nw-1).
__device__ __forceinline__ double block_sum(double v, double* red) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    double r = red[0];
    for (int i = 1; i < nw; ++i) r += red[i];
    return r;
}

}  // namespace qbg
