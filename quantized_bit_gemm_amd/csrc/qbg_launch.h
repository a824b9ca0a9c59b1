// qbg_launch.h -- host-side launchers of the gfx950 kernels (internal to libqbg).
//
// The C ABI layer validates every argument before calling these; the
// launchers only compute grids and enqueue kernels on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qbg {

// ---- quantizers ---------------------------------------------------------------
hipError_t launch_quant_per_token(int qtype, const void* x, int64_t M, int64_t K, void* q,
                                  float* scale, hipStream_t stream);
hipError_t launch_quant_group(const void* x, int64_t M, int64_t K, int ue8m0, void* q,
                              void* scale, hipStream_t stream);
hipError_t launch_quant_weight_block(const void* w, int64_t N, int64_t K, int ue8m0, void* q,
                                     void* scale, hipStream_t stream);
// scale_mode 0: one fp32 scale per row; 1: fp32 scales per 1 x 128 group; 2: UE8M0 per group.
hipError_t launch_rms_norm_quant(const void* x, const void* w, float eps, int64_t M, int64_t H,
                                 int scale_mode, void* q, void* scale, hipStream_t stream);
hipError_t launch_silu_mul_quant(const void* gate_up, int64_t M, int64_t I, int scale_mode,
                                 void* q, void* scale, hipStream_t stream);
hipError_t launch_convert_e4m3(const float* in, uint8_t* out, int64_t n, hipStream_t stream);
// True if a row of `len` bf16 values fits the register-resident fused kernels.
bool rows_fit_registers(int64_t len);

// ---- GEMM family -----------------------------------------------------------
// OP_*_FUSED: per-token quantization of bf16 activations fused into the
// per-channel GEMM launch, published through memory by a few workgroups
// (LDS-staged tile variants only).
// OP_*_GROUPED: per-channel GEMM over expert-grouped rows (mixture of experts).
// OP_*_LOCAL (internal to the library): the fused launch in which every
// workgroup quantizes the rows itself and keeps its chunk's codes in LDS
// (LDS-staged decode tiles only).
enum GemmOp {
    OP_FP8 = 0, OP_INT8 = 1, OP_BLOCK_F32 = 2, OP_BLOCK_UE8M0 = 3,
    OP_FP8_FUSED = 4, OP_INT8_FUSED = 5, OP_FP8_GROUPED = 6, OP_INT8_GROUPED = 7,
    OP_FP8_LOCAL = 8, OP_INT8_LOCAL = 9
};
inline bool op_is_fused(int op) { return op == OP_FP8_FUSED || op == OP_INT8_FUSED; }
inline bool op_is_grouped(int op) { return op == OP_FP8_GROUPED || op == OP_INT8_GROUPED; }
inline bool op_is_local(int op) { return op == OP_FP8_LOCAL || op == OP_INT8_LOCAL; }

// Token count one launch of a decode tile covers (two 16-token MFMA slots);
// the large-M tiles cover their own `tm` tokens per launch.
constexpr int kMaxTokensPerLaunch = 32;

// The workspace starts with kSyncSlots 32-bit synchronization slots of the
// fused launch ([0] activation rows published, [1] workgroups past the wait),
// followed by the per-tile split-K arrival counters.  All are zero between calls.
constexpr int kSyncSlots = 64;

// Poll iterations of the fused launch's bounded wait before a workgroup
// quantizes the rows itself (each iteration sleeps about 0.2 us).
constexpr int kDefaultWaitLimit = 4096;

struct GemmArgs {
    const uint8_t* a;     // [M,K] 8-bit codes
    const void* a_scale;  // fp32 [M], or [M, K/128] fp32 / UE8M0
    const uint8_t* w;     // [N,K] 8-bit codes
    const void* w_scale;  // fp32 [N], or [ceil(N/128), K/128] fp32 / UE8M0
    void* out;            // bf16 [M,N], or int32 [M,N] when raw_i32
    void* partial;        // split-K partials [split_k, M, N] (4-byte elements)
    uint32_t* counters;   // split-K arrival counters [n_tiles]
    int M, N, K;
    int k_chunk;          // K / split_k
    int split_k;
    int raw_i32;          // int8 only: write the int32 accumulators instead of bf16
    int kgroups;          // K / 128 (row length of block scale arrays)
    int rotate;           // start workgroups at different K offsets (see qbg_gemm_config)
    // Fused quantization only: `a` and `a_scale` are written by the launch itself.
    const uint16_t* x;    // bf16 activations [M,K]
    uint8_t* a_out;       // LOCAL mode: a_q, written (the kernel reads its LDS copy)
    float* a_scale_out;   // LOCAL mode: a_scale, written
    uint32_t* sync;       // kSyncSlots synchronization slots (workspace head)
    int wait_limit;       // poll iterations before quantizing the rows locally
    // Grouped launch only: a [rows,K], out [rows,N], w [experts,N,K], w_scale [experts,N].
    const int32_t* offsets;  // [experts + 1] row offsets of the experts (device)
    int experts;
    int rows;                // routed rows in all (M holds min(rows, 32) for sizing)
};

struct TileShape {
    int nt;      // 16-row weight sub-tiles per wave
    int wn;      // waves along N
    int wk;      // waves splitting the K chunk (register kernel) or each LDS stage's steps
    int ku;      // register kernel: 128-wide K steps per load group; LDS kernel: steps per stage
    int ns;      // LDS pipeline depth in stages; 0 = register-streaming kernel
    int wm = 1;  // waves along M (large-M tiles)
    int tm = 0;  // tokens per workgroup of a large-M tile; 0 = decode tile (up to 32)
    int big = 0; // 1: prefill tile (32x32 matrix-core tiles, both operands staged; ku is 0)
    int kb = 64; // prefill tile: K bytes per LDS stage (64 or 128); K % kb == 0
    int rows = 0;  // register kernel, per-channel ops: weight rows a workgroup owns when
                   // fewer than its 16 * nt * wn accumulator rows; 0 = all of them
};

int gemm_kernel_count();
// True if the tile variant supports the op.
bool gemm_kernel_supports(int kernel_id, int op);
// LDS one launch of the tile variant needs for M tokens (M capped at one launch's
// tokens), rows of K bytes and a K chunk of k_chunk bytes (block ops stage the
// chunk's scales in LDS; LOCAL launches keep the chunk's codes and the bf16 rows).
size_t gemm_lds_bytes(int kernel_id, int op, int M, int64_t K, int64_t k_chunk);
// Dynamic LDS a launch may request: the CU's 160 KiB less room for the
// kernels' few static LDS variables.
constexpr size_t kMaxLdsPerWorkgroup = 160 * 1024 - 256;
TileShape gemm_tile(int kernel_id);
inline int tile_n(const TileShape& t) { return t.rows > 0 ? t.rows : 16 * t.nt * t.wn; }
inline int tile_tokens(const TileShape& t) { return t.tm > 0 ? t.tm : kMaxTokensPerLaunch; }

// Enqueue one launch of the family for M <= tile_tokens(tile) tokens.
hipError_t launch_gemm(int op, const GemmArgs& args, int kernel_id, int swap_ab,
                       hipStream_t stream);

// Zero-fill n bytes (n % 4 == 0, 4-byte aligned) with a kernel (graph-safe).
hipError_t launch_fill_zero(void* p, size_t n, hipStream_t stream);

}  // namespace qbg
