/*
 * qbg.h -- C ABI of the MI355X (gfx950) 8-bit scaled-matmul decode backend.
 *
 * The operations are those of an LLM decode step's quantized linear layers,
 * as named on the pages this library follows:
 *   - "PyTorch integra Helion en vLLM para acelerar inferencia FP8"
 *     (mechatronicstore.cl), sections "Patron de fusion del forward pass" and
 *     "Kernels Helion implementados": dynamic per-token FP8 quantization,
 *     per-token-group FP8 quantization, RMSNorm+quant and SiLU-and-mul+quant
 *     fusions, scaled_mm and scaled_mm_blockwise;
 *   - "Helion DSL added to vLLM to autotune linear inference backends"
 *     (signaltitans.com), sections "Unified GEMM Architecture" and "Hybrid
 *     Dispatch and Autotuning": one GEMM implementation for the FP8 Dynamic,
 *     W8A8 INT8 and Block FP8 formats, whose algorithmic variants are tunable
 *     parameters chosen per shape, for token counts up to 32;
 *   - "Helion nel backend vLLM: un solo GEMM, tuning per forma e guadagni fino
 *     al 10%" (ai-radar.it), paragraphs 2-4 and 7: Split-K (K spread over
 *     several workgroups, split_k a power of two up to 256), Swap-AB
 *     (A@B computed as (B^T @ A^T)^T), max_helion_size = 32, precomputed
 *     per-shape configurations with a default configuration.
 *
 * Numeric conventions (readings where the pages are silent):
 *   - FP8 is OCP E4M3 ("E4M3FN": bias 7, largest finite 448, no infinities);
 *     int8 is symmetric in [-127, 127]; UE8M0 byte e stands for 2^(e-127).
 *   - A quantizer computes amax = max|x| over its span, s = amax/qmax as an
 *     IEEE fp32 division (qmax 448 or 127; s = 1 when amax = 0), and
 *     q = encode(clamp(x/s, -qmax, qmax)) with x/s an IEEE fp32 division,
 *     rounding to nearest even and keeping the sign of values that round to 0.
 *     UE8M0 scales are the smallest power of two >= amax/448.
 *   - GEMM outputs are bf16, rounded to nearest even from the fp32 result.
 *   - Inputs are finite.  The pages define nothing for NaN or infinite values;
 *     a quantization span (token row, 1x128 group, 128x128 weight block) whose
 *     values hold one gets scale NaN (UE8M0: code 0xFF) and the NaN code for
 *     every element (E4M3 0x7F; int8 0), so the GEMM outputs of that token are
 *     NaN.
 *
 * Layouts: every tensor is dense and row-major.  Activations A [M,K], weights
 * W [N,K] (K contiguous, the usual linear-layer layout), outputs [M,N].
 * Per-token scales [M], per-channel scales [N], group scales [M,K/128], block
 * scales [ceil(N/128), K/128].  bf16 travels as 16-bit words, E4M3 and UE8M0
 * as bytes, scales as fp32 unless UE8M0.
 *
 * Ownership: the caller owns every buffer (device memory unless marked host),
 * including the split-K workspace; the library never allocates device memory.
 * The library owns its host-side configuration table and one static device
 * array per GPU, the scratch of qbg_scaled_mm_noalloc, which is part of its
 * code object and exists from load until the process ends.
 *
 * Errors: every call validates its arguments before touching the device and
 * returns a status; nothing aborts or throws across the ABI.  qbg_last_error()
 * returns a description of the last failure on the calling thread.
 *
 * Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 * stream).  Calls are asynchronous on that stream; they make no
 * synchronization, no allocation, no host<->device copy and no host read of
 * device data, so they can be captured in a HIP graph.  Calls that share a
 * workspace must not run concurrently.
 */
#ifndef QBG_H
#define QBG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QBG_ABI_VERSION 3

typedef enum {
    QBG_OK = 0,
    QBG_E_NULL = 1,      /* a required pointer is NULL */
    QBG_E_SHAPE = 2,     /* a size is out of range or inconsistent */
    QBG_E_ALIGN = 3,     /* a device pointer is not 16-byte aligned */
    QBG_E_QTYPE = 4,     /* unknown quantized type, scale format or op */
    QBG_E_SPLITK = 5,    /* split_k not a power of two <= 256, or infeasible for K */
    QBG_E_WORKSPACE = 6, /* workspace missing or too small */
    QBG_E_TABLE = 7,     /* configuration table missing, unreadable or malformed */
    QBG_E_HIP = 8,       /* the HIP runtime reported an error (see qbg_last_error) */
    QBG_E_CONFIG = 9     /* a forced configuration names no kernel of this op */
} qbg_status;

typedef enum { QBG_FP8_E4M3 = 0, QBG_INT8 = 1 } qbg_qtype;
typedef enum { QBG_SCALE_F32 = 0, QBG_SCALE_UE8M0 = 1 } qbg_scale_fmt;
typedef enum {
    QBG_OP_FP8 = 0,          /* per-token x per-channel FP8 scaled GEMM */
    QBG_OP_INT8 = 1,         /* per-token x per-channel int8 scaled GEMM */
    QBG_OP_BLOCK_FP8 = 2,    /* 1x128 x 128x128 block FP8, fp32 scales */
    QBG_OP_BLOCK_UE8M0 = 3,  /* 1x128 x 128x128 block FP8, UE8M0 scales */
    QBG_OP_FP8_FUSED = 4,    /* per-token FP8 quantization + FP8 GEMM in one launch */
    QBG_OP_INT8_FUSED = 5,   /* per-token int8 quantization + int8 GEMM in one launch */
    QBG_OP_FP8_GROUPED = 6,  /* FP8 GEMM over expert-grouped rows (mixture of experts) */
    QBG_OP_INT8_GROUPED = 7  /* int8 GEMM over expert-grouped rows */
} qbg_op;

/*
 * A GEMM configuration: the algorithmic variant (swap_ab, split_k) and the
 * tile variant (kernel_id) of the one kernel family.  On input only
 * kernel_id, swap_ab, split_k, rotate and fuse are read; lookups also fill the
 * tile fields.
 *   kernel_id  index of the compiled tile variant (see qbg_kernel_info)
 *   swap_ab    0: tokens in the matrix-core row slot, weight rows in the
 *                 column slot (Standard);
 *              1: weight rows in the row slot, tokens in the column slot,
 *                 result transposed in the epilogue (Swap-AB)
 *   split_k    1..256, a power of two: K is cut into split_k equal
 *              contiguous chunks reduced through the workspace (Split-K)
 *   tile_n     weight rows per workgroup           (filled by lookups); a
 *              multiple of 16, except on decode tiles of the per-channel ops
 *              that own fewer rows than their 16-row matrix-core sub-tiles hold
 *              (e.g. 24, so that 6144 rows make 256 equal workgroups); the
 *              LDS-staged ones of these run the plain GEMMs only
 *   waves_n    waves side by side along N          (filled by lookups)
 *   waves_k    waves splitting a chunk of K, or each LDS stage (filled by lookups)
 *   k_unroll   128-wide K steps per register load group, or per LDS stage;
 *              0 for the prefill tiles, whose LDS stages hold 128 of K
 *   stages     0: the weights stream straight into registers; > 0: depth of
 *              the LDS ring the weights and activations stream through (the
 *              fused ops run on these LDS-staged variants only)
 *   waves_m    waves side by side along the tokens     (filled by lookups)
 *   tile_m     tokens one workgroup covers: 32 for the decode tiles, 64-256
 *              for the large-M tiles (per-channel ops) and the prefill tiles.  A decode tile runs
 *              larger M as several launches; a large-M tile with split_k 1
 *              covers every token in one launch (a grid dimension over
 *              tile_m-token slices)                     (filled by lookups)
 *              The prefill tiles (k_unroll 0) run the plain FP8 and INT8
 *              ops and Block-FP8: UE8M0 scales (K a multiple of 512, the
 *              tile's scale codes staged in LDS; a_scale and w_scale 4-byte
 *              aligned) on every prefill tile, fp32 scales on those with at
 *              most 64 token rows per wave (tile_m / waves_m <= 64); Standard
 *              layout and K a multiple of 128; each workgroup computes
 *              tile_m tokens x tile_n weight rows, and one launch covers every
 *              token.  FP8, INT8 and Block-FP8 (and the fused ops'
 *              quantizer-then-GEMM form) take split_k up to 16 with K a
 *              multiple of 128 x split_k (each chunk whole scale groups);
 *              the workspace then holds every K chunk's whole output tiles
 *              (4-byte sums) and at most 16320 output tiles are allowed.
 *   rotate     input: 1 = workgroups start their K loop at different offsets
 *              and wrap around (spreads simultaneous reads of rows that lie a
 *              power-of-two stride apart over HBM channels; a no-op when K does
 *              not split into whole load groups), 0 = all start at the chunk's
 *              beginning.  The sum's order, not its terms, changes.
 *   fuse       input, read by qbg_quantize_scaled_mm only (0 elsewhere): how
 *              the per-token quantization reaches the GEMM, one of qbg_fuse_mode.
 */
typedef struct {
    int32_t kernel_id;
    int32_t swap_ab;
    int32_t split_k;
    int32_t tile_n;
    int32_t waves_n;
    int32_t waves_k;
    int32_t k_unroll;
    int32_t stages;
    int32_t rotate;
    int32_t waves_m;
    int32_t tile_m;
    int32_t fuse;
} qbg_gemm_config;

/*
 * How qbg_quantize_scaled_mm combines the quantizer with the GEMM (results
 * are identical in every mode; the configuration table picks the fastest per
 * shape).
 *   QBG_FUSE_PUBLISH   one launch: a few workgroups quantize the rows and
 *                      publish them through memory, the others wait for them
 *                      (LDS-staged tiles)
 *   QBG_FUSE_LOCAL     one launch: every workgroup reads the bf16 rows,
 *                      computes the per-token scales itself and keeps the codes
 *                      of its K chunk in LDS for the whole K loop; nothing is
 *                      exchanged between workgroups (LDS-staged decode tiles)
 *   QBG_FUSE_SEPARATE  two launches: the per-token quantizer, then the GEMM
 *                      (any tile variant of the plain op)
 */
typedef enum { QBG_FUSE_PUBLISH = 0, QBG_FUSE_LOCAL = 1, QBG_FUSE_SEPARATE = 2 } qbg_fuse_mode;

/* ---- library information ------------------------------------------------ */

/* QBG_ABI_VERSION of the built library. */
int qbg_abi_version(void);

/* Static English name of a status code (host string, never NULL). */
const char* qbg_status_str(qbg_status status);

/* Description of the last failure on the calling thread (host string, valid
 * until the next call on this thread; "" if none). */
const char* qbg_last_error(void);

/* ---- quantizers --------------------------------------------------------- */

/*
 * Dynamic per-token quantization ("dynamic_per_token_scaled_fp8_quant",
 * mechatronicstore.cl, "Kernels Helion implementados"; the int8 form is the
 * activation side of W8A8 INT8).  Each row of x gets its own scale.
 *   qtype  QBG_FP8_E4M3 (q bytes are E4M3 codes) or QBG_INT8 (q is int8)
 *   x      bf16 [M,K]               in
 *   q      [M,K], 1 byte each       out
 *   scale  fp32 [M]                 out
 * M >= 1, K >= 16, K % 16 == 0; x and q 16-byte aligned, scale 4-byte aligned.
 * Also serves as the per-output-channel weight quantizer (W viewed as [N,K]).
 */
qbg_status qbg_quantize_per_token(qbg_qtype qtype, const void* x, int64_t M, int64_t K,
                                  void* q, float* scale, void* stream);

/*
 * Per-token-group FP8 quantization ("per_token_group_fp8_quant",
 * mechatronicstore.cl, "Kernels Helion implementados"): 1 x group spans of a
 * row share a scale; UE8M0 scales are named in "Patron de fusion del forward
 * pass".
 *   x      bf16 [M,K]                         in
 *   q      E4M3 [M,K]                         out
 *   scale  [M, K/group]: fp32, or one UE8M0 byte each   out
 * group must be 128; K % 128 == 0.
 */
qbg_status qbg_quantize_per_token_group(const void* x, int64_t M, int64_t K, int32_t group,
                                        qbg_scale_fmt fmt, void* q, void* scale, void* stream);

/*
 * 128 x 128 block quantization of a weight matrix W [N,K] (bf16) into E4M3
 * codes and one scale per block, laid out [ceil(N/128), K/128] (the weight
 * side of Block FP8; an offline step, not part of the decode path).
 * K % 128 == 0, N % 16 == 0.
 */
qbg_status qbg_quantize_weight_block(const void* w, int64_t N, int64_t K, qbg_scale_fmt fmt,
                                     void* q, void* scale, void* stream);

/*
 * Fused RMSNorm + dynamic per-token FP8 quantization
 * ("rms_norm_dynamic_per_token_quant", mechatronicstore.cl, "Kernels Helion
 * implementados"; the norm+quant pair of "Patron de fusion del forward pass").
 * y = x / sqrt(mean(x^2) + eps) * w evaluated in fp64 and rounded once to
 * fp32, then quantized per row as qbg_quantize_per_token does.
 *   x bf16 [M,H], w bf16 [H]  in;  q E4M3 [M,H], scale fp32 [M]  out
 * H % 16 == 0, H <= 65536.
 */
qbg_status qbg_rms_norm_quantize_per_token(const void* x, const void* w, float eps, int64_t M,
                                           int64_t H, void* q, float* scale, void* stream);

/*
 * Fused SiLU-and-mul + dynamic per-token FP8 quantization in one launch
 * ("silu_and_mul_dynamic_per_token_quant", mechatronicstore.cl, "Kernels
 * Helion implementados").  gate_up [M, 2I] holds the gate in columns [0, I)
 * and the up projection in [I, 2I); y = silu(gate) * up evaluated in fp64
 * and rounded once to fp32, then quantized per row.
 *   gate_up bf16 [M,2I]  in;  q E4M3 [M,I], scale fp32 [M]  out
 * I % 16 == 0, I <= 65536.
 */
qbg_status qbg_silu_mul_quantize_per_token(const void* gate_up, int64_t M, int64_t I, void* q,
                                           float* scale, void* stream);

/*
 * Block-format fused producers ("rms_norm_per_block_quant" and
 * "silu_and_mul_per_block_quant", mechatronicstore.cl, "Kernels Helion
 * implementados"; group quantization with UE8M0 scales in front of a block
 * GEMM is named in "Patron de fusion del forward pass"): the values y of
 * qbg_rms_norm_quantize_per_token / qbg_silu_mul_quantize_per_token (fp64,
 * rounded once to fp32), quantized in 1 x group spans as
 * qbg_quantize_per_token_group quantizes bf16 values.  The outputs are the
 * activation operands of qbg_block_scaled_mm.
 *   x bf16 [M,H], w bf16 [H]   (RMSNorm)   or   gate_up bf16 [M,2I]   in
 *   q E4M3 [M,H] (or [M,I])                                        out
 *   scale [M, H/group]: fp32, or one UE8M0 byte each                out
 * group must be 128; H (I) a multiple of 128, at most 65536; eps >= 0.
 * x, w, gate_up and q 16-byte aligned, fp32 scales 4-byte aligned.
 */
qbg_status qbg_rms_norm_quantize_per_token_group(const void* x, const void* w, float eps,
                                                 int64_t M, int64_t H, int32_t group,
                                                 qbg_scale_fmt fmt, void* q, void* scale,
                                                 void* stream);
qbg_status qbg_silu_mul_quantize_per_token_group(const void* gate_up, int64_t M, int64_t I,
                                                 int32_t group, qbg_scale_fmt fmt, void* q,
                                                 void* scale, void* stream);

/*
 * Test hook: the device's fp32 -> E4M3 conversion used by every quantizer
 * (values are clamped to [-448, 448] first), applied elementwise to n floats.
 * in/out device arrays, 4- and 1-byte aligned; n >= 0.
 */
qbg_status qbg_convert_f32_to_e4m3(const float* in, uint8_t* out, int64_t n, void* stream);

/* ---- GEMMs -------------------------------------------------------------- */

/*
 * Per-token x per-channel scaled GEMM ("scaled_mm", mechatronicstore.cl,
 * "Kernels Helion implementados"; FP8 Dynamic and W8A8 INT8 of "Unified GEMM
 * Architecture", signaltitans.com):
 *   out[m,n] = bf16( a_scale[m] * w_scale[n] * sum_k a_q[m,k] * w_q[n,k] )
 * with fp32 accumulation for E4M3 and exact int32 accumulation for int8.
 *   qtype    QBG_FP8_E4M3 or QBG_INT8 (both operands)
 *   a_q      [M,K] in;  a_scale fp32 [M] in
 *   w_q      [N,K] in;  w_scale fp32 [N] in
 *   out      bf16 [M,N] out
 *   cfg      host pointer, or NULL to use the configuration table lookup
 *   workspace, workspace_bytes: device scratch for split_k > 1, at least
 *            qbg_workspace_size() bytes and 256-byte aligned.  Its first 64 KiB
 *            hold synchronization slots and per-tile arrival counters that must
 *            be zero before the first use (qbg_workspace_init); every call
 *            leaves them zero again, so one workspace serves calls of any shape,
 *            op and configuration in stream order.  May be NULL/0 when the
 *            configuration has split_k == 1.
 * 1 <= M <= 8192, N % 16 == 0, K % 16 == 0, K / split_k % 16 == 0.  Tokens
 * beyond one launch's tile_m run as further launches, except on a large-M
 * tile with split_k 1 and on a prefill tile, which cover every token in one
 * launch.
 * For int8, K <= 133144 keeps the int32 accumulator exact.
 */
qbg_status qbg_scaled_mm(qbg_qtype qtype, const void* a_q, const float* a_scale,
                         const void* w_q, const float* w_scale, int64_t M, int64_t N, int64_t K,
                         void* out, const qbg_gemm_config* cfg, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code being captured into a
 * HIP graph, serving loops or harnesses that forbid hipMalloc): qbg_scaled_mm
 * without a workspace argument.  Its split-K launches use a scratch array the
 * library holds in each GPU's memory (QBG_NOALLOC_SCRATCH_BYTES: a 64 KiB slot
 * region plus 16 MiB of partials), kept from the first call on that GPU until
 * the process ends; the call itself allocates nothing.  Arguments, results and
 * the configuration lookup are those of qbg_scaled_mm.  A call whose
 * configuration needs more scratch than that (qbg_workspace_size) returns
 * QBG_E_WORKSPACE before any HIP call.  All calls on one GPU share its
 * scratch: calls that overlap in time on one GPU (on different streams or
 * from different threads) race and must not be made.  The stream must belong
 * to the current device; device indexes above 63 return QBG_E_SHAPE.  The
 * first call on a GPU also enqueues a fill kernel on its stream that clears
 * the slot region.
 */
#define QBG_NOALLOC_SCRATCH_BYTES (65536 + (16 << 20))
qbg_status qbg_scaled_mm_noalloc(qbg_qtype qtype, const void* a_q, const float* a_scale,
                                 const void* w_q, const float* w_scale, int64_t M, int64_t N,
                                 int64_t K, void* out, const qbg_gemm_config* cfg, void* stream);

/*
 * Block-FP8 scaled GEMM ("scaled_mm_blockwise", mechatronicstore.cl, "Kernels
 * Helion implementados"; Block FP8 of "Unified GEMM Architecture"):
 *   out[m,n] = bf16( sum_g a_scale[m,g] * w_scale[n/128,g] *
 *                    sum_{k in group g} a_q[m,k] * w_q[n,k] )
 *   fmt      QBG_SCALE_F32 (fp32 scales) or QBG_SCALE_UE8M0 (byte scales)
 *   a_q      E4M3 [M,K]; a_scale [M, K/128]
 *   w_q      E4M3 [N,K]; w_scale [ceil(N/128), K/128]
 * K % 128 == 0 and (K / split_k) % 128 == 0; otherwise as qbg_scaled_mm.
 */
qbg_status qbg_block_scaled_mm(qbg_scale_fmt fmt, const void* a_q, const void* a_scale,
                               const void* w_q, const void* w_scale, int64_t M, int64_t N,
                               int64_t K, void* out, const qbg_gemm_config* cfg,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Dynamic per-token quantization followed by the per-channel scaled GEMM: the
 * quantize-then-scaled_mm pair in front of every FP8 Dynamic / W8A8 INT8
 * linear layer ("Patron de fusion del forward pass" and "Kernels Helion
 * implementados", mechatronicstore.cl).  The results are those of
 * qbg_quantize_per_token(qtype, x, M, K, a_q, a_scale) followed by
 * qbg_scaled_mm(qtype, a_q, a_scale, w_q, w_scale, ...): a_q and a_scale are
 * byte-identical and out is computed from the same codes.
 *   qtype    QBG_FP8_E4M3 or QBG_INT8
 *   x        bf16 [M,K]                 in (16-byte aligned)
 *   w_q      [N,K], w_scale fp32 [N]    in
 *   a_q      [M,K], a_scale fp32 [M]    out (the quantized activations)
 *   out      bf16 [M,N]                 out
 *   cfg      NULL = table lookup for QBG_OP_FP8_FUSED / QBG_OP_INT8_FUSED; a
 *            forced configuration's `fuse` picks the mode (qbg_fuse_mode):
 *            PUBLISH needs an LDS-staged kernel_id (stages > 0); LOCAL an
 *            LDS-staged one with tile_m 32, or a register-streaming one
 *            (stages 0) with K / split_k exactly 256 x waves_k x k_unroll
 *            bytes (two load groups per wave) and bf16 rows and codes that fit
 *            the CU's LDS (at most 16 tokens); SEPARATE takes any kernel_id of
 *            the plain op; else QBG_E_CONFIG
 *   workspace  at least qbg_workspace_size(QBG_OP_*_FUSED, ...) bytes (PUBLISH:
 *            always, 64 KiB or more; LOCAL and SEPARATE: only for split_k > 1),
 *            zeroed once, 256-byte aligned, as for qbg_scaled_mm.  Calls
 *            sharing a workspace must not overlap.
 * PUBLISH: the first min(M, tiles) workgroups quantize the rows and publish
 * them (write-through stores, then a count in the workspace); every workgroup
 * starts streaming its weights, waits for the count (a bounded wait, see
 * qbg_set_fused_wait_limit), then streams the quantized activations.  A
 * workgroup whose wait runs out quantizes the rows itself, so the launch
 * always completes with the same results.
 * LOCAL: every workgroup issues its first weight stages (register tiles: all
 * of its weight loads), reads the M bf16 rows, reduces each row's amax, and
 * writes the codes of its K chunk to LDS, where they stay for the whole K loop
 * (the stages then carry weights only); the workgroups of the first weight
 * tile also store a_q and a_scale.  The LDS holds tile_m (register tiles: M) x
 * (K / split_k) code bytes and the 2 x M x K bytes of bf16 rows, which bounds
 * K / split_k and M.
 * Shapes as qbg_scaled_mm (1 <= M <= 8192).
 */
qbg_status qbg_quantize_scaled_mm(qbg_qtype qtype, const void* x, const void* w_q,
                                  const float* w_scale, int64_t M, int64_t N, int64_t K, void* a_q,
                                  float* a_scale, void* out, const qbg_gemm_config* cfg,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Test hook: poll iterations (each about 0.2 us) of the fused launch's bounded
 * wait for published rows, process-wide; 0 makes every workgroup quantize the
 * rows itself, a negative value restores the default (4096).  Applies to
 * launches enqueued afterwards.  Returns the previous value.
 */
int32_t qbg_set_fused_wait_limit(int32_t iterations);

/*
 * Grouped per-channel scaled GEMM for mixture-of-experts layers.  The pages
 * name the extension of the method to MoE models as a target ("Helion nel
 * backend vLLM", ai-radar.it, paragraph 9) without defining it; this is the
 * plain grouped form: the routed activation rows arrive grouped by expert,
 * and rows offsets[e] .. offsets[e+1]-1 are multiplied with expert e's
 * weights and scales:
 *   out[m,n] = bf16( a_scale[m] * w_scale[e,n] * sum_k a_q[m,k] * w_q[e,n,k] )
 * Routing, the top-k gather and the weighted combination are not part of it.
 *   qtype    QBG_FP8_E4M3 or QBG_INT8
 *   a_q      [T,K]; a_scale fp32 [T]                in (rows grouped by expert)
 *   w_q      [E,N,K]; w_scale fp32 [E,N]            in
 *   offsets  int32 [E+1], device, non-decreasing, offsets[0] = 0, offsets[E] = T;
 *            values outside [0, T] are clamped (no access outside the tensors)
 *   out      bf16 [T,N]                             out
 *   cfg      NULL = table lookup for QBG_OP_*_GROUPED at next_pow2(T) (on a
 *            miss: the 64-token prefill tile when T >= 32 E, K % 128 == 0 and
 *            E <= 1024, else a decode tile); a forced
 *            kernel_id must name an LDS-staged decode tile (stages > 0,
 *            tile_m 32) or a prefill tile (k_unroll 0: swap_ab 0, K % 128 == 0,
 *            E <= 1024, else QBG_E_CONFIG); split_k must be 1.  A looked-up
 *            prefill tile with E > 1024 is replaced by the decode-tile default
 * 0 <= T <= 65536 (T = 0 does nothing), 1 <= E <= 65535, N % 16 == 0,
 * K % 16 == 0.  One launch.  Decode tiles: a workgroup per (weight-row tile,
 * expert), an expert with no rows costs one workgroup that exits at once.
 * Prefill tiles: the experts' token tiles form one list; a workgroup per
 * (token tile, weight-row tile) finds its expert by scanning the offsets on the
 * device, and the grid is sized for ceil(T / tile_m) + min(E, T) token tiles
 * (the most well-formed offsets give; with malformed ones tiles beyond that
 * count are not computed).
 */
qbg_status qbg_grouped_scaled_mm(qbg_qtype qtype, const void* a_q, const float* a_scale,
                                 const void* w_q, const float* w_scale, const int32_t* offsets,
                                 int64_t T, int64_t E, int64_t N, int64_t K, void* out,
                                 const qbg_gemm_config* cfg, void* stream);

/*
 * Test hook: the int8 GEMM's exact int32 accumulator, acc[m,n] =
 * sum_k a_q[m,k] * w_q[n,k], through the same kernels and variants as
 * qbg_scaled_mm with QBG_INT8.  acc int32 [M,N] out.
 */
qbg_status qbg_scaled_mm_i32(const void* a_q, const void* w_q, int64_t M, int64_t N, int64_t K,
                             int32_t* acc, const qbg_gemm_config* cfg, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ---- configurations ----------------------------------------------------- */

/*
 * Load a per-shape configuration table (host path) produced by the offline
 * tuner, replacing any table loaded before ("Helion nel backend vLLM",
 * ai-radar.it, paragraph 7: configurations tuned ahead of time per shape).
 * On failure the previous table stays in force and QBG_E_TABLE is returned.
 * Not thread-safe with respect to concurrent lookups or GEMM calls.
 *
 * Without this call the library loads a table by itself, once, before the
 * first lookup (qbg_config_lookup, qbg_config_table_size, or a GEMM call with
 * cfg == NULL): the file the environment variable QBG_CONFIG_TABLE names (set
 * to the empty string: no table), else configs/gfx950.txt in the directory
 * of the loaded libqbg.so, the table shipped with it.  If that file is
 * missing or malformed, lookups use the built-in defaults (QBG_LOG=1 prints
 * why).  A successful qbg_config_table_load before the first lookup
 * replaces the automatic load.
 *
 * Two more environment variables, read once on the first lookup, steer the
 * lookup (a malformed value is ignored and reported with QBG_LOG=1):
 *   QBG_MAX_TUNED_M=n   table entries serve token counts up to n; larger ones
 *                       get the built-in default (unset: every bucket);
 *   QBG_FORCE_CONFIG=kernel_id,swap_ab,split_k[,rotate[,fuse]]
 *                       every lookup returns that configuration (a debugging
 *                       override; a call it does not fit returns QBG_E_CONFIG).
 *
 * Format (text): the header line "qbg-config-table <version> gfx950", then
 * one entry per line; '#' starts a comment.  Entry fields by version:
 *   1: <op> <m_bucket> <N> <K> <kernel_id> <swap_ab> <split_k>
 *   2: as 1, then <rotate>
 *   3: as 2, then <fuse>   (the tuner writes version 3)
 * <op> is fp8, int8, block_fp8, block_ue8m0, fp8_fused, int8_fused,
 * fp8_grouped or int8_grouped; <m_bucket> a power of two (the token count
 * rounded up); every entry is validated as a configuration for its key.
 */
qbg_status qbg_config_table_load(const char* path);

/* Number of entries in the loaded table (0 if none; triggers the automatic load). */
int64_t qbg_config_table_size(void);

/*
 * Configuration used for (op, M, N, K): the table entry for the bucket
 * next_pow2(M) if there is one, else the built-in default for this shape.
 * out is a host pointer.  *from_table (host, may be NULL) is set to 1 when
 * the entry came from the table.
 */
qbg_status qbg_config_lookup(qbg_op op, int64_t M, int64_t N, int64_t K, qbg_gemm_config* out,
                             int32_t* from_table);

/* Workspace bytes needed by (op, M, N, K) under cfg (NULL = lookup). host out.
 * Also validates cfg for that call: an infeasible configuration (a tile
 * variant that does not serve the op, or that needs more LDS than a CU has at
 * this M and K chunk) returns QBG_E_CONFIG, an infeasible split_k
 * QBG_E_SPLITK.  The fused ops in PUBLISH mode always need at least the
 * 64 KiB slot region. */
qbg_status qbg_workspace_size(qbg_op op, int64_t M, int64_t N, int64_t K,
                              const qbg_gemm_config* cfg, size_t* bytes);

/* Zero-fill a workspace on the stream with a fill kernel (graph-safe). */
qbg_status qbg_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/* Number of compiled tile variants of the GEMM family. */
int32_t qbg_kernel_count(void);

/*
 * Tile fields of kernel_id (host out): tile_n, waves_n, waves_k, k_unroll,
 * stages, waves_m and tile_m are filled, the other fields are left as passed.
 */
qbg_status qbg_kernel_info(int32_t kernel_id, qbg_gemm_config* inout);

#ifdef __cplusplus
}
#endif

#endif /* QBG_H */
