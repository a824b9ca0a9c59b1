/*
 * oracle.c -- plain CPU oracle for the 8-bit scaled-matmul decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test-suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no source, header, table or helper with
 * the HIP library.
 *
 * What it follows.  The pages ("PyTorch integra Helion en vLLM para acelerar
 * inferencia FP8", mechatronicstore.cl, sections "Patron de fusion del forward
 * pass" and "Kernels Helion implementados"; "Helion nel backend vLLM: un solo
 * GEMM, tuning per forma e guadagni fino al 10%", ai-radar.it, paragraphs 1-3;
 * "Helion DSL added to vLLM to autotune linear inference backends",
 * signaltitans.com, section "Unified GEMM Architecture") name the operations
 * -- dynamic per-token FP8 quantization, per-token-group FP8 quantization,
 * fused RMSNorm+quant and SiLU-and-mul+quant, the FP8-dynamic, W8A8-INT8 and
 * Block-FP8 scaled GEMMs, and the Split-K and Swap-AB variants -- but define
 * none of their arithmetic.  The arithmetic below is the plainest reading
 * that the rest supports; every reading is marked READING.
 *
 * Style.  Plain loops, fp64 (or int64) accumulation, no blocking or fusion.
 * OpenMP is used only across independent output rows.  Codecs are written
 * from the format definitions:
 *   - E4M3 ("FN" variant of the OCP 8-bit floating-point formats): sign,
 *     4 exponent bits with bias 7, 3 mantissa bits, subnormals at exponent 0,
 *     no infinities, 0x7F/0xFF are NaN, largest finite 448 (0x7E).
 *   - UE8M0: an unsigned 8-bit exponent, byte e encodes 2^(e-127).
 *   - BF16: the top 16 bits of an IEEE binary32 (8 significant bits).
 *
 * Compile: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC.
 * Floating point here is IEEE: fp32 operations on float operands are
 * correctly rounded binary32 operations (x86-64 SSE, FLT_EVAL_METHOD 0).
 *
 * Conventions.  bf16 tensors travel as uint16 bit patterns, e4m3 as uint8
 * codes, int8 as int8.  All matrices are dense and row-major: activations
 * [M,K], weights [N,K] (K contiguous), outputs [M,N].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_FP8 0
#define ORC_INT8 1
#define ORC_SCALE_F32 0
#define ORC_SCALE_UE8M0 1
#define ORC_GROUP 128 /* activation group width and weight block edge */

/* ------------------------------------------------------------------------ */
/* Codecs                                                                    */
/* ------------------------------------------------------------------------ */

/* Value of an E4M3 code, from the format definition. NaN codes give NaN. */
double orc_e4m3_decode(uint8_t c)
{
    int sign = c >> 7;
    int e = (c >> 3) & 15;
    int m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);          /* subnormal: 2^-6 * m/8 */
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7); /* normal */
    return sign ? -v : v;
}

/*
 * E4M3 code nearest to x, ties to the even code (the code whose mantissa's
 * last bit is 0; codes are ordered like their magnitudes, so "even code" and
 * "even significand" coincide).  READING: the caller has already clamped x to
 * [-448, 448] (a saturating conversion); the sign is kept, so a negative value
 * that rounds to zero encodes as 0x80.
 * The search is a plain nearest-neighbour search over the 127 non-negative
 * finite magnitudes 0x00..0x7E, which are strictly increasing.
 */
uint8_t orc_e4m3_encode(float x)
{
    double a = fabs((double)x);
    int lo = 0, hi = 126;
    while (lo < hi) { /* largest code whose magnitude is <= a */
        int mid = (lo + hi + 1) / 2;
        if (orc_e4m3_decode((uint8_t)mid) <= a)
            lo = mid;
        else
            hi = mid - 1;
    }
    int c = lo;
    if (c < 126) {
        double below = a - orc_e4m3_decode((uint8_t)c);
        double above = orc_e4m3_decode((uint8_t)(c + 1)) - a;
        if (above < below || (above == below && ((c + 1) & 1) == 0))
            c = c + 1;
    }
    return (uint8_t)(c | (signbit(x) ? 0x80 : 0));
}

/* READING: symmetric int8 is round-half-to-even, then clamp to [-127, 127]. */
int8_t orc_i8_encode(float x)
{
    double r = rint((double)x); /* default rounding mode: nearest, ties even */
    if (r > 127.0) r = 127.0;
    if (r < -127.0) r = -127.0;
    return (int8_t)r;
}

/* UE8M0 byte e encodes 2^(e-127). */
double orc_ue8m0_decode(uint8_t e)
{
    return ldexp(1.0, (int)e - 127);
}

/*
 * READING: a UE8M0 scale is the smallest power of two that is >= s, so that
 * no element of the group exceeds 448 after division.  Exponents below the
 * format's range clamp to code 0 (never reached by finite bf16 input of
 * practical size).  s > 0.
 */
uint8_t orc_ue8m0_encode(float s)
{
    int e;
    double f = frexp((double)s, &e); /* s = f * 2^e, f in [0.5, 1) */
    int p = (f == 0.5) ? e - 1 : e;  /* exponent of the smallest 2^p >= s */
    int code = p + 127;
    if (code < 0) code = 0;
    if (code > 254) code = 254;
    return (uint8_t)code;
}

double orc_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/*
 * bf16 nearest to v, ties to even, rounded once from the double.  bf16 keeps
 * 8 significant bits and binary32's exponent range (subnormal spacing 2^-133).
 */
uint16_t orc_bf16_from_double(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return 0x7FC0;
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);
    int lead = e - 1;         /* a in [2^lead, 2^(lead+1)) */
    if (lead < -126)
        lead = -126;          /* subnormal range: fixed spacing */
    double ulp = ldexp(1.0, lead - 7);
    double r = rint(a / ulp) * ulp; /* a/ulp is exact (power-of-two scale) */
    if (r >= ldexp(1.0, 128))
        return sign | 0x7F80; /* overflow to infinity */
    float f = (float)r;       /* exact: r is on the bf16 grid */
    uint32_t u;
    memcpy(&u, &f, 4);
    return sign | (uint16_t)(u >> 16);
}

static float bf16f(uint16_t b)
{
    return (float)orc_bf16_to_double(b);
}

/* ------------------------------------------------------------------------ */
/* Quantizers                                                                */
/* ------------------------------------------------------------------------ */

/*
 * Quantize n fp32 values sharing one scale:  amax = max |v|;  s = amax/qmax in
 * fp32 (READING: IEEE division, qmax = 448 for E4M3 and 127 for int8, s = 1
 * when amax is 0);  q = encode(clamp(v/s, -qmax, qmax)) with v/s an IEEE fp32
 * division.  For UE8M0 scales s is replaced by the power of two
 * 2^ceil(log2(amax/448)), and q is computed with that s.
 * The pages name this "dynamic per-token" quantization (mechatronicstore.cl,
 * "Patron de fusion del forward pass"; "Kernels Helion implementados").
 */
static void quant_span(int qtype, int scale_fmt, const float* v, int64_t n,
                       int64_t stride, void* q, float* s_out, uint8_t* e_out)
{
    float qmax = (qtype == ORC_FP8) ? 448.0f : 127.0f;
    float amax = 0.0f;
    int finite = 1;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(v[i * stride]);
        if (!isfinite(a)) finite = 0;
        if (a > amax) amax = a;
    }
    /* READING (the pages define nothing for NaN or infinite values; the inputs
     * of the contract are finite): a span holding a NaN or an infinity gets the
     * NaN scale (fp32 quiet NaN 0x7FC00000; UE8M0 code 0xFF) and the NaN code
     * for every element (E4M3 0x7F; int8 has no NaN: 0), so every output of
     * that token or group is NaN downstream. */
    if (!finite) {
        const uint32_t nan_bits = 0x7FC00000u;
        float nan_s;
        memcpy(&nan_s, &nan_bits, sizeof nan_s);
        if (s_out) *s_out = nan_s;
        if (e_out) *e_out = 0xFF;
        for (int64_t i = 0; i < n; ++i) {
            if (qtype == ORC_FP8)
                ((uint8_t*)q)[i * stride] = 0x7F;
            else
                ((int8_t*)q)[i * stride] = 0;
        }
        return;
    }
    float s = (amax > 0.0f) ? amax / qmax : 1.0f;
    if (scale_fmt == ORC_SCALE_UE8M0) {
        uint8_t e = orc_ue8m0_encode(s);
        s = (float)orc_ue8m0_decode(e);
        if (e_out) *e_out = e;
    }
    if (s_out) *s_out = s;
    for (int64_t i = 0; i < n; ++i) {
        float t = v[i * stride] / s;
        if (t > qmax) t = qmax;
        if (t < -qmax) t = -qmax;
        if (qtype == ORC_FP8)
            ((uint8_t*)q)[i * stride] = orc_e4m3_encode(t);
        else
            ((int8_t*)q)[i * stride] = orc_i8_encode(t);
    }
}

/* Per-token (per-row) quantization of bf16 x [M,K]: q [M,K], s [M]. */
void orc_quant_per_token(int qtype, const uint16_t* x, int64_t M, int64_t K,
                         void* q, float* s)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float* row = (float*)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1));
        for (int64_t k = 0; k < K; ++k)
            row[k] = bf16f(x[m * K + k]);
        char* qrow = (char*)q + m * K;
        quant_span(qtype, ORC_SCALE_F32, row, K, 1, qrow, &s[m], NULL);
        free(row);
    }
}

/* Per-token quantization of already-fp32 values (the fused producers' last step). */
void orc_quant_per_token_f32(int qtype, const float* y, int64_t M, int64_t K,
                             void* q, float* s)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        quant_span(qtype, ORC_SCALE_F32, y + m * K, K, 1, (char*)q + m * K, &s[m], NULL);
}

/*
 * Per-token-group FP8 quantization: groups of G consecutive K values of one
 * row share a scale ("per_token_group_fp8_quant", mechatronicstore.cl,
 * "Kernels Helion implementados").  READING: G = 128, K % G == 0, scales laid
 * out row-major [M, K/G]; fp32 scales or UE8M0 bytes.
 */
void orc_quant_group(int scale_fmt, const uint16_t* x, int64_t M, int64_t K,
                     int64_t G, uint8_t* q, void* s)
{
    int64_t ng = K / G;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float* row = (float*)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1));
        for (int64_t k = 0; k < K; ++k)
            row[k] = bf16f(x[m * K + k]);
        for (int64_t g = 0; g < ng; ++g) {
            float sf;
            uint8_t se;
            quant_span(ORC_FP8, scale_fmt, row + g * G, G, 1, q + m * K + g * G, &sf, &se);
            if (scale_fmt == ORC_SCALE_UE8M0)
                ((uint8_t*)s)[m * ng + g] = se;
            else
                ((float*)s)[m * ng + g] = sf;
        }
        free(row);
    }
}

/*
 * Weight quantization (offline, not part of the decode path).
 * Per-output-channel: a weight row [K] is quantized like a token row.
 */
void orc_quant_weight_per_channel(int qtype, const uint16_t* w, int64_t N, int64_t K,
                                  void* q, float* s)
{
    orc_quant_per_token(qtype, w, N, K, q, s);
}

/*
 * Block weight quantization: 128x128 blocks anchored at (0,0) share one
 * scale; scales row-major [ceil(N/128), K/128].  A partial last block row
 * (N % 128 != 0) covers the rows that exist.
 */
void orc_quant_weight_block(int scale_fmt, const uint16_t* w, int64_t N, int64_t K,
                            uint8_t* q, void* s)
{
    int64_t B = ORC_GROUP;
    int64_t nb = (N + B - 1) / B, kb = K / B;
#pragma omp parallel for schedule(static)
    for (int64_t bn = 0; bn < nb; ++bn) {
        int64_t rows = (bn * B + B <= N) ? B : N - bn * B;
        float* blk = (float*)malloc(sizeof(float) * (size_t)(B * B));
        uint8_t* qb = (uint8_t*)malloc((size_t)(B * B));
        for (int64_t bk = 0; bk < kb; ++bk) {
            for (int64_t r = 0; r < rows; ++r)
                for (int64_t c = 0; c < B; ++c)
                    blk[r * B + c] = bf16f(w[(bn * B + r) * K + bk * B + c]);
            float sf;
            uint8_t se;
            quant_span(ORC_FP8, scale_fmt, blk, rows * B, 1, qb, &sf, &se);
            for (int64_t r = 0; r < rows; ++r)
                for (int64_t c = 0; c < B; ++c)
                    q[(bn * B + r) * K + bk * B + c] = qb[r * B + c];
            if (scale_fmt == ORC_SCALE_UE8M0)
                ((uint8_t*)s)[bn * kb + bk] = se;
            else
                ((float*)s)[bn * kb + bk] = sf;
        }
        free(blk);
        free(qb);
    }
}

/*
 * Fused RMSNorm + per-token FP8 quantization ("rms_norm_dynamic_per_token_quant",
 * mechatronicstore.cl, "Kernels Helion implementados"; the norm+quant pair of
 * "Patron de fusion del forward pass").
 * READING: y = x * (1/sqrt(mean(x^2) + eps)) * w, evaluated in fp64 from the
 * bf16 inputs and rounded once to fp32, with no bf16 rounding in between;
 * the per-token quantizer then runs on those fp32 values.  y_out (optional)
 * receives the fp32 values.
 */
/* The fp64 RMSNorm value of every element before its rounding to fp32. */
void orc_rms_norm_prequant_f64(const uint16_t* x, const uint16_t* w, float eps, int64_t M,
                               int64_t H, double* y64)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        double ss = 0.0;
        for (int64_t k = 0; k < H; ++k) {
            double v = orc_bf16_to_double(x[m * H + k]);
            ss += v * v;
        }
        double r = 1.0 / sqrt(ss / (double)H + (double)eps);
        for (int64_t k = 0; k < H; ++k)
            y64[m * H + k] = (orc_bf16_to_double(x[m * H + k]) * r) * orc_bf16_to_double(w[k]);
    }
}

void orc_rms_norm_quant(const uint16_t* x, const uint16_t* w, float eps, int64_t M,
                        int64_t H, float* y_out, uint8_t* q, float* s)
{
    double* y64 = (double*)malloc(sizeof(double) * (size_t)(M * H > 0 ? M * H : 1));
    orc_rms_norm_prequant_f64(x, w, eps, M, H, y64);
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float* y = (float*)malloc(sizeof(float) * (size_t)(H > 0 ? H : 1));
        for (int64_t k = 0; k < H; ++k)
            y[k] = (float)y64[m * H + k];
        quant_span(ORC_FP8, ORC_SCALE_F32, y, H, 1, q + m * H, &s[m], NULL);
        if (y_out)
            memcpy(y_out + m * H, y, sizeof(float) * (size_t)H);
        free(y);
    }
    free(y64);
}

/*
 * Fused SiLU-and-mul + per-token FP8 quantization
 * ("silu_and_mul_dynamic_per_token_quant", mechatronicstore.cl, "Kernels Helion
 * implementados": the two steps in one launch).
 * READING: gate_up [M, 2I] holds gate in columns [0, I) and up in [I, 2I);
 * y = (g / (1 + exp(-g))) * u evaluated in fp64 and rounded once to fp32;
 * then the per-token quantizer on y [M, I].
 */
/* The fp64 SiLU-and-mul value of every element before its rounding to fp32. */
void orc_silu_mul_prequant_f64(const uint16_t* gu, int64_t M, int64_t I, double* y64)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < I; ++k) {
            double g = orc_bf16_to_double(gu[m * 2 * I + k]);
            double u = orc_bf16_to_double(gu[m * 2 * I + I + k]);
            y64[m * I + k] = (g / (1.0 + exp(-g))) * u;
        }
}

void orc_silu_mul_quant(const uint16_t* gu, int64_t M, int64_t I, float* y_out,
                        uint8_t* q, float* s)
{
    double* y64 = (double*)malloc(sizeof(double) * (size_t)(M * I > 0 ? M * I : 1));
    orc_silu_mul_prequant_f64(gu, M, I, y64);
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float* y = (float*)malloc(sizeof(float) * (size_t)(I > 0 ? I : 1));
        for (int64_t k = 0; k < I; ++k)
            y[k] = (float)y64[m * I + k];
        quant_span(ORC_FP8, ORC_SCALE_F32, y, I, 1, q + m * I, &s[m], NULL);
        if (y_out)
            memcpy(y_out + m * I, y, sizeof(float) * (size_t)I);
        free(y);
    }
    free(y64);
}

/*
 * Per-token-group FP8 quantization of already-fp32 values: the rule of
 * orc_quant_group applied to fp32 inputs (the block-format fused producers'
 * last step).  q [M,K], s [M, K/G] fp32 or UE8M0 bytes.
 */
void orc_quant_group_f32(int scale_fmt, const float* y, int64_t M, int64_t K, int64_t G,
                         uint8_t* q, void* s)
{
    int64_t ng = K / G;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t g = 0; g < ng; ++g) {
            float sf;
            uint8_t se;
            quant_span(ORC_FP8, scale_fmt, y + m * K + g * G, G, 1, q + m * K + g * G, &sf, &se);
            if (scale_fmt == ORC_SCALE_UE8M0)
                ((uint8_t*)s)[m * ng + g] = se;
            else
                ((float*)s)[m * ng + g] = sf;
        }
}

/*
 * Block-format fused producers ("rms_norm_per_block_quant" and
 * "silu_and_mul_per_block_quant", mechatronicstore.cl, "Kernels Helion
 * implementados"; the 1 x 128 group quantization with UE8M0 scales that the
 * block format pairs them with is named in "Patron de fusion del forward
 * pass").  READING: the same fp64 value as the per-token producers, rounded
 * once to fp32, then 1 x G group quantization of those fp32 values.
 * y_out (optional) receives the fp32 values.
 */
void orc_rms_norm_group_quant(const uint16_t* x, const uint16_t* w, float eps, int64_t M,
                              int64_t H, int64_t G, int scale_fmt, float* y_out, uint8_t* q,
                              void* s)
{
    double* y64 = (double*)malloc(sizeof(double) * (size_t)(M * H > 0 ? M * H : 1));
    float* y = (float*)malloc(sizeof(float) * (size_t)(M * H > 0 ? M * H : 1));
    orc_rms_norm_prequant_f64(x, w, eps, M, H, y64);
    for (int64_t i = 0; i < M * H; ++i)
        y[i] = (float)y64[i];
    orc_quant_group_f32(scale_fmt, y, M, H, G, q, s);
    if (y_out)
        memcpy(y_out, y, sizeof(float) * (size_t)(M * H));
    free(y);
    free(y64);
}

void orc_silu_mul_group_quant(const uint16_t* gu, int64_t M, int64_t I, int64_t G, int scale_fmt,
                              float* y_out, uint8_t* q, void* s)
{
    double* y64 = (double*)malloc(sizeof(double) * (size_t)(M * I > 0 ? M * I : 1));
    float* y = (float*)malloc(sizeof(float) * (size_t)(M * I > 0 ? M * I : 1));
    orc_silu_mul_prequant_f64(gu, M, I, y64);
    for (int64_t i = 0; i < M * I; ++i)
        y[i] = (float)y64[i];
    orc_quant_group_f32(scale_fmt, y, M, I, G, q, s);
    if (y_out)
        memcpy(y_out, y, sizeof(float) * (size_t)(M * I));
    free(y);
    free(y64);
}

/* ------------------------------------------------------------------------ */
/* Scaled GEMMs                                                              */
/* ------------------------------------------------------------------------ */

static double e4m3_table[256];
static int e4m3_table_ready = 0;

static void ensure_table(void)
{
    if (!e4m3_table_ready) {
        for (int c = 0; c < 256; ++c)
            e4m3_table[c] = orc_e4m3_decode((uint8_t)c);
        e4m3_table_ready = 1;
    }
}

/* Decoded value of element i of an 8-bit operand, exact in fp64. */
static double dec8(int qtype, const void* p, int64_t i)
{
    if (qtype == ORC_FP8)
        return e4m3_table[((const uint8_t*)p)[i]];
    return (double)((const int8_t*)p)[i];
}

/*
 * Dot product of activation row m with weight row n over k in [k0, k1).
 * Every 8-bit product is exact in fp64 and so is the running sum for the
 * sizes used (E4M3 products are multiples of 2^-18 below 2^18; int8 products
 * are integers below 2^14), so the result does not depend on the order.
 */
static double dot_range(int qtype, const void* qa, const void* qw, int64_t m, int64_t n,
                        int64_t K, int64_t k0, int64_t k1)
{
    double acc = 0.0;
    for (int64_t k = k0; k < k1; ++k)
        acc += dec8(qtype, qa, m * K + k) * dec8(qtype, qw, n * K + k);
    return acc;
}

/*
 * Grouped per-channel scaled GEMM for mixture-of-experts layers.  The pages
 * only name the extension to MoE models as a target ("Helion nel backend
 * vLLM", ai-radar.it, paragraph 9).  READING: the routed activation rows
 * arrive grouped by expert; rows offsets[e] .. offsets[e+1]-1 use expert e's
 * weights qw[e] [N,K] and scales sw[e] [N]:
 *   ref[m,n] = (a_s[m] * w_s[e(m), n]) * sum_k dec(qa[m,k]) * dec(qw[e(m),n,k])
 * Routing, the top-k gather and the weighted combination are outside it.
 * offsets has E+1 non-decreasing entries, offsets[0] = 0, offsets[E] = T.
 * For int8 acc (may be NULL) receives the exact accumulators (0 where one
 * leaves int32, which is not representable there).  Returns 0, or
 * -1 if an int8 accumulator leaves int32.
 */
int orc_grouped_scaled_mm(int qtype, const void* qa, const float* sa, const void* qw,
                          const float* sw, const int64_t* offsets, int64_t E, int64_t N,
                          int64_t K, double* ref, uint16_t* out, int32_t* acc)
{
    int bad = 0;
    ensure_table();
    size_t wsz = (qtype == ORC_FP8) ? sizeof(uint8_t) : sizeof(int8_t);
    for (int64_t e = 0; e < E; ++e) {
        const char* we = (const char*)qw + (size_t)(e * N * K) * wsz;
        const float* se = sw + e * N;
#pragma omp parallel for schedule(static) reduction(| : bad)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t m = offsets[e]; m < offsets[e + 1]; ++m) {
                double d = 0.0;
                for (int64_t k = 0; k < K; ++k)
                    d += dec8(qtype, qa, m * K + k) * dec8(qtype, we, n * K + k);
                double r = ((double)sa[m] * (double)se[n]) * d;
                if (qtype == ORC_INT8 && fabs(d) >= 2147483648.0) bad = 1;
                if (ref) ref[m * N + n] = r;
                if (out) out[m * N + n] = orc_bf16_from_double(r);
                if (acc && qtype == ORC_INT8) acc[m * N + n] = fabs(d) < 2147483648.0 ? (int32_t)d : 0;
            }
    }
    return bad ? -1 : 0;
}

/*
 * Split-K as a literal re-association: K is cut into S equal contiguous
 * chunks and the chunk partials are summed in chunk order ("Helion nel
 * backend vLLM", ai-radar.it, paragraphs 2-3: Split-K spreads K over several
 * thread blocks; split_k is a power of two up to 256).  S == 1 is the plain
 * sum.  The caller guarantees K % S == 0.
 */
static double dot_split(int qtype, const void* qa, const void* qw, int64_t m, int64_t n,
                        int64_t K, int64_t S)
{
    int64_t chunk = K / S;
    double total = 0.0;
    for (int64_t c = 0; c < S; ++c)
        total += dot_range(qtype, qa, qw, m, n, K, c * chunk, (c + 1) * chunk);
    return total;
}

/*
 * Per-channel scaled GEMM (FP8-dynamic or W8A8-INT8; "scaled_mm",
 * mechatronicstore.cl, "Kernels Helion implementados"; formats named in
 * "Unified GEMM Architecture", signaltitans.com).
 *   ref[m,n] = (a_s[m] * w_s[n]) * sum_k dec(qa[m,k]) * dec(qw[n,k])   (fp64)
 *   out[m,n] = bf16(ref[m,n])   (round to nearest even, once)
 * For int8 the sum is also returned as int32 in acc (the exact accumulator, or 0
 * where it leaves int32); acc may be NULL.  Returns 0, or -1 if an int8
 * accumulator leaves int32.
 * swap_ab != 0 computes the transposed product C' = W * A^T (weights in the
 * row role, activations in the column role, scale roles swapped) and writes
 * its transpose, which is Swap-AB read as A@B = (B^T @ A^T)^T ("Helion nel
 * backend vLLM", paragraph 2, whose printed formula is garbled).  ref, out and
 * acc may each be NULL.
 */
int orc_scaled_mm(int qtype, const void* qa, const float* sa, const void* qw, const float* sw,
                  int64_t M, int64_t N, int64_t K, int64_t split_k, int swap_ab,
                  double* ref, uint16_t* out, int32_t* acc)
{
    int bad = 0;
    ensure_table();
    if (!swap_ab) {
#pragma omp parallel for schedule(static) reduction(| : bad)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t m = 0; m < M; ++m) {
                double d = dot_split(qtype, qa, qw, m, n, K, split_k);
                double r = ((double)sa[m] * (double)sw[n]) * d;
                if (qtype == ORC_INT8 && fabs(d) >= 2147483648.0) bad = 1;
                if (ref) ref[m * N + n] = r;
                if (out) out[m * N + n] = orc_bf16_from_double(r);
                if (acc && qtype == ORC_INT8) acc[m * N + n] = fabs(d) < 2147483648.0 ? (int32_t)d : 0;
            }
    } else {
        /* C'[n,m] = sum_k w[n,k] a[m,k], column factor a_s, row factor w_s. */
        double* ct = (double*)malloc(sizeof(double) * (size_t)(M * N > 0 ? M * N : 1));
#pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t m = 0; m < M; ++m) {
                int64_t chunk = K / split_k;
                double total = 0.0;
                for (int64_t c = 0; c < split_k; ++c) {
                    double part = 0.0;
                    for (int64_t k = c * chunk; k < (c + 1) * chunk; ++k)
                        part += dec8(qtype, qw, n * K + k) * dec8(qtype, qa, m * K + k);
                    total += part;
                }
                ct[n * M + m] = total;
            }
        for (int64_t m = 0; m < M; ++m)
            for (int64_t n = 0; n < N; ++n) {
                double d = ct[n * M + m];
                double r = ((double)sw[n] * (double)sa[m]) * d;
                if (qtype == ORC_INT8 && fabs(d) >= 2147483648.0) bad = 1;
                if (ref) ref[m * N + n] = r;
                if (out) out[m * N + n] = orc_bf16_from_double(r);
                if (acc && qtype == ORC_INT8) acc[m * N + n] = fabs(d) < 2147483648.0 ? (int32_t)d : 0;
            }
        free(ct);
    }
    return bad ? -1 : 0;
}

/* Scale of a block or group as a double, from fp32 or UE8M0 storage. */
static double scale_at(int scale_fmt, const void* s, int64_t i)
{
    if (scale_fmt == ORC_SCALE_UE8M0)
        return orc_ue8m0_decode(((const uint8_t*)s)[i]);
    return (double)((const float*)s)[i];
}

/*
 * Block-FP8 scaled GEMM ("scaled_mm_blockwise", mechatronicstore.cl, "Kernels
 * Helion implementados"; "Block FP8" in "Unified GEMM Architecture").
 * READING: activations carry one scale per 1x128 group a_s[m, g] and weights
 * one per 128x128 block w_s[n/128, g]; for each K group g
 *   S[m,n,g] = sum_{k in g} dec(qa[m,k]) dec(qw[n,k])          (exact, fp64)
 *   ref[m,n] = sum_g (a_s[m,g] * w_s[n/128,g]) * S[m,n,g]       (fp64, g ascending)
 *   out[m,n] = bf16(ref[m,n]).
 * split_k cuts the K groups into S equal contiguous chunks (each a whole
 * number of groups) whose partials are summed in chunk order; swap_ab
 * computes the transposed product and writes its transpose.  K % 128 == 0.
 */
void orc_block_scaled_mm(int scale_fmt, const uint8_t* qa, const void* sa, const uint8_t* qw,
                         const void* sw, int64_t M, int64_t N, int64_t K, int64_t split_k,
                         int swap_ab, double* ref, uint16_t* out)
{
    int64_t G = ORC_GROUP, ng = K / G, per = ng / split_k;
    ensure_table();
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t m = 0; m < M; ++m) {
            double total = 0.0;
            for (int64_t c = 0; c < split_k; ++c) {
                double part = 0.0;
                for (int64_t g = c * per; g < (c + 1) * per; ++g) {
                    double blk = swap_ab
                        ? dot_range(ORC_FP8, qw, qa, n, m, K, g * G, (g + 1) * G)
                        : dot_range(ORC_FP8, qa, qw, m, n, K, g * G, (g + 1) * G);
                    double f = swap_ab
                        ? scale_at(scale_fmt, sw, (n / G) * ng + g) * scale_at(scale_fmt, sa, m * ng + g)
                        : scale_at(scale_fmt, sa, m * ng + g) * scale_at(scale_fmt, sw, (n / G) * ng + g);
                    part += f * blk;
                }
                total += part;
            }
            if (ref) ref[m * N + n] = total;
            if (out) out[m * N + n] = orc_bf16_from_double(total);
        }
}
