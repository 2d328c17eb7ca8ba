/*
 * svdq_oracle.c -- plain, slow, scalar CPU oracle for the SVDQuant W4A4 linear,
 * its NVFP4 variant and the AWQ W4A16 GEMV.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library may link, load or
 * call this file.  It shares no code, header, table or constant with the HIP
 * path; it is compiled by gcc with -O2 -ffp-contract=off and no fast-math, so
 * every float operation below is one IEEE-754 binary32 or binary64 operation
 * rounded to nearest-even, in program order.
 *
 * Sources (the pages this follows; short keys used in the comments):
 *   [margrop]  "Hugging Face 把 Nunchaku 4-bit Diffusion 接到 Diffusers ..." (blog.margrop.com),
 *              section 技术细节 1 ("SVDQuant 的核心思路", four steps) and
 *              section 技术细节 3 (kernel families: svdq_w4a4 int4 / nvfp4, awq_w4a16 int4).
 *   [ainews]   "Diffusers Natively Integrates Nunchaku Lite, Using W4A4 to Reduce
 *              Diffusion Model VRAM Usage and Latency" (ainews.surl.tw), second and
 *              third paragraphs (outlier migration, 16-bit low-rank branch, 4-bit
 *              weights and activations; AWQ W4A16 for modulation layers; config.json
 *              fields method / precision / group size / rank).
 *   [hamidun]  "Nunchaku Lite: 4-битная генерация изображений в Diffusers" (app.hamidun.com),
 *              section "Что такое Nunchaku и SVDQuant".
 *   [keryc]    keryc.com article on Nunchaku in Diffusers, sections "Qué es Nunchaku y por
 *              qué importa" and "Nunchaku Lite: integración y modelo de ejecución".
 *
 * The pages name the method and its kernel families but print no numeric rule.  The
 * numeric conventions implemented here are this library's definitions (each is listed
 * with its reason in the design notes of the repository):
 *   - INT4: groups of 64 consecutive input channels per row; scale s = absmax / 7 in fp32
 *     (correctly rounded division); code q = clamp(rne(x / s), -8, 7) with the fp32
 *     quotient rounded half-to-even; s == 0 gives all-zero codes.
 *   - Packing: two's-complement nibbles, low nibble = even channel, row-major [rows, K/2].
 *   - NVFP4: blocks of 16; E4M3 (OCP "FN": bias 7, max 448, no infinities) block scale
 *     sb = E4M3(min(absmax / (6 * S), 448)); E2M1 code = nearest of x / (sb * S), ties to the
 *     even code, saturating at 6, sign kept; sb == 0 gives all-zero codes.
 *   - AWQ: asymmetric uint4 with integer zero-point per 64-group; bf16 scale and zero.
 *   - The low-rank down-projection is X . L1^T on raw bf16 X, summed in fp64 and rounded
 *     once to bf16; the GEMM result is returned in fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- bf16 */

static float bf16_to_f32(uint16_t h) {
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Nearest bf16 to a binary64 value, ties to even, with one rounding.
 * bf16 has an 8-bit significand, exponent range of binary32 (min normal 2^-126,
 * subnormal spacing 2^-133, max finite (2 - 2^-7) * 2^127). */
uint16_t oracle_f64_to_bf16(double d) {
    if (isnan(d)) return 0x7FC0;
    double a = fabs(d);
    uint16_t sign = signbit(d) ? 0x8000 : 0;
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                 /* a = f * 2^e, f in [0.5, 1) */
    int q = e - 8;                /* spacing of 8-significant-bit numbers in this binade */
    if (q < -133) q = -133;       /* subnormal spacing floor */
    double r = nearbyint(ldexp(a, -q));   /* round half to even (default mode) */
    double v = ldexp(r, q);
    const double maxf = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
    if (v > maxf) return sign | 0x7F80;    /* overflow rounds to infinity */
    float f = (float)v;                    /* exact: v has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return sign | (uint16_t)(u >> 16);
}

uint16_t oracle_f32_to_bf16(float f) { return oracle_f64_to_bf16((double)f); }

/* ---------------------------------------------------------------- INT4 */

/* Quantize one group of fp32 values (already smoothed) to int4 codes and its fp32
 * scale: s = absmax / 7, q = clamp(rne(v / s), -8, 7).  [margrop 技术细节 1 step 3:
 * the residual and the activations are carried in 4 bits.] */
static float int4_group(const float* v, int n, int8_t* q) {
    float a = 0.0f;
    for (int i = 0; i < n; ++i) {
        float t = fabsf(v[i]);
        if (t > a) a = t;
    }
    float s = a / 7.0f;
    for (int i = 0; i < n; ++i) {
        if (s == 0.0f) { q[i] = 0; continue; }
        float t = v[i] / s;
        float r = nearbyintf(t);          /* half to even */
        if (r < -8.0f) r = -8.0f;
        if (r > 7.0f) r = 7.0f;
        q[i] = (int8_t)r;
    }
    return s;
}

static void pack_nibbles(const int8_t* q, int n, uint8_t* out) {
    for (int i = 0; i < n; i += 2)
        out[i / 2] = (uint8_t)(((uint8_t)q[i] & 0x0F) | (((uint8_t)q[i + 1] & 0x0F) << 4));
}

static int int4_code(const uint8_t* row, int64_t k) {
    uint8_t b = row[k >> 1];
    int nib = (k & 1) ? (b >> 4) : (b & 0x0F);
    return nib >= 8 ? nib - 16 : nib;
}

/* Low-rank down-projection of one token row: lora[j] = bf16(sum_k x[k] * l1[j,k]),
 * summed in fp64 and rounded once.  [margrop 技术细节 1 step 4: the 16-bit low-rank
 * branch's down-projection runs inside the quantization kernel.] */
static void lowrank_down_row(int64_t K, int r, const uint16_t* xrow, const uint16_t* l1,
                             uint16_t* lora_row) {
    for (int j = 0; j < r; ++j) {
        double acc = 0.0;
        const uint16_t* lj = l1 + (int64_t)j * K;
        for (int64_t k = 0; k < K; ++k)
            acc += (double)bf16_to_f32(xrow[k]) * (double)bf16_to_f32(lj[k]);
        lora_row[j] = oracle_f64_to_bf16(acc);
    }
}

/* Activation stage, INT4 precision.  Smoothing: x_hat = fp32(x) * smooth_inv[k]
 * (outlier migration, [margrop 技术细节 1 step 1], [ainews] paragraph 3), then group
 * quantization and packing, then the low-rank down-projection on raw x. */
void oracle_quant_act_int4(int64_t M, int64_t K, int r, const uint16_t* x,
                           const float* smooth_inv, const uint16_t* l1,
                           uint8_t* codes, float* scales, uint16_t* lora) {
    const int G = 64;
    float v[64];
    int8_t q[64];
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t* xr = x + m * K;
        for (int64_t g = 0; g < K / G; ++g) {
            for (int i = 0; i < G; ++i) {
                int64_t k = g * G + i;
                v[i] = bf16_to_f32(xr[k]) * smooth_inv[k];
            }
            scales[m * (K / G) + g] = int4_group(v, G, q);
            pack_nibbles(q, G, codes + m * (K / 2) + g * (G / 2));
        }
        if (r > 0) lowrank_down_row(K, r, xr, l1, lora + m * r);
    }
}

/* The same 64-group rule applied to fp32 rows (the 4-bit residual weights,
 * [margrop 技术细节 1 step 3]). */
void oracle_quant_rows_int4(int64_t rows, int64_t K, const float* vals, uint8_t* codes,
                            float* scales) {
    const int G = 64;
    int8_t q[64];
    for (int64_t n = 0; n < rows; ++n)
        for (int64_t g = 0; g < K / G; ++g) {
            scales[n * (K / G) + g] = int4_group(vals + n * K + g * G, G, q);
            pack_nibbles(q, G, codes + n * (K / 2) + g * (G / 2));
        }
}

static double gelu_tanh(double y) {
    const double c = sqrt(2.0 / 3.14159265358979323846);
    return 0.5 * y * (1.0 + tanh(c * (y + 0.044715 * y * y * y)));
}

/* Low-rank up-projection + bias + optional GELU(tanh) for one output element.
 * [margrop 技术细节 1 step 4: the up-projection is fused into the 4-bit compute
 * kernel]; GELU/MLP fusion is what the original engine adds [margrop 技术细节 2]. */
static double epilogue(double acc, int64_t m, int64_t n, int r, const uint16_t* lora,
                       const uint16_t* l2, const uint16_t* bias, int act) {
    for (int j = 0; j < r; ++j)
        acc += (double)bf16_to_f32(lora[m * r + j]) * (double)bf16_to_f32(l2[n * r + j]);
    if (bias) acc += (double)bf16_to_f32(bias[n]);
    if (act == 1) acc = gelu_tanh(acc);
    return acc;
}

/* One output of the INT4 W4A4 GEMM: per 64-group exact integer dot product D_g, scaled
 * by fp64(sa) * fp64(sw), summed in fp64; then the epilogue. */
static double gemm_int4_one(int64_t m, int64_t n, int64_t K, int r, const uint8_t* ca,
                            const float* sa, const uint8_t* cw, const float* sw,
                            const uint16_t* lora, const uint16_t* l2, const uint16_t* bias,
                            int act) {
    const int64_t G = K / 64;
    const uint8_t* ar = ca + m * (K / 2);
    const uint8_t* wr = cw + n * (K / 2);
    double acc = 0.0;
    for (int64_t g = 0; g < G; ++g) {
        int64_t d = 0;
        for (int64_t k = g * 64; k < g * 64 + 64; ++k)
            d += (int64_t)int4_code(ar, k) * (int64_t)int4_code(wr, k);
        acc += (double)sa[m * G + g] * (double)sw[n * G + g] * (double)d;
    }
    return epilogue(acc, m, n, r, lora, l2, bias, act);
}

void oracle_gemm_w4a4_int4(int64_t M, int64_t N, int64_t K, int r, const uint8_t* ca,
                           const float* sa, const uint8_t* cw, const float* sw,
                           const uint16_t* lora, const uint16_t* l2, const uint16_t* bias,
                           int act, double* out) {
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            out[m * N + n] = gemm_int4_one(m, n, K, r, ca, sa, cw, sw, lora, l2, bias, act);
}

/* Selected outputs (m[i], n[i]) only, for parity at full size. */
void oracle_gemm_w4a4_int4_at(int64_t npts, const int64_t* mi, const int64_t* ni, int64_t K,
                              int r, const uint8_t* ca, const float* sa, const uint8_t* cw,
                              const float* sw, const uint16_t* lora, const uint16_t* l2,
                              const uint16_t* bias, int act, double* out) {
    for (int64_t i = 0; i < npts; ++i)
        out[i] = gemm_int4_one(mi[i], ni[i], K, r, ca, sa, cw, sw, lora, l2, bias, act);
}

/* ---------------------------------------------------------------- NVFP4 */

/* E4M3 ("FN" variant, OCP 8-bit float): bias 7, exponent field 0 is subnormal with
 * spacing 2^-9, largest finite 448 = 1.75 * 2^8, no infinities.  Decode of a
 * non-negative code. */
double oracle_e4m3_decode(uint8_t b) {
    int e = (b >> 3) & 0xF, m = b & 7;
    double mag = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return (b & 0x80) ? -mag : mag;
}

/* Nearest E4M3 to v >= 0 with ties to even, after clamping to 448 (saturation). */
uint8_t oracle_e4m3_encode(float vf) {
    double v = (double)vf;
    if (!(v > 0.0)) return 0;
    if (v > 448.0) v = 448.0;
    int e;
    frexp(v, &e);                 /* v in [2^(e-1), 2^e) */
    int q = e - 4;                /* 4 significant bits */
    if (q < -9) q = -9;           /* subnormal spacing */
    double r = nearbyint(ldexp(v, -q)) ;
    double w = ldexp(r, q);       /* the rounded value (may be 2^e exactly) */
    /* encode w */
    if (w == 0.0) return 0;
    if (w < ldexp(1.0, -6)) return (uint8_t)(int)ldexp(w, 9); /* subnormal: m = w / 2^-9 */
    int ew;
    double f = frexp(w, &ew);     /* w = f * 2^ew, f in [0.5,1) */
    int exp_field = ew - 1 + 7;
    int mant = (int)((f * 2.0 - 1.0) * 8.0);
    return (uint8_t)((exp_field << 3) | mant);
}

/* E2M1 (4-bit float): magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7, sign in bit 3. */
double oracle_e2m1_decode(uint8_t c) {
    static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    double v = mag[c & 7];
    return (c & 8) ? -v : v;
}

/* Nearest E2M1 magnitude to |v|, ties to the even code, saturating at 6; sign kept. */
uint8_t oracle_e2m1_encode(float vf) {
    double a = fabs((double)vf);
    int best = 0;
    double bd = INFINITY;
    for (int c = 0; c < 8; ++c) {
        double d = fabs(a - oracle_e2m1_decode((uint8_t)c));
        if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) { bd = d; best = c; }
    }
    return (uint8_t)(best | (signbit(vf) ? 8 : 0));
}

/* One 16-block: block scale and codes.  S is the per-tensor fp32 scale. */
static uint8_t nvfp4_block(const float* v, float S, uint8_t* codes) {
    float a = 0.0f;
    for (int i = 0; i < 16; ++i) {
        float t = fabsf(v[i]);
        if (t > a) a = t;
    }
    float den = 6.0f * S;
    float sbv = a / den;
    uint8_t sb = oracle_e4m3_encode(sbv);
    if (sb == 0) {
        for (int i = 0; i < 16; ++i) codes[i] = 0;
        return 0;
    }
    float d = (float)oracle_e4m3_decode(sb) * S;
    for (int i = 0; i < 16; ++i) codes[i] = oracle_e2m1_encode(v[i] / d);
    return sb;
}

static void pack_u4(const uint8_t* c, int n, uint8_t* out) {
    for (int i = 0; i < n; i += 2) out[i / 2] = (uint8_t)((c[i] & 0xF) | ((c[i + 1] & 0xF) << 4));
}

/* Activation stage, NVFP4 precision ([margrop 技术细节 3]: svdq_w4a4 with precision
 * nvfp4).  Smoothing and the low-rank branch are those of the INT4 stage. */
void oracle_quant_act_nvfp4(int64_t M, int64_t K, int r, const uint16_t* x,
                            const float* smooth_inv, const uint16_t* l1, float S,
                            uint8_t* codes, uint8_t* scales, uint16_t* lora) {
    float v[16];
    uint8_t c[16];
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t* xr = x + m * K;
        for (int64_t b = 0; b < K / 16; ++b) {
            for (int i = 0; i < 16; ++i) {
                int64_t k = b * 16 + i;
                v[i] = bf16_to_f32(xr[k]) * smooth_inv[k];
            }
            scales[m * (K / 16) + b] = nvfp4_block(v, S, c);
            pack_u4(c, 16, codes + m * (K / 2) + b * 8);
        }
        if (r > 0) lowrank_down_row(K, r, xr, l1, lora + m * r);
    }
}

void oracle_quant_rows_nvfp4(int64_t rows, int64_t K, const float* vals, float S,
                             uint8_t* codes, uint8_t* scales) {
    uint8_t c[16];
    for (int64_t n = 0; n < rows; ++n)
        for (int64_t b = 0; b < K / 16; ++b) {
            scales[n * (K / 16) + b] = nvfp4_block(vals + n * K + b * 16, S, c);
            pack_u4(c, 16, codes + n * (K / 2) + b * 8);
        }
}

static double gemm_nvfp4_one(int64_t m, int64_t n, int64_t K, int r, const uint8_t* ca,
                             const uint8_t* sa, float Sa, const uint8_t* cw,
                             const uint8_t* sw, float Sw, const uint16_t* lora,
                             const uint16_t* l2, const uint16_t* bias, int act) {
    const int64_t B = K / 16;
    const uint8_t* ar = ca + m * (K / 2);
    const uint8_t* wr = cw + n * (K / 2);
    double acc = 0.0;
    for (int64_t b = 0; b < B; ++b) {
        double d = 0.0;   /* exact: products of E2M1 values are multiples of 1/4 below 36 */
        for (int64_t k = b * 16; k < b * 16 + 16; ++k) {
            uint8_t xa = (k & 1) ? (ar[k >> 1] >> 4) : (ar[k >> 1] & 0xF);
            uint8_t xw = (k & 1) ? (wr[k >> 1] >> 4) : (wr[k >> 1] & 0xF);
            d += oracle_e2m1_decode(xa) * oracle_e2m1_decode(xw);
        }
        acc += d * oracle_e4m3_decode(sa[m * B + b]) * oracle_e4m3_decode(sw[n * B + b]);
    }
    acc *= (double)Sa * (double)Sw;
    return epilogue(acc, m, n, r, lora, l2, bias, act);
}

void oracle_gemm_w4a4_nvfp4(int64_t M, int64_t N, int64_t K, int r, const uint8_t* ca,
                            const uint8_t* sa, float Sa, const uint8_t* cw, const uint8_t* sw,
                            float Sw, const uint16_t* lora, const uint16_t* l2,
                            const uint16_t* bias, int act, double* out) {
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            out[m * N + n] =
                gemm_nvfp4_one(m, n, K, r, ca, sa, Sa, cw, sw, Sw, lora, l2, bias, act);
}

void oracle_gemm_w4a4_nvfp4_at(int64_t npts, const int64_t* mi, const int64_t* ni, int64_t K,
                               int r, const uint8_t* ca, const uint8_t* sa, float Sa,
                               const uint8_t* cw, const uint8_t* sw, float Sw,
                               const uint16_t* lora, const uint16_t* l2, const uint16_t* bias,
                               int act, double* out) {
    for (int64_t i = 0; i < npts; ++i)
        out[i] = gemm_nvfp4_one(mi[i], ni[i], K, r, ca, sa, Sa, cw, sw, Sw, lora, l2, bias, act);
}

/* ---------------------------------------------------------------- AWQ W4A16 */

/* Weight quantization for the W4A16 path ([ainews] paragraph 3 and [hamidun]
 * "Что такое Nunchaku и SVDQuant": awq_w4a16 keeps 4-bit weights and 16-bit
 * activations for the modulation layers).  Per (row n, 64-group g):
 *   lo, hi = min, max;  sc = bf16((hi - lo) / 15) (1 if that is 0);
 *   z = clamp(rne(-lo / sc), 0, 15);  q = clamp(rne(w / sc) + z, 0, 15).
 * q is unsigned, low nibble = even channel; sc and z are stored as bf16. */
void oracle_awq_quant_weight(int64_t N, int64_t K, const float* w, uint8_t* qweight,
                             uint16_t* scales, uint16_t* zeros) {
    const int64_t G = K / 64;
    uint8_t q[64];
    for (int64_t n = 0; n < N; ++n)
        for (int64_t g = 0; g < G; ++g) {
            const float* v = w + n * K + g * 64;
            float lo = v[0], hi = v[0];
            for (int i = 1; i < 64; ++i) {
                if (v[i] < lo) lo = v[i];
                if (v[i] > hi) hi = v[i];
            }
            float range = hi - lo;
            uint16_t scb = oracle_f32_to_bf16(range / 15.0f);
            float sc = bf16_to_f32(scb);
            if (sc == 0.0f) { scb = 0x3F80; sc = 1.0f; }
            float z = nearbyintf(-lo / sc);
            if (z < 0.0f) z = 0.0f;
            if (z > 15.0f) z = 15.0f;
            z = z + 0.0f;  /* -0 -> +0 */
            for (int i = 0; i < 64; ++i) {
                float t = nearbyintf(v[i] / sc) + z;
                if (t < 0.0f) t = 0.0f;
                if (t > 15.0f) t = 15.0f;
                q[i] = (uint8_t)t;
            }
            scales[n * G + g] = scb;
            zeros[n * G + g] = oracle_f32_to_bf16(z);
            pack_u4(q, 64, qweight + n * (K / 2) + g * 32);
        }
}

/* Y[m,n] = sum_k x[m,k] * (q[n,k] - z[n,g]) * sc[n,g] + b[n], in fp64. */
void oracle_awq_gemv(int64_t M, int64_t N, int64_t K, const uint16_t* x, const uint8_t* qweight,
                     const uint16_t* scales, const uint16_t* zeros, const uint16_t* bias,
                     double* out) {
    const int64_t G = K / 64;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                int64_t g = k / 64;
                uint8_t b = qweight[n * (K / 2) + (k >> 1)];
                int q = (k & 1) ? (b >> 4) : (b & 0xF);
                double sc = bf16_to_f32(scales[n * G + g]);
                double z = bf16_to_f32(zeros[n * G + g]);
                acc += (double)bf16_to_f32(x[m * K + k]) * ((double)q - z) * sc;
            }
            if (bias) acc += (double)bf16_to_f32(bias[n]);
            out[m * N + n] = acc;
        }
}

/* GELU(tanh) on a vector, fp64, for chaining stages in tests. */
void oracle_gelu_tanh(int64_t n, const double* y, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = gelu_tanh(y[i]);
}
