/*
 * oracle_driver.c -- runs every entry point of the C oracle on small inputs holding the
 * edge values its arithmetic meets (exact quotient ties, all-equal and all-zero groups,
 * subnormals, the largest finite bf16, negative zero), for a build with
 * -fsanitize=address,undefined.  Test infrastructure: compiles the oracle source in.
 * Prints one checksum line; any sanitizer report fails the run.
 */
#include <stdio.h>

#include "../../oracle/svdq_oracle.c"

static uint16_t bits_of(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static float edge_value(int i) {
    switch (i % 12) {
        case 0: return 0.0f;
        case 1: return -0.0f;
        case 2: return 3.3895314e38f;        /* largest finite bf16 */
        case 3: return -3.3895314e38f;
        case 4: return 1.0e-40f;             /* subnormal */
        case 5: return 1.17549435e-38f;      /* smallest normal */
        case 6: return 3.5f;                 /* halves: ties in the quotient */
        case 7: return -2.5f;
        case 8: return 7.0f;
        case 9: return 1.0f;
        default: return (float)((i * 37) % 101 - 50) / 8.0f;
    }
}

int main(void) {
    enum { M = 3, K = 128, N = 5, R = 16, KA = 256, NA = 6, MA = 2 };
    static uint16_t x[M * K], l1[R * K], l2[N * R], bias[N], lora[M * R], xa[MA * KA];
    static float si[K], w[N * K], wa[NA * KA], sa[M * (K / 64)], sw[N * (K / 64)];
    static uint8_t ca[M * K / 2], cw[N * K / 2], na[M * K / 2], nsa[M * K / 16], nw[N * K / 2],
        nsw[N * K / 16], qa[NA * KA / 2];
    static uint16_t asc[NA * (KA / 64)], azr[NA * (KA / 64)], abias[NA];
    static double out[M * N], outa[MA * NA], y[16], g[16];
    double sum = 0.0;
    for (int i = 0; i < M * K; ++i) x[i] = bits_of(i < K ? edge_value(i) : (i % K < 64 ? 2.0f : 0.0f));
    for (int i = 0; i < K; ++i) si[i] = i % 3 == 0 ? 1.0f : 0.5f;
    for (int i = 0; i < R * K; ++i) l1[i] = bits_of(edge_value(i + 5) * 1e-3f);
    for (int i = 0; i < N * R; ++i) l2[i] = bits_of((float)(i % 7 - 3) * 0.01f);
    for (int i = 0; i < N; ++i) bias[i] = bits_of((float)i * 0.1f);
    for (int i = 0; i < N * K; ++i) w[i] = edge_value(i * 5 + 1) * 1e-3f;

    oracle_quant_act_int4(M, K, R, x, si, l1, ca, sa, lora);
    oracle_quant_rows_int4(N, K, w, cw, sw);
    for (int act = 0; act < 2; ++act) {
        oracle_gemm_w4a4_int4(M, N, K, R, ca, sa, cw, sw, lora, l2, bias, act, out);
        for (int i = 0; i < M * N; ++i) sum += out[i];
        oracle_gemm_w4a4_int4(M, N, K, 0, ca, sa, cw, sw, NULL, NULL, NULL, act, out);
        for (int i = 0; i < M * N; ++i) sum += out[i];
    }
    int64_t mi[4] = {0, 2, 1, 0}, ni[4] = {4, 0, 3, 1};
    oracle_gemm_w4a4_int4_at(4, mi, ni, K, R, ca, sa, cw, sw, lora, l2, bias, 1, out);

    const float S = 1.0e-3f;
    oracle_quant_act_nvfp4(M, K, R, x, si, l1, S, na, nsa, lora);
    oracle_quant_rows_nvfp4(N, K, w, 1.0e-6f, nw, nsw);
    oracle_gemm_w4a4_nvfp4(M, N, K, R, na, nsa, S, nw, nsw, 1.0e-6f, lora, l2, bias, 1, out);
    for (int i = 0; i < M * N; ++i) sum += out[i];
    oracle_gemm_w4a4_nvfp4_at(4, mi, ni, K, 0, na, nsa, S, nw, nsw, 1.0e-6f, NULL, NULL, NULL, 0, out);

    for (int i = 0; i < 512; ++i) {
        const float v = (float)(i - 256) / 32.0f;
        sum += oracle_e4m3_decode(oracle_e4m3_encode(v < 0 ? -v : v));
        sum += oracle_e2m1_decode(oracle_e2m1_encode(v));
        sum += oracle_f32_to_bf16(edge_value(i)) + oracle_f64_to_bf16((double)v * 1e300);
    }

    for (int i = 0; i < NA * KA; ++i) wa[i] = i % 64 == 7 ? 0.0f : edge_value(i) * 1e-3f;
    for (int i = 0; i < 64; ++i) wa[i] = 0.25f;                     /* an all-equal group */
    oracle_awq_quant_weight(NA, KA, wa, qa, asc, azr);
    for (int i = 0; i < MA * KA; ++i) xa[i] = bits_of((float)(i % 9 - 4) * 0.5f);
    for (int i = 0; i < NA; ++i) abias[i] = bits_of((float)i * -0.25f);
    oracle_awq_gemv(MA, NA, KA, xa, qa, asc, azr, abias, outa);
    oracle_awq_gemv(MA, NA, KA, xa, qa, asc, azr, NULL, outa);
    for (int i = 0; i < MA * NA; ++i) sum += outa[i];

    for (int i = 0; i < 16; ++i) y[i] = (double)(i - 8) * 1.5;
    oracle_gelu_tanh(16, y, g);
    for (int i = 0; i < 16; ++i) sum += g[i];
    printf("oracle driver checksum %.17g\n", sum);
    return 0;
}
