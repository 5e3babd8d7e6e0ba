/*
 * oracle_driver.c -- runs every function of the CPU oracle (oracle/moe_oracle.c)
 * on small seeded inputs and on the edge shapes the tests use (one token, k = N,
 * group-limited routing, ragged experts, experts without rows, all-zero FP8
 * tiles, NaN keys), for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer.  Values are not checked here (the pins in
 * tests/test_oracle_*.py do that); any out-of-bounds access, leak or undefined
 * operation aborts the run.  Exit status 0 and the line "oracle driver ok"
 * mean every call completed cleanly.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void orc_round_to_dtype(int64_t n, int dtype, const double* v, void* out);
void orc_logits(int64_t T, int64_t d, int64_t N, int x_dtype, const void* x,
                const float* centroids, float* z);
void orc_sigmoid(int64_t n, const float* z, float* s);
void orc_select(int64_t T, int64_t N, int64_t k, int64_t G, int64_t TG, const float* s,
                const float* bias, int32_t* idx, float* gate);
void orc_histogram(int64_t T, int64_t k, int64_t N, const int32_t* idx, int32_t* counts);
void orc_route(int64_t T, int64_t d, int64_t N, int64_t k, int64_t G, int64_t TG, int x_dtype,
               const void* x, const float* centroids, const float* bias, float* scores,
               int32_t* idx, float* gate, int32_t* counts);
void orc_permute(int64_t T, int64_t k, int64_t N, const int32_t* idx, int32_t* offsets,
                 int32_t* src_token, int32_t* dst_row);
void orc_gather_rows(int64_t rows, int64_t row_bytes, const int32_t* src, const void* in,
                     void* out);
void orc_swiglu_ffn(int64_t M, int64_t d, int64_t I, int dtype, const void* A, const void* w13,
                    const void* w2, void* y);
void orc_e4m3_encode_array(int64_t n, const float* v, uint8_t* out);
void orc_e4m3_decode_array(int64_t n, const uint8_t* c, float* out);
void orc_quant_act_fp8(int64_t rows, int64_t cols, int dtype, const void* x, uint8_t* q,
                       float* scales);
void orc_quant_weight_fp8(int64_t n_mats, int64_t rows, int64_t cols, int dtype, const void* w,
                          uint8_t* q, float* scales);
void orc_swiglu_gateup_fp8(int64_t M, int64_t d, int64_t I, const uint8_t* Aq, const float* As,
                           const uint8_t* w13q, const float* w13s, float* h);
void orc_ffn_down_fp8(int64_t M, int64_t I, int64_t d, const uint8_t* hq, const float* hs,
                      const uint8_t* w2q, const float* w2s, uint16_t* y_bf16);
void orc_swiglu_ffn_fp8(int64_t M, int64_t d, int64_t I, const uint8_t* Aq, const float* As,
                        const uint8_t* w13q, const float* w13s, const uint8_t* w2q,
                        const float* w2s, uint16_t* y_bf16);
void orc_combine(int64_t T, int64_t d, int64_t k, int dtype, const void* x, const void* y_shared,
                 const void* y_perm, const float* gate, const int32_t* dst_row, void* out);
void orc_bias_update(int64_t N, int64_t TK, const int32_t* counts, float gamma, float* bias);
void orc_combine_backward(int64_t T, int64_t d, int64_t k, int dtype, const void* dout,
                          const void* y_perm, const float* gate, const int32_t* dst_row,
                          void* dy_perm, float* dgate);
void orc_swiglu_ffn_backward(int64_t M, int64_t d, int64_t I, int dtype, const void* A,
                             const void* w13, const void* w2, const void* dY, void* dA,
                             void* dw13, void* dw2);
void orc_route_backward(int64_t T, int64_t N, int64_t k, const float* scores, const int32_t* idx,
                        const float* dgate, float* dz);
void orc_centroid_grad(int64_t T, int64_t d, int64_t N, int64_t k, int dtype, const void* x,
                       const int32_t* idx, const float* dz, float* dE);
void orc_input_grad(int64_t T, int64_t d, int64_t k, int dtype, const void* dout,
                    const void* dx_shared, const void* dx_perm, const int32_t* dst_row,
                    const float* dz, const int32_t* idx, const float* centroids, void* dx);
void orc_quant_cols_fp8(int64_t M, int64_t C, int dtype, const void* x, uint8_t* q, float* s);
void orc_swiglu_ffn_backward_fp8(int64_t M, int64_t d, int64_t I, const uint8_t* Aq,
                                 const float* As, const uint16_t* A, const uint8_t* w13q,
                                 const float* w13s, const uint8_t* w2q, const float* w2s,
                                 const uint16_t* dY, uint16_t* dA, uint16_t* dw13,
                                 uint16_t* dw2);

static uint64_t rng = 88172645463325252ull;
static double unif(void) { /* xorshift64, uniform in [-1, 1) */
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return (double)(rng >> 11) / 4503599627370496.0 - 1.0;
}
static float* randf(int64_t n, double scale) {
    float* p = malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    for (int64_t i = 0; i < n; ++i) p[i] = (float)(unif() * scale);
    return p;
}
static uint16_t* randbf(int64_t n, double scale) { /* bf16 bits of random values */
    uint16_t* p = malloc((size_t)(n > 0 ? n : 1) * 2);
    for (int64_t i = 0; i < n; ++i) {
        float f = (float)(unif() * scale);
        uint32_t u;
        memcpy(&u, &f, 4);
        p[i] = (uint16_t)(u >> 16);
    }
    return p;
}

/* one forward + backward through every oracle function for one shape */
static void layer(int64_t T, int64_t d, int64_t N, int64_t k, int64_t G, int64_t TG, int64_t I,
                  int nan_row) {
    const int64_t TK = T * k;
    uint16_t* x = randbf(T * d, 2.0);
    if (nan_row && T > 1) for (int64_t j = 0; j < d; ++j) x[1 * d + j] = 0x7fc0;
    float* E = randf(N * d, 0.1);
    float* b = randf(N, 1e-3);
    float* scores = malloc((size_t)(T * N + 1) * 4);
    int32_t* idx = malloc((size_t)(TK + 1) * 4);
    float* gate = malloc((size_t)(TK + 1) * 4);
    int32_t* counts = malloc((size_t)N * 4);
    orc_route(T, d, N, k, G, TG, 1, x, E, b, scores, idx, gate, counts);
    int32_t* offsets = malloc((size_t)(N + 1) * 4);
    int32_t* src = malloc((size_t)(TK + 1) * 4);
    int32_t* dst = malloc((size_t)(TK + 1) * 4);
    orc_permute(T, k, N, idx, offsets, src, dst);
    uint16_t* xp = malloc((size_t)(TK * d + 1) * 2);
    orc_gather_rows(TK, d * 2, src, x, xp);
    /* bf16 experts (every expert, including ones without rows) */
    uint16_t* w13 = randbf(2 * I * d, 0.05);
    uint16_t* w2 = randbf(d * I, 0.05);
    uint16_t* yp = malloc((size_t)(TK * d + 1) * 2);
    for (int64_t e = 0; e < N; ++e) {
        int64_t a0 = offsets[e], a1 = offsets[e + 1];
        if (a1 > a0) orc_swiglu_ffn(a1 - a0, d, I, 1, xp + a0 * d, w13, w2, yp + a0 * d);
    }
    uint16_t* ys = malloc((size_t)(T * d + 1) * 2);
    orc_swiglu_ffn(T, d, I, 1, x, w13, w2, ys);
    uint16_t* out = malloc((size_t)(T * d + 1) * 2);
    orc_combine(T, d, k, 1, x, ys, yp, gate, dst, out);
    orc_combine(T, d, k, 1, NULL, NULL, yp, gate, dst, out);
    orc_bias_update(N, TK, counts, 0.001f, b);
    /* backward */
    uint16_t* dout = randbf(T * d, 1.0);
    uint16_t* dyp = malloc((size_t)(TK * d + 1) * 2);
    float* dgate = malloc((size_t)(TK + 1) * 4);
    orc_combine_backward(T, d, k, 1, dout, yp, gate, dst, dyp, dgate);
    uint16_t* dxp = malloc((size_t)(TK * d + 1) * 2);
    uint16_t* dw13 = malloc((size_t)(2 * I * d) * 2);
    uint16_t* dw2 = malloc((size_t)(d * I) * 2);
    for (int64_t e = 0; e < N; ++e) {
        int64_t a0 = offsets[e], a1 = offsets[e + 1];
        orc_swiglu_ffn_backward(a1 - a0, d, I, 1, xp + a0 * d, w13, w2, dyp + a0 * d,
                                dxp + a0 * d, dw13, dw2);
    }
    float* dz = malloc((size_t)(TK + 1) * 4);
    orc_route_backward(T, N, k, scores, idx, dgate, dz);
    float* dE = malloc((size_t)(N * d) * 4);
    orc_centroid_grad(T, d, N, k, 1, x, idx, dz, dE);
    uint16_t* dxs = malloc((size_t)(T * d + 1) * 2);
    orc_swiglu_ffn_backward(T, d, I, 1, x, w13, w2, dout, dxs, dw13, dw2);
    uint16_t* dx = malloc((size_t)(T * d + 1) * 2);
    orc_input_grad(T, d, k, 1, dout, dxs, dxp, dst, dz, idx, E, dx);
    orc_input_grad(T, d, k, 1, NULL, NULL, dxp, dst, dz, idx, E, dx);
    /* FP8 (d, I multiples of 128) */
    if (d % 128 == 0 && I % 128 == 0) {
        uint8_t* xq = malloc((size_t)(T * d + 1));
        float* xs = malloc((size_t)(T * d / 128 + 1) * 4);
        if (T > 0) for (int64_t j = 0; j < 128; ++j) x[j] = 0; /* an all-zero tile */
        orc_quant_act_fp8(T, d, 1, x, xq, xs);
        uint8_t* w13q = malloc((size_t)(2 * I * d));
        float* w13s = malloc((size_t)(2 * I * d / 16384) * 4);
        uint8_t* w2q = malloc((size_t)(d * I));
        float* w2s = malloc((size_t)(d * I / 16384) * 4);
        orc_quant_weight_fp8(1, 2 * I, d, 1, w13, w13q, w13s);
        orc_quant_weight_fp8(1, d, I, 1, w2, w2q, w2s);
        float* h = malloc((size_t)(T * I + 1) * 4);
        uint8_t* hq = malloc((size_t)(T * I + 1));
        float* hs = malloc((size_t)(T * I / 128 + 1) * 4);
        uint16_t* y8 = malloc((size_t)(T * d + 1) * 2);
        orc_swiglu_gateup_fp8(T, d, I, xq, xs, w13q, w13s, h);
        orc_quant_act_fp8(T, I, 0, h, hq, hs);
        orc_ffn_down_fp8(T, I, d, hq, hs, w2q, w2s, y8);
        orc_swiglu_ffn_fp8(T, d, I, xq, xs, w13q, w13s, w2q, w2s, y8);
        uint8_t* cq = malloc((size_t)(T * d + 1));
        float* cs = malloc((size_t)(((T + 127) / 128) * d + 1) * 4);
        orc_quant_cols_fp8(T, d, 1, x, cq, cs);
        uint16_t* dA8 = malloc((size_t)(T * d + 1) * 2);
        orc_swiglu_ffn_backward_fp8(T, d, I, xq, xs, x, w13q, w13s, w2q, w2s, dout, dA8, dw13,
                                    dw2);
        free(xq); free(xs); free(w13q); free(w13s); free(w2q); free(w2s); free(h); free(hq);
        free(hs); free(y8); free(cq); free(cs); free(dA8);
    }
    free(x); free(E); free(b); free(scores); free(idx); free(gate); free(counts); free(offsets);
    free(src); free(dst); free(xp); free(w13); free(w2); free(yp); free(ys); free(out);
    free(dout); free(dyp); free(dgate); free(dxp); free(dw13); free(dw2); free(dz); free(dE);
    free(dxs); free(dx);
}

int main(void) {
    /* shapes: T, d, N, k, G, TG, I, a NaN row */
    layer(64, 128, 16, 2, 1, 1, 128, 0);
    layer(1, 128, 16, 2, 1, 1, 128, 0);      /* one token */
    layer(77, 256, 8, 8, 1, 1, 128, 1);      /* k = N, NaN row */
    layer(130, 128, 32, 6, 8, 3, 256, 1);    /* group-limited, ragged */
    layer(300, 256, 64, 4, 32, 4, 128, 0);   /* 32 groups of 2 experts */
    layer(200, 384, 4, 1, 1, 1, 128, 0);     /* k = 1, d % 256 != 0 */
    layer(0, 128, 16, 2, 1, 1, 128, 0);      /* no tokens */
    /* encoder / decoder over every code and some specials */
    uint8_t codes[256];
    float dec[256];
    for (int i = 0; i < 256; ++i) codes[i] = (uint8_t)i;
    orc_e4m3_decode_array(256, codes, dec);
    float v[8] = {0.0f, -0.0f, 448.0f, -448.0f, 1e-30f, 2.5f, 0.001953125f, 300.0f};
    uint8_t q[8];
    orc_e4m3_encode_array(8, v, q);
    double r[4] = {1.0, -2.5, 1e300, -0.0};
    uint16_t rb[4];
    float rf[4];
    orc_round_to_dtype(4, 1, r, rb);
    orc_round_to_dtype(4, 0, r, rf);
    float z[3] = {0.5f, -20.0f, 20.0f}, s[3];
    orc_sigmoid(3, z, s);
    printf("oracle driver ok\n");
    return 0;
}
