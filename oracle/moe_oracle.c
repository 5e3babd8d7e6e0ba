/*
 * moe_oracle.c -- plain, slow, obviously-correct CPU oracle for one
 * DeepSeekMoE feed-forward layer: its forward pass, its per-step bias update,
 * and the gradients of the forward (bf16 / fp32 storage).
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the reference the GPU library is
 * checked against.  Only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load it.  It shares no code, header, table or
 * constant generator with the HIP library, and it never touches a GPU.
 *
 * Sources (the pages are web copies of material about the DeepSeek-V3
 * technical report, arXiv:2412.19437):
 *  [P4]  "DeepSeek-V3 Technischer Bericht" reading guide (xyznot.com/de),
 *        section "Methode", item 2 "DeepSeekMoE mit Auxiliary-Loss-Free
 *        Balancing": the layer output h'_t, the sigmoid affinity s_{i,t},
 *        the biased Topk definition of g'_{i,t}, the normalisation of g',
 *        and the end-of-step bias rule with gamma = 0.001.
 *  [P4k] same page, "Kernideen", FP8 bullet: E4M3 for all tensors, 1x128
 *        activation tiles, 128x128 weight blocks, FP32 promotion every
 *        N_c = 128 accumulation steps.
 *  [P1]  "DeepSeek-V3 技術報告書：MLAと極小スパースMoE..." (singularity-lens.com),
 *        its formula paragraph: bias rule b <- b + gamma*sign(mean_load - load),
 *        and FP8 scaling S = max|X|/448, X_fp8 = clip(round(X/S), -448, 448).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - logits are a fixed-order fp32 FMA chain over the hidden dimension
 *    (index ascending, starting from +0.0f); the pages give only u^T e_i;
 *  - sigmoid is evaluated in double and rounded once to fp32;
 *  - ties in the Topk are broken toward the lower expert index; -0 == +0;
 *    a NaN key (or a NaN group score) ranks as -inf, so a token whose keys
 *    are all NaN still gets k valid experts (the lowest eligible indices);
 *  - group-limited routing: G contiguous groups of N/G experts; a group's
 *    score is the fp32 sum of its two largest biased keys; the TG best
 *    groups (ties to the lower group) are kept; the pages do not define it
 *    (parity unpinned by the pages; pinned only by brute force against this
 *    reading);
 *  - gates: g_j = s_j / sum of the selected s, no extra scaling factor;
 *  - the FFN is SwiGLU without biases: W2 (silu(W1 u) * (W3 u)); the pages
 *    only write FFN_i (parity unpinned by the pages; pinned by the dense
 *    textbook reduction against an independent library matmul);
 *  - the sequence-wise balance loss (named, with alpha = 0.0001, in [P4]'s
 *    last sentence of "Methode" item 2, without a formula) is read as
 *    alpha * sum_i f_i P_i per sequence, see orc_seq_balance_loss (parity
 *    unpinned by the pages; pinned by closed forms and invariances of that
 *    reading);
 *  - permutation: stable counting sort of (token, slot) pairs by expert;
 *  - the bias update compares load_i * N with T*k exactly in integers;
 *    gamma is the fp32 value nearest 0.001; sign(0) = 0;
 *  - FP8 is OCP E4M3FN (largest finite 448); scale = amax/448 as an fp32
 *    divide; x/scale is an fp32 divide, clamped to +-448, then rounded to the
 *    nearest E4M3 value, ties to even; an all-zero tile has scale 0 and all
 *    codes 0;
 *  - FP8 backward ("E4M3 for all tensors" read as: every operand of every
 *    expert GEMM of the backward is E4M3, activations and gradients in tiles
 *    of 128 along that GEMM's contraction, weights in their 128x128 blocks):
 *    dh = dY W2 and dX = [da db] [W1; W3] contract over features, so dY and
 *    [da db] are quantised 1x128 per row; dW2 = dY^T h and dW13 = [da db]^T X
 *    contract over the expert's rows, so dY, h, [da db] and X are quantised
 *    in 128x1 tiles along the rows (128 consecutive rows of one expert from
 *    its first row, the last tile partial), each from its bf16 value; a, b
 *    come from the FP8 forward (fp32) and are kept in bf16 with
 *    h = silu(a) b; dh, da, db and every output are rounded to bf16.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1

/* ---------------------------------------------------------------------- */
/* scalar helpers                                                         */
/* ---------------------------------------------------------------------- */

static float bf16_bits_to_float(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round a double to bfloat16 with a single rounding, nearest-even.  bf16
 * keeps 8 significant bits; below 2^-126 the grid step is fixed at 2^-133. */
static uint16_t double_to_bf16_bits(double v) {
    if (isnan(v)) return 0x7fc0;
    double a = fabs(v), r = 0.0;
    if (a != 0.0 && !isinf(a)) {
        int ex;
        frexp(a, &ex); /* a in [2^(ex-1), 2^ex) */
        int step = ex - 8;
        if (step < -133) step = -133;
        r = ldexp(nearbyint(ldexp(a, -step)), step); /* exact in double */
    } else if (isinf(a)) {
        r = a;
    }
    float f = (float)r; /* exact, or +inf past the largest finite bf16 */
    uint32_t u;
    memcpy(&u, &f, 4);
    u >>= 16;
    if (signbit(v)) u |= 0x8000u;
    return (uint16_t)u;
}

static float load_elem(const void* p, int dtype, int64_t i) {
    if (dtype == ORC_BF16) return bf16_bits_to_float(((const uint16_t*)p)[i]);
    return ((const float*)p)[i];
}

static void store_elem_from_double(void* p, int dtype, int64_t i, double v) {
    if (dtype == ORC_BF16)
        ((uint16_t*)p)[i] = double_to_bf16_bits(v);
    else
        ((float*)p)[i] = (float)v;
}

/* Exposed for the pins: round doubles to the storage dtype. */
void orc_round_to_dtype(int64_t n, int dtype, const double* v, void* out) {
    for (int64_t i = 0; i < n; ++i) store_elem_from_double(out, dtype, i, v[i]);
}

/* ---------------------------------------------------------------------- */
/* routing: affinity, biased selection, gates   [P4] Methode 2            */
/* ---------------------------------------------------------------------- */

/* z[t,i] = u_t . e_i as the chain acc = fma(x[t,j], e[i,j], acc), j = 0..d-1,
 * starting from +0.0f.  The loop runs over j outermost so that several
 * independent chains advance together; each output's own order is the
 * definition above. */
void orc_logits(int64_t T, int64_t d, int64_t N, int x_dtype, const void* x,
                const float* centroids, float* z) {
    float* et = (float*)malloc((size_t)(d * N) * sizeof(float));
    for (int64_t i = 0; i < N; ++i)
        for (int64_t j = 0; j < d; ++j) et[j * N + i] = centroids[i * d + j];
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        float* zt = z + t * N;
        for (int64_t i = 0; i < N; ++i) zt[i] = 0.0f;
        for (int64_t j = 0; j < d; ++j) {
            float xv = load_elem(x, x_dtype, t * d + j);
            const float* ej = et + j * N;
            for (int64_t i = 0; i < N; ++i) zt[i] = fmaf(xv, ej[i], zt[i]);
        }
    }
    free(et);
}

/* s = Sigmoid(z), in double, rounded once to fp32.   [P4] s_{i,t} */
void orc_sigmoid(int64_t n, const float* z, float* s) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) s[i] = (float)(1.0 / (1.0 + exp(-(double)z[i])));
}

/* total order used for every selection: larger key first, lower index on ties */
static int beats(float ra, int64_t a, float rb, int64_t b) {
    return ra > rb || (ra == rb && a < b);
}

/* For one token: scores s[N], bias b[N] -> idx[k] (selection order), gate[k].
 * [P4]: g'_{i,t} = s_{i,t} if s_{i,t}+b_i is among the K_r largest of
 * {s_{j,t}+b_j}; gates are the g' normalised over the chosen experts; the bias
 * only enters the key. */
static void select_one(int64_t N, int64_t k, int64_t G, int64_t TG, const float* s,
                       const float* b, int32_t* idx, float* gate, float* r,
                       unsigned char* allowed) {
    for (int64_t i = 0; i < N; ++i) {
        float v = s[i] + b[i];
        if (v == 0.0f) v = 0.0f; /* -0 -> +0 */
        if (isnan(v)) v = -INFINITY; /* a NaN key ranks below every number */
        r[i] = v;
        allowed[i] = 1;
    }
    if (G > 1) {
        int64_t gs = N / G;
        float gscore[1024];
        unsigned char gkeep[1024];
        for (int64_t g = 0; g < G; ++g) {
            /* two largest keys of the group under the total order */
            int64_t i1 = -1, i2 = -1;
            for (int64_t i = g * gs; i < (g + 1) * gs; ++i) {
                if (i1 < 0 || beats(r[i], i, r[i1], i1)) {
                    i2 = i1;
                    i1 = i;
                } else if (i2 < 0 || beats(r[i], i, r[i2], i2)) {
                    i2 = i;
                }
            }
            float sc = r[i1] + r[i2];
            if (sc == 0.0f) sc = 0.0f;
            if (isnan(sc)) sc = -INFINITY; /* +inf + -inf: ranks lowest, like a NaN key */
            gscore[g] = sc;
            gkeep[g] = 0;
        }
        for (int64_t pick = 0; pick < TG; ++pick) {
            int64_t best = -1;
            for (int64_t g = 0; g < G; ++g) {
                if (gkeep[g]) continue;
                if (best < 0 || beats(gscore[g], g, gscore[best], best)) best = g;
            }
            gkeep[best] = 1;
        }
        for (int64_t i = 0; i < N; ++i) allowed[i] = gkeep[i / gs];
    }
    for (int64_t j = 0; j < k; ++j) {
        int64_t best = -1;
        for (int64_t i = 0; i < N; ++i) {
            if (!allowed[i]) continue;
            if (best < 0 || beats(r[i], i, r[best], best)) best = i;
        }
        idx[j] = (int32_t)best;
        allowed[best] = 0;
    }
    double S = 0.0;
    for (int64_t j = 0; j < k; ++j) S += (double)s[idx[j]];
    for (int64_t j = 0; j < k; ++j) gate[j] = (float)((double)s[idx[j]] / S);
}

void orc_select(int64_t T, int64_t N, int64_t k, int64_t G, int64_t TG, const float* s,
                const float* bias, int32_t* idx, float* gate) {
#pragma omp parallel
    {
        float* r = (float*)malloc((size_t)N * sizeof(float));
        unsigned char* allowed = (unsigned char*)malloc((size_t)N);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t)
            select_one(N, k, G, TG, s + t * N, bias, idx + t * k, gate + t * k, r, allowed);
        free(r);
        free(allowed);
    }
}

/* counts[e] = number of (token, slot) pairs routed to e (the step's load) */
void orc_histogram(int64_t T, int64_t k, int64_t N, const int32_t* idx, int32_t* counts) {
    for (int64_t e = 0; e < N; ++e) counts[e] = 0;
    for (int64_t p = 0; p < T * k; ++p) counts[idx[p]] += 1;
}

/* Whole routing step: logits, sigmoid, biased selection, gates, counts.
 * scores may be NULL. */
void orc_route(int64_t T, int64_t d, int64_t N, int64_t k, int64_t G, int64_t TG,
               int x_dtype, const void* x, const float* centroids, const float* bias,
               float* scores, int32_t* idx, float* gate, int32_t* counts) {
    float* z = (float*)malloc((size_t)(T * N) * sizeof(float));
    float* s = scores ? scores : (float*)malloc((size_t)(T * N) * sizeof(float));
    orc_logits(T, d, N, x_dtype, x, centroids, z);
    orc_sigmoid(T * N, z, s);
    orc_select(T, N, k, G, TG, s, bias, idx, gate);
    orc_histogram(T, k, N, idx, counts);
    if (!scores) free(s);
    free(z);
}

/* ---------------------------------------------------------------------- */
/* permutation by expert (stable counting sort)                           */
/* ---------------------------------------------------------------------- */

/* offsets[N+1] = exclusive prefix sum of the per-expert counts; rows are
 * handed out scanning tokens t ascending, then slots j ascending:
 * row = offsets[e] + (rows of e handed out so far). */
void orc_permute(int64_t T, int64_t k, int64_t N, const int32_t* idx, int32_t* offsets,
                 int32_t* src_token, int32_t* dst_row) {
    int32_t* counts = (int32_t*)calloc((size_t)N, sizeof(int32_t));
    int32_t* cursor = (int32_t*)calloc((size_t)N, sizeof(int32_t));
    orc_histogram(T, k, N, idx, counts);
    offsets[0] = 0;
    for (int64_t e = 0; e < N; ++e) offsets[e + 1] = offsets[e] + counts[e];
    for (int64_t t = 0; t < T; ++t)
        for (int64_t j = 0; j < k; ++j) {
            int32_t e = idx[t * k + j];
            int32_t row = offsets[e] + cursor[e]++;
            src_token[row] = (int32_t)t;
            dst_row[t * k + j] = row;
        }
    free(counts);
    free(cursor);
}

/* out[r] = in[src[r]], rows of row_bytes bytes, bit for bit */
void orc_gather_rows(int64_t rows, int64_t row_bytes, const int32_t* src, const void* in,
                     void* out) {
    for (int64_t r = 0; r < rows; ++r)
        memcpy((char*)out + r * row_bytes, (const char*)in + (int64_t)src[r] * row_bytes,
               (size_t)row_bytes);
}

/* ---------------------------------------------------------------------- */
/* expert FFN (SwiGLU) in double accumulation                              */
/* ---------------------------------------------------------------------- */

static double silu_d(double a) { return a / (1.0 + exp(-a)); }

/* A [M,d] rows of one expert; w13 [2I,d]: rows 0..I-1 are W1 (gate), rows
 * I..2I-1 are W3 (up); w2 [d,I].  y[m,:] = W2 (silu(W1 a_m) * (W3 a_m)).
 * a, b: double sums rounded to fp32; h: double, rounded to the storage dtype;
 * y: double sum rounded to the storage dtype. */
void orc_swiglu_ffn(int64_t M, int64_t d, int64_t I, int dtype, const void* A,
                    const void* w13, const void* w2, void* y) {
    double* h = (double*)malloc((size_t)(M * I) * sizeof(double));
    /* h[m,n]: one (row, column) per iteration; parallel over both */
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < I; ++n) {
            double sa = 0.0, sb = 0.0;
            for (int64_t j = 0; j < d; ++j) {
                double av = (double)load_elem(A, dtype, m * d + j);
                sa += av * (double)load_elem(w13, dtype, n * d + j);
                sb += av * (double)load_elem(w13, dtype, (I + n) * d + j);
            }
            double a = (double)(float)sa, b = (double)(float)sb;
            double hv = silu_d(a) * b;
            /* h is stored in the storage dtype between the two projections */
            if (dtype == ORC_BF16)
                h[m * I + n] = (double)bf16_bits_to_float(double_to_bf16_bits(hv));
            else
                h[m * I + n] = (double)(float)hv;
        }
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int64_t n = 0; n < I; ++n)
                acc += h[m * I + n] * (double)load_elem(w2, dtype, c * I + n);
            store_elem_from_double(y, dtype, m * d + c, acc);
        }
    free(h);
}

/* ---------------------------------------------------------------------- */
/* FP8 E4M3FN   [P4k] tiles/blocks, [P1] scale rule                        */
/* ---------------------------------------------------------------------- */

/* E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;
 * S.1111.111 is NaN; largest finite 448 = 1.75 * 2^8; smallest normal 2^-6;
 * subnormals m * 2^-9, m = 1..7. */
float orc_e4m3_decode(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 0xf, m = c & 7;
    double v;
    if (e == 0xf && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return (float)(s ? -v : v);
}

/* nearest E4M3FN code, ties to even; |v| must be <= 448 (callers clamp); a
 * NaN (which no clamp removes) encodes as the format's NaN, S.1111.111 */
uint8_t orc_e4m3_encode(float v) {
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v)) return (uint8_t)(sign | 0x7f);
    double a = fabs((double)v);
    if (a < ldexp(1.0, -6)) {
        /* subnormal grid step 2^-9; a result of 8 steps is the smallest
         * normal, whose code is also 8 (exponent field 1, mantissa 0) */
        double q = nearbyint(ldexp(a, 9)); /* default rounding: nearest-even */
        return (uint8_t)(sign | (uint8_t)q);
    }
    int ex;
    frexp(a, &ex);      /* a = f * 2^ex, f in [0.5, 1) */
    int e = ex - 1;     /* a = 1.xxx * 2^e, e in [-6, 8] */
    double q = nearbyint(ldexp(a, 3 - e)); /* 8..16 : 1.mmm scaled by 8 */
    if (q == 16.0) {
        q = 8.0;
        e += 1;
    }
    int mant = (int)q - 8;
    return (uint8_t)(sign | (uint8_t)(((e + 7) << 3) | mant));
}

void orc_e4m3_encode_array(int64_t n, const float* v, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(v[i]);
}

void orc_e4m3_decode_array(int64_t n, const uint8_t* c, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_decode(c[i]);
}

/* quantise a group of values that share one scale: scale = amax/448 (fp32
 * divide); q = E4M3(clamp(v/scale, -448, 448)); all-zero -> scale 0, codes 0 */
static float quant_scale(float amax) { return amax / 448.0f; }

static uint8_t quant_one(float v, float scale) {
    if (scale == 0.0f) return 0;
    float t = v / scale;
    if (t > 448.0f) t = 448.0f;
    if (t < -448.0f) t = -448.0f;
    return orc_e4m3_encode(t);
}

/* activations: rows x cols (cols % 128 == 0), one scale per row per 128
 * consecutive columns (a 1x128 tile along the contraction dimension).
 * scales: [rows, cols/128] */
void orc_quant_act_fp8(int64_t rows, int64_t cols, int dtype, const void* x, uint8_t* q,
                       float* scales) {
    int64_t nt = cols / 128;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < nt; ++c) {
            float amax = 0.0f;
            for (int64_t j = 0; j < 128; ++j) {
                float a = fabsf(load_elem(x, dtype, r * cols + c * 128 + j));
                if (a > amax) amax = a;
            }
            float sc = quant_scale(amax);
            scales[r * nt + c] = sc;
            for (int64_t j = 0; j < 128; ++j)
                q[r * cols + c * 128 + j] = quant_one(load_elem(x, dtype, r * cols + c * 128 + j), sc);
        }
}

/* weights: n_mats matrices of rows x cols (both % 128 == 0), one scale per
 * 128x128 block.  scales: [n_mats, rows/128, cols/128] */
void orc_quant_weight_fp8(int64_t n_mats, int64_t rows, int64_t cols, int dtype, const void* w,
                          uint8_t* q, float* scales) {
    int64_t br = rows / 128, bc = cols / 128;
#pragma omp parallel for schedule(static)
    for (int64_t mb = 0; mb < n_mats * br; ++mb) {
        int64_t mat = mb / br, rb = mb % br;
        for (int64_t cb = 0; cb < bc; ++cb) {
            float amax = 0.0f;
            for (int64_t i = 0; i < 128; ++i)
                for (int64_t j = 0; j < 128; ++j) {
                    int64_t off = mat * rows * cols + (rb * 128 + i) * cols + cb * 128 + j;
                    float a = fabsf(load_elem(w, dtype, off));
                    if (a > amax) amax = a;
                }
            float sc = quant_scale(amax);
            scales[(mat * br + rb) * bc + cb] = sc;
            for (int64_t i = 0; i < 128; ++i)
                for (int64_t j = 0; j < 128; ++j) {
                    int64_t off = mat * rows * cols + (rb * 128 + i) * cols + cb * 128 + j;
                    q[off] = quant_one(load_elem(w, dtype, off), sc);
                }
        }
    }
}

/* sum over one 128-wide contraction block of decoded code products; exact in
 * double (each product has at most 8 significant bits, 128 terms) */
static double block_dot(const uint8_t* a, const uint8_t* b, const double* lut) {
    double s = 0.0;
    for (int j = 0; j < 128; ++j) s += lut[a[j]] * lut[b[j]];
    return s;
}

static void e4m3_lut(double* lut) {
    for (int c = 0; c < 256; ++c) {
        float v = orc_e4m3_decode((uint8_t)c);
        lut[c] = isnan(v) ? 0.0 : (double)v;
    }
}

/* FP8 gate/up half of the SwiGLU expert:  A_q [M,d] codes with A_s [M,d/128];
 * w13_q [2I,d] with w13_s [2I/128, d/128] (rows 0..I-1 W1, I..2I-1 W3).
 * a[m,n] and b[m,n] are sums over the 128-wide contraction blocks kb of
 * (s_a[m,kb] * s_w[nb,kb]) times the block's exact code-product sum (the
 * "promotion every 128" of [P4k]), each rounded to fp32;
 * h[m,n] = silu(a) * b evaluated in double and rounded to fp32. */
void orc_swiglu_gateup_fp8(int64_t M, int64_t d, int64_t I, const uint8_t* Aq, const float* As,
                           const uint8_t* w13q, const float* w13s, float* h) {
    double lut[256];
    e4m3_lut(lut);
    int64_t kd = d / 128;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < I; ++n) {
            const uint8_t* am = Aq + m * d;
            double sa = 0.0, sb = 0.0;
            for (int64_t kb = 0; kb < kd; ++kb) {
                double pa = block_dot(am + kb * 128, w13q + n * d + kb * 128, lut);
                double pb = block_dot(am + kb * 128, w13q + (I + n) * d + kb * 128, lut);
                double xs = (double)As[m * kd + kb];
                sa += xs * (double)w13s[(n / 128) * kd + kb] * pa;
                sb += xs * (double)w13s[((I + n) / 128) * kd + kb] * pb;
            }
            double a = (double)(float)sa, b = (double)(float)sb;
            h[m * I + n] = (float)(silu_d(a) * b);
        }
}

/* FP8 down half:  h_q [M,I] codes with h_s [M,I/128] (1x128 tiles of h);
 * w2_q [d,I] with w2_s [d/128, I/128].  y[m,c] = sum over the 128-wide blocks
 * kb of (s_h[m,kb] * s_w[cb,kb]) times the block's exact code-product sum,
 * rounded once to bf16. */
void orc_ffn_down_fp8(int64_t M, int64_t I, int64_t d, const uint8_t* hq, const float* hs,
                      const uint8_t* w2q, const float* w2s, uint16_t* y_bf16) {
    double lut[256];
    e4m3_lut(lut);
    int64_t ki = I / 128;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int64_t kb = 0; kb < ki; ++kb) {
                double p = block_dot(hq + m * I + kb * 128, w2q + c * I + kb * 128, lut);
                acc += (double)hs[m * ki + kb] * (double)w2s[(c / 128) * ki + kb] * p;
            }
            y_bf16[m * d + c] = double_to_bf16_bits(acc);
        }
}

/* The whole FP8 SwiGLU expert: the gate/up half gives h in fp32; h is
 * re-quantised per 1x128 tile exactly like the activations ([P4k]: E4M3 for
 * all tensors); the down half gives y in bf16. */
void orc_swiglu_ffn_fp8(int64_t M, int64_t d, int64_t I, const uint8_t* Aq, const float* As,
                        const uint8_t* w13q, const float* w13s, const uint8_t* w2q,
                        const float* w2s, uint16_t* y_bf16) {
    int64_t ki = I / 128;
    float* h = (float*)malloc((size_t)(M * I) * sizeof(float));
    uint8_t* hq = (uint8_t*)malloc((size_t)(M * I));
    float* hs = (float*)malloc((size_t)(M * ki) * sizeof(float));
    orc_swiglu_gateup_fp8(M, d, I, Aq, As, w13q, w13s, h);
    orc_quant_act_fp8(M, I, ORC_F32, h, hq, hs);
    orc_ffn_down_fp8(M, I, d, hq, hs, w2q, w2s, y_bf16);
    free(h);
    free(hq);
    free(hs);
}

/* ---------------------------------------------------------------------- */
/* combine   [P4] h'_t = u_t + sum shared FFN + sum_i g_{i,t} FFN_i        */
/* ---------------------------------------------------------------------- */

/* out[t,:] = x[t,:] (if x != NULL) + y_shared[t,:] + sum_j gate[t,j] *
 * y_perm[dst_row[t,j], :], summed in double, rounded to the dtype. */
void orc_combine(int64_t T, int64_t d, int64_t k, int dtype, const void* x,
                 const void* y_shared, const void* y_perm, const float* gate,
                 const int32_t* dst_row, void* out) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t c = 0; c < d; ++c) {
            double acc = 0.0;
            if (x) acc += (double)load_elem(x, dtype, t * d + c);
            if (y_shared) acc += (double)load_elem(y_shared, dtype, t * d + c);
            for (int64_t j = 0; j < k; ++j)
                acc += (double)gate[t * k + j] *
                       (double)load_elem(y_perm, dtype, (int64_t)dst_row[t * k + j] * d + c);
            store_elem_from_double(out, dtype, t * d + c, acc);
        }
}

/* ---------------------------------------------------------------------- */
/* bias update   [P4] end-of-step rule, [P1] sign form                     */
/* ---------------------------------------------------------------------- */

/* expert i is overloaded when its load exceeds the mean load T*k/N, i.e.
 * counts[i]*N > T*k: b_i <- b_i - gamma; underloaded: b_i <- b_i + gamma;
 * exactly at the mean: unchanged.  fp32 arithmetic. */
void orc_bias_update(int64_t N, int64_t TK, const int32_t* counts, float gamma, float* bias) {
    for (int64_t i = 0; i < N; ++i) {
        int64_t lhs = (int64_t)counts[i] * N;
        if (lhs > TK)
            bias[i] = bias[i] - gamma;
        else if (lhs < TK)
            bias[i] = bias[i] + gamma;
    }
}

/* ---------------------------------------------------------------------- */
/* sequence-wise balance loss   [P4] "Methode" item 2, last sentence        */
/* ---------------------------------------------------------------------- */

/* The pages name a minimal sequence-wise balance loss (alpha = 0.0001) that
 * complements the bias rule by keeping any single sequence away from extreme
 * imbalance, and the issoh.co.jp page describes the conventional auxiliary
 * loss as a penalty on inputs crowding onto particular experts; neither
 * prints a formula.  Reading (parity unpinned by the pages): the batch is
 * T / S sequences of S consecutive tokens, and for sequence b
 *   f_i = N / (k S) * #{(t, j) : t in b, idx[t][j] = i}   (load relative to
 *         the uniform share k S / N, the same load the bias rule compares)
 *   P_i = (1 / S) * sum_{t in b} s_{i,t} / sum_{j<N} s_{j,t}   (mean affinity
 *         of expert i, normalised over all N experts per token)
 *   loss[b] = alpha * sum_i f_i P_i.
 * Every sum in double, in index order; loss[b] rounded once to fp32.  With
 * equal affinities the loss is alpha whatever the routing; with every token
 * on the same k experts holding all of its affinity it is alpha * N / k. */
void orc_seq_balance_loss(int64_t T, int64_t N, int64_t k, int64_t S, float alpha,
                          const float* scores, const int32_t* idx, float* loss) {
    int64_t B = T / S;
    double* P = (double*)malloc((size_t)N * sizeof(double));
    int64_t* cnt = (int64_t*)malloc((size_t)N * sizeof(int64_t));
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t i = 0; i < N; ++i) {
            P[i] = 0.0;
            cnt[i] = 0;
        }
        for (int64_t t = b * S; t < (b + 1) * S; ++t) {
            double row = 0.0;
            for (int64_t i = 0; i < N; ++i) row += (double)scores[t * N + i];
            for (int64_t i = 0; i < N; ++i) P[i] += (double)scores[t * N + i] / row;
            for (int64_t j = 0; j < k; ++j) cnt[idx[t * k + j]] += 1;
        }
        double sum = 0.0;
        for (int64_t i = 0; i < N; ++i) {
            double f = (double)N / ((double)k * (double)S) * (double)cnt[i];
            sum += f * (P[i] / (double)S);
        }
        loss[b] = (float)((double)alpha * sum);
    }
    free(P);
    free(cnt);
}

/* ====================================================================== */
/* backward pass of the layer                                              */
/* ====================================================================== */
/*
 * The gradient of the layer statement ([P4] "Methode" item 2) with respect to
 * its inputs and parameters, by the chain rule, given the upstream gradient
 * dout = dL/dh'_t.  The selection (idx) is piecewise constant and the bias
 * enters only the selection key, so neither carries a gradient; gates carry
 * one through s_{i,t} = sigmoid(u_t^T e_i) into u_t and the centroids e_i.
 *
 * Storage points mirror the forward: a, b are fp32 sums; h = silu(a)*b is
 * stored in the storage dtype; the backward also reads a and b back from
 * storage (rounded to the dtype) and stores da, db in the dtype.  Every sum is
 * a double sum; each output is rounded once.
 */

/* combine backward.  out[t] = x[t] + y_s[t] + sum_j gate[t,j] y_perm[dst[t,j]]:
 *   dy_perm[dst[t,j], c] = gate[t,j] * dout[t,c]       (rounded to the dtype)
 *   dgate[t,j] = sum_c dout[t,c] * y_perm[dst[t,j], c]  (fp32)
 * The residual and shared-expert gradients are dout itself. */
void orc_combine_backward(int64_t T, int64_t d, int64_t k, int dtype, const void* dout,
                          const void* y_perm, const float* gate, const int32_t* dst_row,
                          void* dy_perm, float* dgate) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t j = 0; j < k; ++j) {
            const int64_t row = dst_row[t * k + j];
            double acc = 0.0;
            for (int64_t c = 0; c < d; ++c) {
                const double g = (double)load_elem(dout, dtype, t * d + c);
                acc += g * (double)load_elem(y_perm, dtype, row * d + c);
                store_elem_from_double(dy_perm, dtype, row * d + c, (double)gate[t * k + j] * g);
            }
            dgate[t * k + j] = (float)acc;
        }
}

static double sigmoid_d(double a) { return 1.0 / (1.0 + exp(-a)); }

static double round_dtype(int dtype, double v) {
    if (dtype == ORC_BF16) return (double)bf16_bits_to_float(double_to_bf16_bits(v));
    return (double)(float)v;
}

/* SwiGLU expert backward over the M rows A [M,d] of one expert, with
 * w13 [2I,d] (W1 rows, then W3 rows), w2 [d,I] and the gradient dY [M,d] of
 * its output y = W2 (silu(W1 a) * (W3 a)):
 *   a, b = W1 A, W3 A (fp32); h = silu(a)*b (dtype)           -- forward values
 *   dh[m,n] = sum_c dY[m,c] w2[c,n]
 *   da = dh * b * silu'(a),  silu'(a) = sig(a) (1 + a (1 - sig(a)));  db = dh * silu(a)
 *       (a, b read back in the dtype; da, db stored in the dtype)
 *   dA[m,c]   = sum_n da[m,n] w13[n,c] + db[m,n] w13[I+n,c]
 *   dw2[c,n]  = sum_m dY[m,c] h[m,n]
 *   dw13[n,c] = sum_m da[m,n] A[m,c];  dw13[I+n,c] = sum_m db[m,n] A[m,c]
 * M may be 0 (dA empty, weight gradients zero). */
void orc_swiglu_ffn_backward(int64_t M, int64_t d, int64_t I, int dtype, const void* A,
                             const void* w13, const void* w2, const void* dY, void* dA,
                             void* dw13, void* dw2) {
    double* h = (double*)malloc((size_t)(M * I + 1) * sizeof(double));
    double* da = (double*)malloc((size_t)(M * I + 1) * sizeof(double));
    double* db = (double*)malloc((size_t)(M * I + 1) * sizeof(double));
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < I; ++n) {
            double sa = 0.0, sb = 0.0, sh = 0.0;
            for (int64_t c = 0; c < d; ++c) {
                const double av = (double)load_elem(A, dtype, m * d + c);
                sa += av * (double)load_elem(w13, dtype, n * d + c);
                sb += av * (double)load_elem(w13, dtype, (I + n) * d + c);
                sh += (double)load_elem(dY, dtype, m * d + c) *
                      (double)load_elem(w2, dtype, c * I + n);
            }
            const double a = (double)(float)sa, b = (double)(float)sb;
            h[m * I + n] = round_dtype(dtype, a / (1.0 + exp(-a)) * b);
            const double ar = round_dtype(dtype, a), br = round_dtype(dtype, b);
            const double sg = sigmoid_d(ar);
            da[m * I + n] = round_dtype(dtype, sh * br * sg * (1.0 + ar * (1.0 - sg)));
            db[m * I + n] = round_dtype(dtype, sh * ar * sg);
        }
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int64_t n = 0; n < I; ++n)
                acc += da[m * I + n] * (double)load_elem(w13, dtype, n * d + c) +
                       db[m * I + n] * (double)load_elem(w13, dtype, (I + n) * d + c);
            store_elem_from_double(dA, dtype, m * d + c, acc);
        }
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t c = 0; c < d; ++c)
        for (int64_t n = 0; n < I; ++n) {
            double acc = 0.0;
            for (int64_t m = 0; m < M; ++m)
                acc += (double)load_elem(dY, dtype, m * d + c) * h[m * I + n];
            store_elem_from_double(dw2, dtype, c * I + n, acc);
        }
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t n = 0; n < I; ++n)
        for (int64_t c = 0; c < d; ++c) {
            double ga = 0.0, gb = 0.0;
            for (int64_t m = 0; m < M; ++m) {
                const double av = (double)load_elem(A, dtype, m * d + c);
                ga += da[m * I + n] * av;
                gb += db[m * I + n] * av;
            }
            store_elem_from_double(dw13, dtype, n * d + c, ga);
            store_elem_from_double(dw13, dtype, (I + n) * d + c, gb);
        }
    free(h);
    free(da);
    free(db);
}

/* gate backward.  g_j = s_j / S with S the sum of the chosen s (j < k):
 * dg_j/ds_m = (delta_jm - g_j) / S, so ds_m = (dgate_m - sum_j dgate_j g_j) / S,
 * with g_j = s_j / S in double; then through the sigmoid, ds/dz = s (1 - s):
 *   dz[t,m] = ds_m * s_m * (1 - s_m)   (fp32), s_m = scores[t, idx[t,m]]. */
void orc_route_backward(int64_t T, int64_t N, int64_t k, const float* scores,
                        const int32_t* idx, const float* dgate, float* dz) {
    for (int64_t t = 0; t < T; ++t) {
        double S = 0.0, gd = 0.0;
        for (int64_t j = 0; j < k; ++j) S += (double)scores[t * N + idx[t * k + j]];
        for (int64_t j = 0; j < k; ++j)
            gd += (double)dgate[t * k + j] * ((double)scores[t * N + idx[t * k + j]] / S);
        for (int64_t j = 0; j < k; ++j) {
            const double s = (double)scores[t * N + idx[t * k + j]];
            dz[t * k + j] = (float)(((double)dgate[t * k + j] - gd) / S * s * (1.0 - s));
        }
    }
}

/* centroid gradient.  z[t,i] = u_t . e_i, so
 *   dcentroids[i, c] = sum over (t, j) with idx[t,j] = i of dz[t,j] * x[t,c]  (fp32);
 * rows of experts nobody chose are zero. */
void orc_centroid_grad(int64_t T, int64_t d, int64_t N, int64_t k, int dtype, const void* x,
                       const int32_t* idx, const float* dz, float* dcentroids) {
    /* one expert per iteration; each column's terms are added in (t, j) order */
#pragma omp parallel
    {
        double* acc = (double*)malloc((size_t)(d + 1) * sizeof(double));
#pragma omp for schedule(static)
        for (int64_t i = 0; i < N; ++i) {
            for (int64_t c = 0; c < d; ++c) acc[c] = 0.0;
            for (int64_t t = 0; t < T; ++t)
                for (int64_t j = 0; j < k; ++j)
                    if (idx[t * k + j] == i)
                        for (int64_t c = 0; c < d; ++c)
                            acc[c] += (double)dz[t * k + j] * (double)load_elem(x, dtype, t * d + c);
            for (int64_t c = 0; c < d; ++c) dcentroids[i * d + c] = (float)acc[c];
        }
        free(acc);
    }
}

/* input gradient.  u_t reaches the output through the residual, the shared
 * expert, each chosen routed expert's rows, and each chosen logit:
 *   dx[t,c] = dout[t,c] + dx_shared[t,c] + sum_j dx_perm[dst[t,j], c]
 *             + sum_j dz[t,j] * centroids[idx[t,j], c]          (rounded to the dtype)
 * dout (no residual) and dx_shared (no shared expert) may be NULL. */
void orc_input_grad(int64_t T, int64_t d, int64_t k, int dtype, const void* dout,
                    const void* dx_shared, const void* dx_perm, const int32_t* dst_row,
                    const float* dz, const int32_t* idx, const float* centroids, void* dx) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t c = 0; c < d; ++c) {
            double acc = 0.0;
            if (dout) acc += (double)load_elem(dout, dtype, t * d + c);
            if (dx_shared) acc += (double)load_elem(dx_shared, dtype, t * d + c);
            for (int64_t j = 0; j < k; ++j) {
                acc += (double)load_elem(dx_perm, dtype, (int64_t)dst_row[t * k + j] * d + c);
                acc += (double)dz[t * k + j] * (double)centroids[(int64_t)idx[t * k + j] * d + c];
            }
            store_elem_from_double(dx, dtype, t * d + c, acc);
        }
}

/* ---------------------------------------------------------------------- */
/* FP8 backward of one SwiGLU expert   [P4k] applied to the backward GEMMs */
/* ---------------------------------------------------------------------- */

/* token-direction tiles: x [M, C] -> codes q [M, C] and scales
 * [ceil(M/128), C]; tile (u, c) is column c of rows 128u .. min(M, 128u+128)-1,
 * quantised like an activation tile (scale = amax/448, codes of x/scale) */
void orc_quant_cols_fp8(int64_t M, int64_t C, int dtype, const void* x, uint8_t* q,
                        float* scales) {
    int64_t nb = (M + 127) / 128;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t u = 0; u < nb; ++u)
        for (int64_t c = 0; c < C; ++c) {
            int64_t r1 = (u + 1) * 128 < M ? (u + 1) * 128 : M;
            float amax = 0.0f;
            for (int64_t r = u * 128; r < r1; ++r) {
                float a = fabsf(load_elem(x, dtype, r * C + c));
                if (a > amax) amax = a;
            }
            float sc = quant_scale(amax);
            scales[u * C + c] = sc;
            for (int64_t r = u * 128; r < r1; ++r)
                q[r * C + c] = quant_one(load_elem(x, dtype, r * C + c), sc);
        }
}

/* The FP8 backward's steps, each on given inputs (the composite below chains
 * them); contractions are sums over 128-blocks of (product of the two scales)
 * times the block's exact sum of decoded code products, in double. */

/* a, b of the FP8 forward (its promoted sums rounded to fp32), kept in bf16:
 * ab [M, 2I] = [a | b] rounded to bf16; h [M, I] = bf16(silu(a) b) of the
 * fp32 a, b. */
void orc_fp8_recompute_ab(int64_t M, int64_t d, int64_t I, const uint8_t* Aq, const float* As,
                          const uint8_t* w13q, const float* w13s, uint16_t* ab, uint16_t* h) {
    double lut[256];
    e4m3_lut(lut);
    const int64_t kd = d / 128;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < I; ++n) {
            double sa = 0.0, sb = 0.0;
            for (int64_t kb = 0; kb < kd; ++kb) {
                double pa = block_dot(Aq + m * d + kb * 128, w13q + n * d + kb * 128, lut);
                double pb = block_dot(Aq + m * d + kb * 128, w13q + (I + n) * d + kb * 128, lut);
                double xs = (double)As[m * kd + kb];
                sa += xs * (double)w13s[(n / 128) * kd + kb] * pa;
                sb += xs * (double)w13s[((I + n) / 128) * kd + kb] * pb;
            }
            double a = (double)(float)sa, b = (double)(float)sb;
            h[m * I + n] = double_to_bf16_bits(a / (1.0 + exp(-a)) * b);
            ab[m * 2 * I + n] = double_to_bf16_bits(a);
            ab[m * 2 * I + I + n] = double_to_bf16_bits(b);
        }
}

/* data gradient through one weight matrix W [K, N] (E4M3 codes, 128x128 block
 * scales ws [K/128, N/128]) of M gradient rows in 1x128 tiles along K:
 * out[m, n] = bf16( sum_k g[m, k] W[k, n] ).  dh = dY W2 (K = d, N = I);
 * dA = [da db] [W1; W3] (K = 2I, N = d). */
void orc_fp8_dgrad(int64_t M, int64_t K, int64_t N, const uint8_t* gq, const float* gs,
                   const uint8_t* wq, const float* ws, uint16_t* out) {
    double lut[256];
    e4m3_lut(lut);
    const int64_t kk = K / 128, kn = N / 128;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t kb = 0; kb < kk; ++kb) {
                double p = 0.0;
                for (int64_t k = kb * 128; k < kb * 128 + 128; ++k)
                    p += lut[gq[m * K + k]] * lut[wq[k * N + n]];
                acc += (double)gs[m * kk + kb] * (double)ws[kb * kn + n / 128] * p;
            }
            out[m * N + n] = double_to_bf16_bits(acc);
        }
}

/* SwiGLU derivative on stored (bf16) values: from dh [M, I] and [a | b]
 * [M, 2I], da = bf16(dh b s (1 + a (1 - s))), db = bf16(dh a s), s = sig(a),
 * into dab [M, 2I] = [da | db]; evaluated in double. */
void orc_swiglu_bwd_bf16(int64_t M, int64_t I, const uint16_t* dh, const uint16_t* ab,
                         uint16_t* dab) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < I; ++n) {
            const double g = (double)bf16_bits_to_float(dh[m * I + n]);
            const double a = (double)bf16_bits_to_float(ab[m * 2 * I + n]);
            const double b = (double)bf16_bits_to_float(ab[m * 2 * I + I + n]);
            const double sg = sigmoid_d(a);
            dab[m * 2 * I + n] = double_to_bf16_bits(g * b * sg * (1.0 + a * (1.0 - sg)));
            dab[m * 2 * I + I + n] = double_to_bf16_bits(g * a * sg);
        }
}

/* weight gradient over M rows in 128x1 row-direction tiles (128 consecutive
 * rows from row 0, the last partial): A codes [M, FA] with scales
 * [ceil(M/128), FA], B codes [M, FB] with scales [ceil(M/128), FB];
 * out[a, b] = bf16( sum_m A[m, a] B[m, b] ).  dW2 = dY^T h; dW13 = [da db]^T X. */
void orc_fp8_wgrad(int64_t M, int64_t FA, int64_t FB, const uint8_t* Aq, const float* As,
                   const uint8_t* Bq, const float* Bs, uint16_t* out) {
    double lut[256];
    e4m3_lut(lut);
    const int64_t nb = (M + 127) / 128;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t a = 0; a < FA; ++a)
        for (int64_t b = 0; b < FB; ++b) {
            double acc = 0.0;
            for (int64_t u = 0; u < nb; ++u) {
                int64_t r1 = (u + 1) * 128 < M ? (u + 1) * 128 : M;
                double p = 0.0;
                for (int64_t m = u * 128; m < r1; ++m) p += lut[Aq[m * FA + a]] * lut[Bq[m * FB + b]];
                acc += (double)As[u * FA + a] * (double)Bs[u * FB + b] * p;
            }
            out[a * FB + b] = double_to_bf16_bits(acc);
        }
}

/* Backward of the FP8 SwiGLU expert over its M rows:
 *  Aq [M,d] codes, As [M,d/128]   the forward's activation tiles (to recompute a, b)
 *  A  [M,d] bf16                  the same rows before quantisation (for dW13)
 *  w13q [2I,d], w13s [2I/128,d/128], w2q [d,I], w2s [d/128,I/128]  forward blocks
 *  dY [M,d] bf16                  gradient of the expert output
 * out dA [M,d], dw13 [2I,d], dw2 [d,I], all bf16 (gradients of the unquantised
 * weights: the block quantisation passes the gradient through).  The steps:
 *   a~, b~, h~ = orc_fp8_recompute_ab
 *   dh    = bf16( dY W2 )            dY in 1x128 row tiles, W2 in its blocks
 *   da, db = orc_swiglu_bwd_bf16(dh, a~, b~)
 *   dA    = bf16( [da db] [W1; W3] ) [da db] in 1x128 row tiles
 *   dw2   = bf16( dY^T h~ )          both in 128x1 row-direction tiles
 *   dw13  = bf16( [da db]^T A )      both in 128x1 row-direction tiles */
void orc_swiglu_ffn_backward_fp8(int64_t M, int64_t d, int64_t I, const uint8_t* Aq,
                                 const float* As, const uint16_t* A, const uint8_t* w13q,
                                 const float* w13s, const uint8_t* w2q, const float* w2s,
                                 const uint16_t* dY, uint16_t* dA, uint16_t* dw13,
                                 uint16_t* dw2) {
    const int64_t kd = d / 128, k2 = 2 * I / 128, nb = (M + 127) / 128;
    const size_t MI = (size_t)(M * I + 1), M2I = (size_t)(2 * M * I + 1);
    uint16_t* h = (uint16_t*)malloc(MI * 2);
    uint16_t* ab = (uint16_t*)malloc(M2I * 2);
    uint16_t* dh = (uint16_t*)malloc(MI * 2);
    uint16_t* dab = (uint16_t*)malloc(M2I * 2);
    orc_fp8_recompute_ab(M, d, I, Aq, As, w13q, w13s, ab, h);
    uint8_t* gq = (uint8_t*)malloc((size_t)(M * d + 1));
    float* gs = (float*)malloc((size_t)(M * kd + 1) * sizeof(float));
    orc_quant_act_fp8(M, d, ORC_BF16, dY, gq, gs);
    orc_fp8_dgrad(M, d, I, gq, gs, w2q, w2s, dh);
    orc_swiglu_bwd_bf16(M, I, dh, ab, dab);
    uint8_t* tq = (uint8_t*)malloc(M2I);
    float* ts = (float*)malloc((size_t)(M * k2 + 1) * sizeof(float));
    orc_quant_act_fp8(M, 2 * I, ORC_BF16, dab, tq, ts);
    orc_fp8_dgrad(M, 2 * I, d, tq, ts, w13q, w13s, dA);
    uint8_t* cg = (uint8_t*)malloc((size_t)(M * d + 1));
    float* cgs = (float*)malloc((size_t)(nb * d + 1) * sizeof(float));
    uint8_t* ch = (uint8_t*)malloc(MI);
    float* chs = (float*)malloc((size_t)(nb * I + 1) * sizeof(float));
    uint8_t* ct = (uint8_t*)malloc(M2I);
    float* cts = (float*)malloc((size_t)(nb * 2 * I + 1) * sizeof(float));
    uint8_t* cx = (uint8_t*)malloc((size_t)(M * d + 1));
    float* cxs = (float*)malloc((size_t)(nb * d + 1) * sizeof(float));
    orc_quant_cols_fp8(M, d, ORC_BF16, dY, cg, cgs);
    orc_quant_cols_fp8(M, I, ORC_BF16, h, ch, chs);
    orc_quant_cols_fp8(M, 2 * I, ORC_BF16, dab, ct, cts);
    orc_quant_cols_fp8(M, d, ORC_BF16, A, cx, cxs);
    orc_fp8_wgrad(M, d, I, cg, cgs, ch, chs, dw2);
    orc_fp8_wgrad(M, 2 * I, d, ct, cts, cx, cxs, dw13);
    free(h); free(ab); free(dh); free(dab); free(gq); free(gs); free(tq); free(ts);
    free(cg); free(cgs); free(ch); free(chs); free(ct); free(cts); free(cx); free(cxs);
}

/* Timing support only (the CPU baseline times the oracle with all host
 * threads and with one): the number of OpenMP threads the next parallel
 * regions use; returns the previous maximum.  n < 1 leaves it unchanged. */
#ifdef _OPENMP
#include <omp.h>
int orc_set_threads(int n) {
    const int prev = omp_get_max_threads();
    if (n >= 1) omp_set_num_threads(n);
    return prev;
}
#else
int orc_set_threads(int n) {  /* a build without OpenMP runs on one thread */
    (void)n;
    return 1;
}
#endif
