// route.hip -- affinity, biased (group-limited) top-k, gates and per-expert
// load for the DeepSeekMoE router.
//
// DeepSeek-V3 report reading guide (xyznot.com/de), "Methode" item 2:
// s_{i,t} = Sigmoid(u_t^T e_i); g'_{i,t} = s_{i,t} when s_{i,t} + b_i is in the
// Topk of {s_{j,t} + b_j}, else 0; g = normalised g'.  The bias only decides
// membership of the Topk.
//
// Two kernels:
//  router_logits: z = x E^T as a fixed-order fp32 FMA chain per output (k
//    ascending from +0), so that the chosen indices are reproducible bit for
//    bit; the chain runs on the VALU (MFMA has no defined summation order).
//    Epilogue: s = fp32(1 / (1 + exp(-(double)z))).
//  router_select: one wavefront per token; keys s+b; optional group limit;
//    k rounds of a wave-wide argmax under the total order (key desc, index
//    asc); gates in double; per-expert load via integer atomics (order-free).
#include "moe_internal.h"

namespace moe {

// ------------------------------------------------------------------ logits

// Tile: TM = 16*TY tokens x 64 experts per 256-thread workgroup; each thread
// owns TY tokens x 4 experts (4*TY independent FMA chains).  BK = 32 hidden
// elements per LDS stage, double buffered, held transposed ([k][token],
// [k][expert]) so each thread reads its tokens and experts as float4s.
// Global loads are 16-byte vectors; FULL = (d % BK == 0) drops every
// per-element bound check, the other instance pads the last stage with zeros
// (an fma with two zero operands leaves a chain unchanged: the chain starts
// at +0 and never holds -0).
constexpr int RL_TN = 64, RL_BK = 32, RL_KG = 2;
static_assert(RL_TN * RL_BK / 256 == 8, "each thread copies 8 centroid values per stage");

// one stage's global loads, held in registers until the stage's FMAs are done
// (x stays in its input type: converting at load time would make the wait
// for the loads come right after issuing them)
template <typename XT, int TY>
struct RlRegs {
    static constexpr int XE = 16 * TY * RL_BK / 256;  // x elements per thread per stage
    static constexpr int XW = XE * (int)sizeof(XT) / 4;  // as 32-bit words
    uint32_t xw[XW];
    float e[8];   // expert tid/4, hidden (tid&3)*8 .. +7
};

template <typename XT, bool FULL, int TY>
__device__ __forceinline__ void rl_load(const XT* __restrict__ x, const float* __restrict__ E,
                                        int64_t T, int64_t d, int64_t N, int64_t t0, int64_t n0,
                                        int64_t k0, int tid, RlRegs<XT, TY>& r) {
    constexpr int XE = RlRegs<XT, TY>::XE, TPT = RL_BK / XE;  // threads per token row
    int64_t t = t0 + tid / TPT;
    if (t >= T) t = T - 1;  // clamp: a valid row, the result is never stored
    const int64_t kx = k0 + XE * (tid % TPT);
    const XT* xrow = x + t * d + kx;
    if (FULL) {
        // XE consecutive elements: one vector load of XE * sizeof(XT) bytes
        __builtin_memcpy(r.xw, xrow, sizeof(r.xw));
    } else {
        XT v[XE];
#pragma unroll
        for (int i = 0; i < XE; ++i) v[i] = kx + i < d ? xrow[i] : XT(0);  // +0 in either type
        __builtin_memcpy(r.xw, v, sizeof(r.xw));
    }
    const int64_t n = n0 + (tid >> 2);
    const int64_t ke = k0 + 8 * (tid & 3);
    if (n < N) {
        const float* erow = E + n * d + ke;
        if (FULL) {
            const float4 a = *(const float4*)erow;
            const float4 b = *(const float4*)(erow + 4);
            r.e[0] = a.x; r.e[1] = a.y; r.e[2] = a.z; r.e[3] = a.w;
            r.e[4] = b.x; r.e[5] = b.y; r.e[6] = b.z; r.e[7] = b.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) r.e[i] = ke + i < d ? erow[i] : 0.0f;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) r.e[i] = 0.0f;
    }
}

template <typename XT, bool FULL, int TY>
__global__ void __launch_bounds__(256) router_logits_kernel(const XT* __restrict__ x,
                                                            const float* __restrict__ E,
                                                            float* __restrict__ s_out,
                                                            int64_t T, int64_t d, int64_t N) {
    constexpr int TM = 16 * TY;
    constexpr int XE = RlRegs<XT, TY>::XE, TPT = RL_BK / XE;
    __shared__ __attribute__((aligned(16))) float xs[2][RL_BK][TM + 4];
    __shared__ __attribute__((aligned(16))) float es[2][RL_BK][RL_TN + 4];
    const int tid = threadIdx.x;
    const int64_t n0 = (int64_t)blockIdx.x * RL_TN;
    const int64_t t0 = (int64_t)blockIdx.y * TM;
    const int ty = tid >> 4;  // 0..15 -> tokens ty*TY .. +TY-1
    const int tx = tid & 15;  // 0..15 -> experts tx*4 .. +3

    float acc[TY][4];
#pragma unroll
    for (int i = 0; i < TY; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

    auto store = [&](int buf, const RlRegs<XT, TY>& r) {
#pragma unroll
        for (int i = 0; i < XE; ++i) {
            float v;
            if constexpr (sizeof(XT) == 2)  // bf16: element i is half i%2 of word i/2
                v = __uint_as_float(i & 1 ? r.xw[i / 2] & 0xffff0000u : r.xw[i / 2] << 16);
            else
                v = __uint_as_float(r.xw[i]);
            xs[buf][XE * (tid % TPT) + i][tid / TPT] = v;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) es[buf][8 * (tid & 3) + i][tid >> 2] = r.e[i];
    };

    RlRegs<XT, TY> r;
    const int64_t nk = cdiv(d, RL_BK);
    rl_load<XT, FULL, TY>(x, E, T, d, N, t0, n0, 0, tid, r);
    store(0, r);
    __syncthreads();

    for (int64_t kb = 0; kb < nk; ++kb) {
        const int buf = kb & 1;
        const bool more = kb + 1 < nk;
        if (more) rl_load<XT, FULL, TY>(x, E, T, d, N, t0, n0, (kb + 1) * RL_BK, tid, r);
        // groups of RL_KG steps, the LDS operands of group g+1 read while group
        // g's FMAs run; a fence per group keeps the compiler from hoisting every
        // read of the stage ahead of the FMAs (it runs out of registers)
        float xv[2][RL_KG][TY];
        float ev[2][RL_KG][4];
        auto ld = [&](int g, int slot) {
#pragma unroll
            for (int kk = 0; kk < RL_KG; ++kk) {
                const int k = g * RL_KG + kk;
#pragma unroll
                for (int i = 0; i < TY; ++i) xv[slot][kk][i] = xs[buf][k][ty * TY + i];
                const float4 eb = *reinterpret_cast<const float4*>(&es[buf][k][tx * 4]);
                ev[slot][kk][0] = eb.x; ev[slot][kk][1] = eb.y;
                ev[slot][kk][2] = eb.z; ev[slot][kk][3] = eb.w;
            }
        };
        ld(0, 0);
#pragma unroll
        for (int g = 0; g < RL_BK / RL_KG; ++g) {
            if (g + 1 < RL_BK / RL_KG) ld(g + 1, (g + 1) & 1);
            // fence: the reads above stay above, the FMAs below (they consume
            // the accumulators this empty asm passes through) stay below
#pragma unroll
            for (int i = 0; i < TY; ++i)
                asm volatile("" : "+v"(acc[i][0]), "+v"(acc[i][1]), "+v"(acc[i][2]), "+v"(acc[i][3])
                             :: "memory");
#pragma unroll
            for (int kk = 0; kk < RL_KG; ++kk)
#pragma unroll
                for (int i = 0; i < TY; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_fmaf(xv[g & 1][kk][i], ev[g & 1][kk][j], acc[i][j]);
        }
        if (more) store(buf ^ 1, r);
        __syncthreads();
    }

    // epilogue: affinity s = Sigmoid(z), evaluated in double, rounded once
    // (one value at a time: the double-precision exp unrolled over all
    // outputs would claim registers the main loop then goes without)
#pragma unroll 1
    for (int i = 0; i < TY; ++i) {
        const int64_t t = t0 + ty * TY + i;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + tx * 4 + j;
            if (n < N) s_out[t * N + n] = (float)(1.0 / (1.0 + exp(-(double)acc[i][j])));
        }
    }
}

// Small batches: the tiled kernel above would leave most CUs idle (each of
// its threads runs 4*TY chains), so here every lane runs one chain.  A
// workgroup of 8 waves covers 8 tokens x 64 experts: wave w owns token t0+w,
// lane l expert n0+l.  The centroid tile [64 experts][RR_BK] is staged in LDS
// once per workgroup and read by lane l as float4s along k (rows padded by 4
// floats, so the 16 lanes served together hit distinct banks); the token tile
// [8][RR_BK] is read by all lanes of a wave at one address.  Same chain as
// above: k ascending from +0, fma(x, e, acc); zero padding past d.
constexpr int RR_BK = 256, RR_TM = 8;
constexpr int RR_EQ = RL_TN * RR_BK / 4 / 512;  // centroid float4s per thread and stage
constexpr int RR_XE = RR_TM * RR_BK / 512;       // token elements per thread and stage

template <typename XT, bool FULL>
__global__ void __launch_bounds__(512) router_logits_rows_kernel(const XT* __restrict__ x,
                                                                const float* __restrict__ E,
                                                                float* __restrict__ s_out,
                                                                int64_t T, int64_t d, int64_t N) {
    __shared__ __attribute__((aligned(16))) float es[2][RL_TN][RR_BK + 4];
    __shared__ __attribute__((aligned(16))) float xs[2][RR_TM][RR_BK];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t n0 = (int64_t)blockIdx.x * RL_TN, t0 = (int64_t)blockIdx.y * RR_TM;

    // stage loads, held in registers while the previous stage is multiplied:
    // centroids 64 rows x RR_BK/4 float4s, tokens 8 rows x RR_BK elements
    constexpr int Q4 = RR_BK / 4;  // float4s per centroid row
    float4 er[RR_EQ];
    float xr[RR_XE];
    auto load = [&](int64_t k0) {
#pragma unroll
        for (int c = 0; c < RR_EQ; ++c) {
            const int q = tid + 512 * c, row = q / Q4, c4 = q % Q4;
            const int64_t n = n0 + row, k = k0 + 4 * c4;
            float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (n < N) {
                const float* e = E + n * d + k;
                if (FULL) {
                    v = *(const float4*)e;
                } else {
                    v.x = k < d ? e[0] : 0.0f;
                    v.y = k + 1 < d ? e[1] : 0.0f;
                    v.z = k + 2 < d ? e[2] : 0.0f;
                    v.w = k + 3 < d ? e[3] : 0.0f;
                }
            }
            er[c] = v;
        }
        {
            constexpr int TPR = RR_BK / RR_XE;  // threads per token row
            int64_t t = t0 + tid / TPR;
            if (t >= T) t = T - 1;  // clamp: a valid row, the result is never stored
            const int64_t k = k0 + RR_XE * (tid % TPR);
            const XT* xp = x + t * d + k;
#pragma unroll
            for (int i = 0; i < RR_XE; ++i) {
                float v = 0.0f;
                if (FULL || k + i < d) {
                    if constexpr (sizeof(XT) == 2)
                        v = __uint_as_float((uint32_t)xp[i] << 16);
                    else
                        v = (float)xp[i];
                }
                xr[i] = v;
            }
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int c = 0; c < RR_EQ; ++c) {
            const int q = tid + 512 * c;
            *(float4*)&es[buf][q / Q4][4 * (q % Q4)] = er[c];
        }
        constexpr int TPR = RR_BK / RR_XE;
        float* xp = &xs[buf][tid / TPR][RR_XE * (tid % TPR)];
#pragma unroll
        for (int i = 0; i < RR_XE; i += 4) *(float4*)(xp + i) = make_float4(xr[i], xr[i + 1], xr[i + 2], xr[i + 3]);
    };

    float acc = 0.0f;
    const int64_t nk = cdiv(d, RR_BK);
    load(0);
    store(0);
    __syncthreads();
    for (int64_t kb = 0; kb < nk; ++kb) {
        const int buf = kb & 1;
        const bool more = kb + 1 < nk;
        if (more) load((kb + 1) * RR_BK);
        const float* erow = &es[buf][lane][0];
        const float* xrow = &xs[buf][wave][0];
#pragma unroll 8
        for (int k = 0; k < RR_BK; k += 4) {
            const float4 ev = *(const float4*)(erow + k);
            const float4 xv = *(const float4*)(xrow + k);
            acc = __builtin_fmaf(xv.x, ev.x, acc);
            acc = __builtin_fmaf(xv.y, ev.y, acc);
            acc = __builtin_fmaf(xv.z, ev.z, acc);
            acc = __builtin_fmaf(xv.w, ev.w, acc);
        }
        if (more) store(buf ^ 1);
        __syncthreads();
    }
    const int64_t t = t0 + wave, n = n0 + lane;
    if (t < T && n < N) s_out[t * N + n] = (float)(1.0 / (1.0 + exp(-(double)acc)));
}

// ------------------------------------------------------------------ select

// "a beats b": larger key, or equal key and lower index
__device__ __forceinline__ bool beats(float ra, int ia, float rb, int ib) {
    return ra > rb || (ra == rb && ia < ib);
}

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int m) {
    return __shfl_xor(v, m, 64);
}

// Each lane holds up to SEL_RK keys of one token: experts lane + 64*r
// (SEL_RK = 16 covers N <= 1024).
template <int SEL_RK>
__global__ void __launch_bounds__(256) router_select_kernel(
    const float* __restrict__ s, const float* __restrict__ bias, int32_t* __restrict__ idx_out,
    float* __restrict__ gate_out, int32_t* __restrict__ counts, int64_t T, int N, int k, int G,
    int TG) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (t >= T) return;
    const float* st = s + t * N;

    float sv[SEL_RK], rv[SEL_RK];
    bool ok[SEL_RK];
#pragma unroll
    for (int r = 0; r < SEL_RK; ++r) {
        const int i = lane + 64 * r;
        if (i < N) {
            sv[r] = st[i];
            float key = sv[r] + bias[i];
            if (key == 0.0f) key = 0.0f;  // -0 -> +0
            rv[r] = key;
            ok[r] = true;
        } else {
            sv[r] = 0.0f;
            rv[r] = -__builtin_inff();
            ok[r] = false;
        }
    }

    if (G > 1) {
        // group g = experts [g*gs, (g+1)*gs); score = sum of its two best keys;
        // lane g ends up holding group g's score
        const int gs = N / G;
        float my_gscore = -__builtin_inff();
        for (int g = 0; g < G; ++g) {
            float r1 = -__builtin_inff(), r2 = -__builtin_inff();
            int i1 = 0x7fffffff, i2 = 0x7fffffff;
#pragma unroll
            for (int r = 0; r < SEL_RK; ++r) {
                const int i = lane + 64 * r;
                if (!ok[r] || i / gs != g) continue;
                if (beats(rv[r], i, r1, i1)) {
                    r2 = r1; i2 = i1; r1 = rv[r]; i1 = i;
                } else if (beats(rv[r], i, r2, i2)) {
                    r2 = rv[r]; i2 = i;
                }
            }
#pragma unroll
            for (int m = 1; m < 64; m <<= 1) {
                const float p1 = shfl_xor(r1, m), p2 = shfl_xor(r2, m);
                const int q1 = shfl_xor(i1, m), q2 = shfl_xor(i2, m);
                // merge two sorted pairs, keep the best two
                if (beats(p1, q1, r1, i1)) {
                    // partner's first wins; second is the better of (r1, p2)
                    if (beats(r1, i1, p2, q2)) { r2 = r1; i2 = i1; } else { r2 = p2; i2 = q2; }
                    r1 = p1; i1 = q1;
                } else {
                    if (beats(p1, q1, r2, i2)) { r2 = p1; i2 = q1; }
                }
            }
            float sc = r1 + r2;
            if (sc == 0.0f) sc = 0.0f;
            if (lane == g) my_gscore = sc;
        }
        // keep the TG best groups: TG rounds of argmax over lanes 0..G-1
        bool kept = false;
        bool cand = lane < G;
        for (int p = 0; p < TG; ++p) {
            float bv = cand ? my_gscore : -__builtin_inff();
            int bi = cand ? lane : 0x7fffffff;
#pragma unroll
            for (int m = 1; m < 64; m <<= 1) {
                const float ov = shfl_xor(bv, m);
                const int oi = shfl_xor(bi, m);
                if (beats(ov, oi, bv, bi)) { bv = ov; bi = oi; }
            }
            if (lane == bi) { kept = true; cand = false; }
        }
        // experts outside the kept groups are not eligible
#pragma unroll
        for (int r = 0; r < SEL_RK; ++r) {
            const int i = lane + 64 * r;
            const int g = ok[r] ? i / gs : 0;
            const bool gk = __shfl(kept, g, 64);
            if (ok[r] && !gk) ok[r] = false;
        }
    }

    // k rounds of wave argmax; lane j records the j-th winner
    int my_idx = 0;
    float my_s = 0.0f;
    for (int j = 0; j < k; ++j) {
        float bv = -__builtin_inff();
        int bi = 0x7fffffff;
        float bs = 0.0f;
#pragma unroll
        for (int r = 0; r < SEL_RK; ++r) {
            const int i = lane + 64 * r;
            if (ok[r] && beats(rv[r], i, bv, bi)) { bv = rv[r]; bi = i; bs = sv[r]; }
        }
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
            const float ov = shfl_xor(bv, m);
            const int oi = shfl_xor(bi, m);
            const float os = shfl_xor(bs, m);
            if (beats(ov, oi, bv, bi)) { bv = ov; bi = oi; bs = os; }
        }
        // the owner lane drops the winner from its candidates
#pragma unroll
        for (int r = 0; r < SEL_RK; ++r)
            if (lane + 64 * r == bi) ok[r] = false;
        if (lane == j) { my_idx = bi; my_s = bs; }
    }
    // gates: g_j = s_j / sum_j' s_j', the sum in double in selection order
    double S = 0.0;
    for (int j = 0; j < k; ++j) S += (double)__shfl(my_s, j, 64);
    if (lane < k) {
        idx_out[t * k + lane] = my_idx;
        gate_out[t * k + lane] = (float)((double)my_s / S);
        atomicAdd(&counts[my_idx], 1);
    }
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// ------------------------------------------------------------------ launch

template <int TY>
static void launch_logits(int32_t act_dtype, bool full, const void* x, const float* centroids,
                          float* scores, int64_t T, int64_t d, int64_t N, hipStream_t st) {
    const dim3 g1((unsigned)cdiv(N, RL_TN), (unsigned)cdiv(T, 16 * TY));
    if (act_dtype == MOE_BF16) {
        if (full)
            router_logits_kernel<uint16_t, true, TY><<<g1, 256, 0, st>>>(
                (const uint16_t*)x, centroids, scores, T, d, N);
        else
            router_logits_kernel<uint16_t, false, TY><<<g1, 256, 0, st>>>(
                (const uint16_t*)x, centroids, scores, T, d, N);
    } else {
        if (full)
            router_logits_kernel<float, true, TY><<<g1, 256, 0, st>>>((const float*)x, centroids,
                                                                      scores, T, d, N);
        else
            router_logits_kernel<float, false, TY><<<g1, 256, 0, st>>>(
                (const float*)x, centroids, scores, T, d, N);
    }
}

hipError_t launch_route(const moe_cfg& c, const void* x, const float* centroids,
                        const float* bias, float* scores, int32_t* idx, float* gate,
                        int32_t* counts, hipStream_t st) {
    const int64_t T = c.tokens, d = c.hidden, N = c.n_experts;
    if (T == 0) {
        fill_i32_kernel<<<dim3((unsigned)cdiv(N, 256)), 256, 0, st>>>(counts, N, 0);
        return hipGetLastError();
    }
    // Each (token, expert) logit is one serial chain over d, so the tile per
    // thread trades chains (latency hiding) against workgroups (parallelism):
    // 4 tokens per thread for large batches (two workgroups per CU at
    // 8192 x 256), fewer for smaller ones, and one chain per lane for
    // decode-sized batches.
    const bool full = d % RL_BK == 0;
    if (cdiv(N, RL_TN) * cdiv(T, 64) < 64) {
        // decode-sized batch: one chain per lane
        const dim3 g1((unsigned)cdiv(N, RL_TN), (unsigned)cdiv(T, RR_TM));
        const bool fr = d % RR_BK == 0;
        if (c.act_dtype == MOE_BF16) {
            if (fr)
                router_logits_rows_kernel<uint16_t, true><<<g1, 512, 0, st>>>(
                    (const uint16_t*)x, centroids, scores, T, d, N);
            else
                router_logits_rows_kernel<uint16_t, false><<<g1, 512, 0, st>>>(
                    (const uint16_t*)x, centroids, scores, T, d, N);
        } else {
            if (fr)
                router_logits_rows_kernel<float, true><<<g1, 512, 0, st>>>(
                    (const float*)x, centroids, scores, T, d, N);
            else
                router_logits_rows_kernel<float, false><<<g1, 512, 0, st>>>(
                    (const float*)x, centroids, scores, T, d, N);
        }
    } else if (cdiv(N, RL_TN) * cdiv(T, 16 * 4) >= 384)
        launch_logits<4>(c.act_dtype, full, x, centroids, scores, T, d, N, st);
    else if (cdiv(N, RL_TN) * cdiv(T, 16 * 2) >= 192)
        launch_logits<2>(c.act_dtype, full, x, centroids, scores, T, d, N, st);
    else
        launch_logits<1>(c.act_dtype, full, x, centroids, scores, T, d, N, st);
    fill_i32_kernel<<<dim3((unsigned)cdiv(N, 256)), 256, 0, st>>>(counts, N, 0);
    const int G = c.n_group > 1 ? (int)c.n_group : 1;
    const dim3 gs((unsigned)cdiv(T, 4));
    const int K = (int)c.top_k, TG = (int)c.topk_group, NN = (int)N;
    if (N <= 64)
        router_select_kernel<1><<<gs, 256, 0, st>>>(scores, bias, idx, gate, counts, T, NN, K, G, TG);
    else if (N <= 128)
        router_select_kernel<2><<<gs, 256, 0, st>>>(scores, bias, idx, gate, counts, T, NN, K, G, TG);
    else if (N <= 256)
        router_select_kernel<4><<<gs, 256, 0, st>>>(scores, bias, idx, gate, counts, T, NN, K, G, TG);
    else if (N <= 512)
        router_select_kernel<8><<<gs, 256, 0, st>>>(scores, bias, idx, gate, counts, T, NN, K, G, TG);
    else
        router_select_kernel<16><<<gs, 256, 0, st>>>(scores, bias, idx, gate, counts, T, NN, K, G, TG);
    return hipGetLastError();
}

}  // namespace moe
