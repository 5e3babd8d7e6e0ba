// misc.hip -- combine (un-permute), end-of-step bias update, the
// sequence-wise balance loss, and the FP8 weight block quantiser used as
// preparation.
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------- combine
// h'_t = u_t + y_shared[t] + sum_j g_{t,j} * y_perm[dst_row[t,j]]
// (DeepSeek-V3 report reading guide, xyznot.com/de, "Methode" item 2).
// A gather: each output row is produced by one block reading its k rows, so no
// atomics and a fixed fp32 summation order (residual, shared, slots 0..k-1).
// One thread per 16-byte vector of the row, up to 1024 (V3 shape: 896).

template <bool BF16>
__global__ void __launch_bounds__(1024) combine_kernel(const uint4* __restrict__ x,
                                                      const uint4* __restrict__ ys,
                                                      const uint4* __restrict__ yp,
                                                      const float* __restrict__ gate,
                                                      const int32_t* __restrict__ dst_row,
                                                      uint4* __restrict__ out, int k,
                                                      int64_t row_vecs) {
    __shared__ int32_t rows[64];
    __shared__ float g[64];
    const int64_t t = blockIdx.x;
    if (threadIdx.x < k) {
        rows[threadIdx.x] = dst_row[t * k + threadIdx.x];
        g[threadIdx.x] = gate[t * k + threadIdx.x];
    }
    __syncthreads();
    constexpr int E = BF16 ? 8 : 4;
    for (int64_t v = threadIdx.x; v < row_vecs; v += blockDim.x) {
        float acc[E];
#pragma unroll
        for (int i = 0; i < E; ++i) acc[i] = 0.0f;
        auto add = [&](const uint4 q, float s) {
            const uint32_t w[4] = {q.x, q.y, q.z, q.w};
            if constexpr (BF16) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[2 * i] = __builtin_fmaf(s, __uint_as_float(w[i] << 16), acc[2 * i]);
                    acc[2 * i + 1] =
                        __builtin_fmaf(s, __uint_as_float(w[i] & 0xffff0000u), acc[2 * i + 1]);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(s, __uint_as_float(w[i]), acc[i]);
            }
        };
        if (x) add(x[t * row_vecs + v], 1.0f);
        if (ys) add(ys[t * row_vecs + v], 1.0f);
        // the routed rows are read once and the output written once: both
        // bypass the caches' retention (non-temporal), which the measured
        // rate favours; x and y_shared come from earlier stages and are
        // left to the caches
        for (int j = 0; j < k; ++j) {
            const u32x4_t q =
                __builtin_nontemporal_load((const u32x4_t*)(yp + (int64_t)rows[j] * row_vecs + v));
            add(make_uint4(q.x, q.y, q.z, q.w), g[j]);
        }
        uint4 o;
        if constexpr (BF16) {
            o.x = pack_bf16x2(acc[0], acc[1]);
            o.y = pack_bf16x2(acc[2], acc[3]);
            o.z = pack_bf16x2(acc[4], acc[5]);
            o.w = pack_bf16x2(acc[6], acc[7]);
        } else {
            o.x = __float_as_uint(acc[0]);
            o.y = __float_as_uint(acc[1]);
            o.z = __float_as_uint(acc[2]);
            o.w = __float_as_uint(acc[3]);
        }
        __builtin_nontemporal_store(u32x4_t{o.x, o.y, o.z, o.w}, (u32x4_t*)(out + t * row_vecs + v));
    }
}

hipError_t launch_combine(const moe_cfg& c, const void* x, const void* y_shared,
                          const void* y_perm, const float* gate, const int32_t* dst_row,
                          void* out, hipStream_t st) {
    const int64_t T = c.tokens;
    if (T == 0) return hipSuccess;
    const int64_t esz = c.act_dtype == MOE_BF16 ? 2 : 4;
    const int64_t row_vecs = c.hidden * esz / 16;
    const int threads = (int)(row_vecs >= 1024 ? 1024 : (row_vecs + 63) / 64 * 64);
    if (c.act_dtype == MOE_BF16)
        combine_kernel<true><<<dim3((unsigned)T), threads, 0, st>>>(
            (const uint4*)x, (const uint4*)y_shared, (const uint4*)y_perm, gate, dst_row,
            (uint4*)out, (int)c.top_k, row_vecs);
    else
        combine_kernel<false><<<dim3((unsigned)T), threads, 0, st>>>(
            (const uint4*)x, (const uint4*)y_shared, (const uint4*)y_perm, gate, dst_row,
            (uint4*)out, (int)c.top_k, row_vecs);
    return hipGetLastError();
}

// ---------------------------------------------------------------- bias update
// End-of-step rule (reading guide "Methode" item 2; singularity-lens formula
// paragraph: b_i += gamma * sign(mean_load - load_i)).  Overload is decided
// exactly in integers: counts[i] * N versus T*k.

__global__ void bias_update_kernel(const int32_t* __restrict__ counts, float gamma,
                                   float* __restrict__ bias, int64_t N, int64_t TK) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= N) return;
    const int64_t lhs = (int64_t)counts[i] * N;
    const float b = bias[i];
    if (lhs > TK)
        bias[i] = b - gamma;
    else if (lhs < TK)
        bias[i] = b + gamma;
}

hipError_t launch_bias_update(int64_t N, int64_t TK, const int32_t* counts, float gamma,
                              float* bias, hipStream_t st) {
    bias_update_kernel<<<dim3((unsigned)cdiv(N, 256)), 256, 0, st>>>(counts, gamma, bias, N, TK);
    return hipGetLastError();
}

// ---------------------------------------------------------------- balance loss
// Sequence-wise balance loss (reading guide "Methode" item 2, last sentence:
// a minimal sequence-wise balance loss, alpha = 0.0001, beside the bias rule;
// no formula on the pages).  Reading: per sequence b of S consecutive tokens,
//   loss[b] = alpha * sum_i f_i P_i,  f_i = N/(kS) * load_i,
//   P_i = 1/S * sum_t s_{i,t} / sum_j s_{j,t}.
// Two launches, no atomics on floating values, so the result is the same bits
// on every run:
//   partial: block (b, c) takes tokens c*64 .. c*64+63 of sequence b; each
//     wave walks 16 of them, four at a time (all four rows' loads in flight
//     together), lane l holding experts l, l+64, ...; a token's row sum is a
//     butterfly over the wave (every lane ends with the same double); the four
//     waves' sums of s/row are added in wave order and stored as
//     part[b][c][i] (double), the chunk's load of each expert (an LDS integer
//     histogram of its idx entries) as cnt[b][c][i];
//   final: one block of 1024 threads per sequence; thread (g, i) adds the
//     chunks c = g, g+4, ... of expert i, the four groups are added in group
//     order, then f_i P_i goes through a fixed-shape tree.  Everything in
//     double; one rounding to fp32.
constexpr int SBL_CH = 64;   // tokens per partial block
constexpr int SBL_TB = 4;    // tokens per wave in flight together
constexpr int SBL_MAXN = 1024;

template <int Q>  // Q = cdiv(N, 64) expert slots per lane
__global__ void __launch_bounds__(256) seq_balance_partial_kernel(const float* __restrict__ s,
                                                                  const int32_t* __restrict__ idx,
                                                                  int64_t N, int64_t k, int64_t S,
                                                                  int cps, double* __restrict__ part,
                                                                  int32_t* __restrict__ cnt) {
    __shared__ double wsum[4][SBL_MAXN];
    __shared__ int32_t hist[SBL_MAXN];
    const int64_t b = blockIdx.x / cps;
    const int c = blockIdx.x % cps;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t t0 = (int64_t)c * SBL_CH;
    const int64_t t_end = S < t0 + SBL_CH ? S : t0 + SBL_CH;
    for (int64_t i = threadIdx.x; i < N; i += 256) hist[i] = 0;
    __syncthreads();
    // the chunk's idx entries (token-major, so the chunk is one contiguous run)
    const int32_t* ib = idx + (b * S + t0) * k;
    for (int64_t p = threadIdx.x; p < (t_end - t0) * k; p += 256) {
        const int32_t e = ib[p];
        if (e >= 0 && e < N) atomicAdd(&hist[e], 1);
    }
    double p[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) p[q] = 0.0;
    // wave w takes tokens t0 + 16w .. t0 + 16w + 15, four at a time
    for (int64_t tb = t0 + wave * (SBL_CH / 4); tb < t0 + (wave + 1) * (SBL_CH / 4) && tb < t_end;
         tb += SBL_TB) {
        float v[SBL_TB][Q];
        double r[SBL_TB];
#pragma unroll
        for (int u = 0; u < SBL_TB; ++u) {
            const float* row = s + (b * S + tb + u) * N;
            const bool tok = tb + u < t_end;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int64_t i = q * 64 + lane;
                v[u][q] = tok && i < N ? row[i] : 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < SBL_TB; ++u) {
            r[u] = 0.0;
#pragma unroll
            for (int q = 0; q < Q; ++q) r[u] += (double)v[u][q];
        }
#pragma unroll
        for (int m = 1; m < 64; m <<= 1)
#pragma unroll
            for (int u = 0; u < SBL_TB; ++u) r[u] += __shfl_xor(r[u], m, 64);
#pragma unroll
        for (int u = 0; u < SBL_TB; ++u)
            if (tb + u < t_end)
#pragma unroll
                for (int q = 0; q < Q; ++q)
                    if (q * 64 + lane < N) p[q] += (double)v[u][q] / r[u];
    }
#pragma unroll
    for (int q = 0; q < Q; ++q)
        if (q * 64 + lane < N) wsum[wave][q * 64 + lane] = p[q];
    __syncthreads();
    for (int64_t i = threadIdx.x; i < N; i += 256) {
        part[(int64_t)blockIdx.x * N + i] = ((wsum[0][i] + wsum[1][i]) + wsum[2][i]) + wsum[3][i];
        cnt[(int64_t)blockIdx.x * N + i] = hist[i];
    }
}

__global__ void __launch_bounds__(1024) seq_balance_final_kernel(const double* __restrict__ part,
                                                                 const int32_t* __restrict__ cnt,
                                                                 int64_t N, int64_t k, int64_t S,
                                                                 int cps, float alpha,
                                                                 float* __restrict__ loss) {
    __shared__ double gp[4][256];
    __shared__ int64_t gc[4][256];
    __shared__ double red[256];
    const int64_t b = blockIdx.x;
    const int g = threadIdx.x >> 8, il = threadIdx.x & 255;
    const double fscale = (double)N / ((double)k * (double)S);
    double acc = 0.0;  // threads of group 0: f_i P_i over their experts
    for (int64_t i0 = 0; i0 < N; i0 += 256) {
        const int64_t i = i0 + il;
        double P = 0.0;
        int64_t n = 0;
        if (i < N) {
            const double* pp = part + b * cps * N + i;
            const int32_t* cp = cnt + b * cps * N + i;
#pragma unroll 4
            for (int c = g; c < cps; c += 4) {
                P += pp[(int64_t)c * N];
                n += cp[(int64_t)c * N];
            }
        }
        gp[g][il] = P;
        gc[g][il] = n;
        __syncthreads();
        if (g == 0 && i < N) {
            const double Pi = ((gp[0][il] + gp[1][il]) + gp[2][il]) + gp[3][il];
            const int64_t ni = gc[0][il] + gc[1][il] + gc[2][il] + gc[3][il];
            acc += fscale * (double)ni * (Pi / (double)S);
        }
        __syncthreads();
    }
    if (g == 0) red[il] = acc;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) loss[b] = (float)((double)alpha * red[0]);
}

size_t seq_balance_workspace_bytes(int64_t T, int64_t N, int64_t S) {
    if (S <= 0 || T <= 0) return 0;
    const int64_t n = (T / S) * cdiv(S, SBL_CH) * N;
    return (size_t)(n * 8 + ((n * 4 + 255) & ~(int64_t)255));
}

hipError_t launch_seq_balance_loss(int64_t T, int64_t N, int64_t k, int64_t S, float alpha,
                                   const float* scores, const int32_t* idx, float* loss,
                                   void* ws, hipStream_t st) {
    const int64_t B = T / S;
    const int cps = (int)cdiv(S, SBL_CH);
    double* part = (double*)ws;
    int32_t* cnt = (int32_t*)(part + B * cps * N);
    const dim3 grid((unsigned)(B * cps));
    const int q = (int)cdiv(N, 64);
    if (q <= 1)
        seq_balance_partial_kernel<1><<<grid, 256, 0, st>>>(scores, idx, N, k, S, cps, part, cnt);
    else if (q <= 2)
        seq_balance_partial_kernel<2><<<grid, 256, 0, st>>>(scores, idx, N, k, S, cps, part, cnt);
    else if (q <= 4)
        seq_balance_partial_kernel<4><<<grid, 256, 0, st>>>(scores, idx, N, k, S, cps, part, cnt);
    else if (q <= 8)
        seq_balance_partial_kernel<8><<<grid, 256, 0, st>>>(scores, idx, N, k, S, cps, part, cnt);
    else
        seq_balance_partial_kernel<16><<<grid, 256, 0, st>>>(scores, idx, N, k, S, cps, part, cnt);
    seq_balance_final_kernel<<<dim3((unsigned)B), 1024, 0, st>>>(part, cnt, N, k, S, cps, alpha,
                                                                loss);
    return hipGetLastError();
}

// ---------------------------------------------------------------- weight FP8
// One 256-thread block per 128x128 block (reading guide "Kernideen", FP8
// bullet: block-wise weight scaling): amax -> scale = amax/448 -> E4M3 codes.

__global__ void __launch_bounds__(256) quant_weight_kernel(const uint4* __restrict__ w,
                                                           uint2* __restrict__ q,
                                                           float* __restrict__ s, int64_t rows,
                                                           int64_t cols) {
    __shared__ float sh[4];
    const int64_t br = rows / 128, bc = cols / 128;
    const int64_t blk = blockIdx.x;
    const int64_t mat = blk / (br * bc), rb = (blk / bc) % br, cb = blk % bc;
    const int64_t vec_cols = cols / 8;
    // 128 rows x 16 vectors of 8 bf16; thread handles 8 of the 2048 vectors
    uint4 v[8];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = threadIdx.x + 256 * i;
        const int64_t r = rb * 128 + (c >> 4);
        const int64_t vc = cb * 16 + (c & 15);
        v[i] = w[(mat * rows + r) * vec_cols + vc];
        const uint32_t ww[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            amax = fmaxf(amax, fabsf(__uint_as_float(ww[j] << 16)));
            amax = fmaxf(amax, fabsf(__uint_as_float(ww[j] & 0xffff0000u)));
        }
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
    const float scale = amax / 448.0f;
    if (threadIdx.x == 0) s[blk] = scale;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = threadIdx.x + 256 * i;
        const int64_t r = rb * 128 + (c >> 4);
        const int64_t vc = cb * 16 + (c & 15);
        const uint32_t ww[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            lo |= quant_e4m3(__uint_as_float(ww[j] << 16), scale) << (16 * j);
            lo |= quant_e4m3(__uint_as_float(ww[j] & 0xffff0000u), scale) << (16 * j + 8);
            hi |= quant_e4m3(__uint_as_float(ww[2 + j] << 16), scale) << (16 * j);
            hi |= quant_e4m3(__uint_as_float(ww[2 + j] & 0xffff0000u), scale) << (16 * j + 8);
        }
        q[(mat * rows + r) * vec_cols + vc] = make_uint2(lo, hi);
    }
}

// The E4M3 quantisation step on given fp32 values, both ways the kernels
// perform it: c4 as the FP8 gate/up epilogue does (IEEE quotient v/scale,
// clamp to +-448, four values per two converter instructions) and c1 as the
// activation and weight quantisers do (quant_e4m3, one value per converter
// instruction).  Thread i handles values 4i .. 4i+3 (zero-padded past n).
__global__ void __launch_bounds__(256) e4m3_inspect_kernel(const float* __restrict__ v, int64_t n,
                                                           float scale, uint8_t* __restrict__ c4,
                                                           uint8_t* __restrict__ c1) {
    const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i >= n) return;
    float t[4], x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        x[j] = i + j < n ? v[i + j] : 0.0f;
        t[j] = scale > 0.0f ? fminf(fmaxf(x[j] / scale, -448.0f), 448.0f) : 0.0f;
    }
    const uint32_t q = e4m3_encode4(t[0], t[1], t[2], t[3]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (i + j < n) {
            c4[i + j] = (uint8_t)(q >> (8 * j));
            c1[i + j] = (uint8_t)quant_e4m3(x[j], scale);
        }
}

hipError_t launch_e4m3_inspect(const float* v, int64_t n, float scale, uint8_t* c4, uint8_t* c1,
                               hipStream_t st) {
    if (n == 0) return hipSuccess;
    e4m3_inspect_kernel<<<dim3((unsigned)cdiv(cdiv(n, 4), 256)), 256, 0, st>>>(v, n, scale, c4,
                                                                              c1);
    return hipGetLastError();
}

hipError_t launch_quantize_weights(int64_t n_mats, int64_t rows, int64_t cols, const void* w,
                                   uint8_t* q, float* s, hipStream_t st) {
    const int64_t nblk = n_mats * (rows / 128) * (cols / 128);
    if (nblk == 0) return hipSuccess;
    quant_weight_kernel<<<dim3((unsigned)nblk), 256, 0, st>>>((const uint4*)w, (uint2*)q, s, rows,
                                                              cols);
    return hipGetLastError();
}

}  // namespace moe
