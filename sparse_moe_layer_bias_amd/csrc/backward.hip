// backward.hip -- the layer's backward outside the expert GEMMs: combine,
// gate normalisation and sigmoid, centroid gradient, and the assembly of the
// input gradient.
//
// Layer (DeepSeek-V3 report reading guide, xyznot.com/de, "Methode" item 2):
//   h'_t = u_t + FFN^(s)(u_t) + sum_j g_{t,j} FFN^(r)_{idx_j}(u_t),
//   s_{i,t} = sigmoid(u_t^T e_i), g_{t,j} = s_{t,idx_j} / sum_j' s_{t,idx_j'}.
// The selection idx is piecewise constant and the balancing bias enters only
// the selection key, so neither carries a gradient.  Every kernel here is a
// gather with a fixed summation order (no atomics): results are bitwise
// deterministic.
#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ void unpack8(const uint4 q, float* f) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

// ---------------------------------------------------------------- combine
// dy_perm[dst[t,j]] = g_{t,j} dout[t] (rounded to the storage dtype) and
// dgate[t,j] = dout[t] . y_perm[dst[t,j]] (fp32).  One block per token, one
// thread per 16-byte vector of the row; the dot product is summed per thread
// (its vectors in order), then over the wave by a fixed butterfly, then over
// the waves in order.
template <bool BF16>
__global__ void __launch_bounds__(1024) combine_backward_kernel(
    const uint4* __restrict__ dout, const uint4* __restrict__ yp, const float* __restrict__ gate,
    const int32_t* __restrict__ dst_row, uint4* __restrict__ dyp, float* __restrict__ dgate,
    int k, int64_t row_vecs) {
    __shared__ int32_t rows[64];
    __shared__ float g[64];
    __shared__ float part[64][16];
    const int64_t t = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    if (threadIdx.x < k) {
        rows[threadIdx.x] = dst_row[t * k + threadIdx.x];
        g[threadIdx.x] = gate[t * k + threadIdx.x];
    }
    __syncthreads();
    constexpr int E = BF16 ? 8 : 4;
    for (int j = 0; j < k; ++j) {
        const int64_t row = rows[j];
        const float gj = g[j];
        float dot = 0.0f;
        for (int64_t v = threadIdx.x; v < row_vecs; v += blockDim.x) {
            const uint4 qd = dout[t * row_vecs + v];
            const uint4 qy = yp[row * row_vecs + v];
            float fd[8], fy[8];
            uint4 o;
            if constexpr (BF16) {
                unpack8(qd, fd);
                unpack8(qy, fy);
                o.x = pack_bf16x2(gj * fd[0], gj * fd[1]);
                o.y = pack_bf16x2(gj * fd[2], gj * fd[3]);
                o.z = pack_bf16x2(gj * fd[4], gj * fd[5]);
                o.w = pack_bf16x2(gj * fd[6], gj * fd[7]);
            } else {
                const uint32_t wd[4] = {qd.x, qd.y, qd.z, qd.w}, wy[4] = {qy.x, qy.y, qy.z, qy.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    fd[i] = __uint_as_float(wd[i]);
                    fy[i] = __uint_as_float(wy[i]);
                }
                o.x = __float_as_uint(gj * fd[0]);
                o.y = __float_as_uint(gj * fd[1]);
                o.z = __float_as_uint(gj * fd[2]);
                o.w = __float_as_uint(gj * fd[3]);
            }
#pragma unroll
            for (int i = 0; i < E; ++i) dot = __builtin_fmaf(fd[i], fy[i], dot);
            dyp[row * row_vecs + v] = o;
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) dot += __shfl_xor(dot, m, 64);
        if (lane == 0) part[j][wave] = dot;
    }
    __syncthreads();
    if (threadIdx.x < k) {
        float s = 0.0f;
        for (int w = 0; w < nw; ++w) s += part[threadIdx.x][w];
        dgate[t * k + threadIdx.x] = s;
    }
}

hipError_t launch_combine_backward(const moe_cfg& c, const void* dout, const void* y_perm,
                                   const float* gate, const int32_t* dst_row, void* dy_perm,
                                   float* dgate, hipStream_t st) {
    const int64_t T = c.tokens;
    if (T == 0) return hipSuccess;
    const int64_t esz = c.act_dtype == MOE_BF16 ? 2 : 4;
    const int64_t row_vecs = c.hidden * esz / 16;
    const int threads = (int)(row_vecs >= 1024 ? 1024 : (row_vecs + 63) / 64 * 64);
    if (c.act_dtype == MOE_BF16)
        combine_backward_kernel<true><<<dim3((unsigned)T), threads, 0, st>>>(
            (const uint4*)dout, (const uint4*)y_perm, gate, dst_row, (uint4*)dy_perm, dgate,
            (int)c.top_k, row_vecs);
    else
        combine_backward_kernel<false><<<dim3((unsigned)T), threads, 0, st>>>(
            (const uint4*)dout, (const uint4*)y_perm, gate, dst_row, (uint4*)dy_perm, dgate,
            (int)c.top_k, row_vecs);
    return hipGetLastError();
}

// ---------------------------------------------------------------- gates -> logits
// With S = sum of the chosen s and g_j = s_j / S:  dg_j/ds_m = (delta_jm - g_j)/S,
// so ds_m = (dgate_m - sum_j dgate_j g_j) / S, and through the sigmoid
// dz_m = ds_m s_m (1 - s_m).  One wavefront per token, lane j < k holds slot j;
// S and the weighted sum are double sums (fixed butterfly).  Writes dz[t, j]
// and the same value at the slot's permuted row.
__global__ void __launch_bounds__(256) route_backward_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ idx,
    const float* __restrict__ dgate, const int32_t* __restrict__ dst_row, float* __restrict__ dz,
    float* __restrict__ dz_perm, int64_t T, int64_t N, int k) {
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (t >= T) return;  // whole wavefronts
    const bool on = lane < k;
    const double s = on ? (double)scores[t * N + idx[t * k + lane]] : 0.0;
    const double dg = on ? (double)dgate[t * k + lane] : 0.0;
    double S = s;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) S += __shfl_xor(S, m, 64);
    double gd = on ? dg * (s / S) : 0.0;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) gd += __shfl_xor(gd, m, 64);
    if (on) {
        const float v = (float)((dg - gd) / S * s * (1.0 - s));
        dz[t * k + lane] = v;
        dz_perm[dst_row[t * k + lane]] = v;
    }
}

// ---------------------------------------------------------------- centroids
// z[t,i] = u_t . e_i, so dE[i, c] = sum over the rows r of expert i of
// dz_perm[r] * x[src_token[r], c] (rows ascending, fp32 FMAs).  Block =
// (expert, 2048-column slice for bf16 / 1024 for fp32); thread = one 16-byte
// vector of columns.  Experts without rows get zeros.
template <bool BF16>
__global__ void __launch_bounds__(256) centroid_grad_kernel(
    const uint4* __restrict__ x, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ src_token, const float* __restrict__ dz_perm,
    float* __restrict__ dE, int64_t row_vecs, int64_t d) {
    constexpr int E = BF16 ? 8 : 4;
    const int i = blockIdx.x;
    const int64_t v = (int64_t)blockIdx.y * 256 + threadIdx.x;
    if (v >= row_vecs) return;
    const int32_t r0 = offsets[i], r1 = offsets[i + 1];
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0f;
    for (int32_t r = r0; r < r1; ++r) {
        const float w = dz_perm[r];
        const uint4 q = x[(int64_t)src_token[r] * row_vecs + v];
        float f[8];
        if constexpr (BF16) {
            unpack8(q, f);
        } else {
            f[0] = __uint_as_float(q.x);
            f[1] = __uint_as_float(q.y);
            f[2] = __uint_as_float(q.z);
            f[3] = __uint_as_float(q.w);
        }
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = __builtin_fmaf(w, f[e], acc[e]);
    }
    float* out = dE + (int64_t)i * d + v * E;
#pragma unroll
    for (int e = 0; e < E; e += 4) *(float4*)(out + e) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
}

hipError_t launch_route_backward(const moe_cfg& c, const void* x, const float* scores,
                                 const int32_t* idx, const float* dgate, const int32_t* offsets,
                                 const int32_t* src_token, const int32_t* dst_row, float* dz,
                                 float* dz_perm, float* dcentroids, hipStream_t st) {
    const int64_t T = c.tokens, N = c.n_experts, d = c.hidden;
    if (T > 0)
        route_backward_kernel<<<dim3((unsigned)cdiv(T, 4)), 256, 0, st>>>(
            scores, idx, dgate, dst_row, dz, dz_perm, T, N, (int)c.top_k);
    const int64_t esz = c.act_dtype == MOE_BF16 ? 2 : 4;
    const int64_t row_vecs = d * esz / 16;
    const dim3 grid((unsigned)N, (unsigned)cdiv(row_vecs, 256));
    if (c.act_dtype == MOE_BF16)
        centroid_grad_kernel<true><<<grid, 256, 0, st>>>((const uint4*)x, offsets, src_token,
                                                         dz_perm, dcentroids, row_vecs, d);
    else
        centroid_grad_kernel<false><<<grid, 256, 0, st>>>((const uint4*)x, offsets, src_token,
                                                          dz_perm, dcentroids, row_vecs, d);
    return hipGetLastError();
}

// ---------------------------------------------------------------- input gradient
// dx[t] = dout[t] (residual) + dx_shared[t] + sum_j dx_perm[dst[t,j]]
//         + sum_j dz[t,j] e_{idx[t,j]}
// summed in fp32 in that order (slot by slot), rounded once.  One block per
// token, one thread per 16-byte vector of the row.
template <bool BF16>
__global__ void __launch_bounds__(1024) input_grad_kernel(
    const uint4* __restrict__ dout, const uint4* __restrict__ dxs, const uint4* __restrict__ dxp,
    const int32_t* __restrict__ dst_row, const float* __restrict__ dz,
    const int32_t* __restrict__ idx, const float* __restrict__ E, uint4* __restrict__ dx, int k,
    int64_t row_vecs, int64_t d) {
    __shared__ int32_t rows[64];
    __shared__ int32_t ex[64];
    __shared__ float w[64];
    const int64_t t = blockIdx.x;
    if (threadIdx.x < k) {
        rows[threadIdx.x] = dst_row[t * k + threadIdx.x];
        ex[threadIdx.x] = idx[t * k + threadIdx.x];
        w[threadIdx.x] = dz[t * k + threadIdx.x];
    }
    __syncthreads();
    constexpr int NE = BF16 ? 8 : 4;
    for (int64_t v = threadIdx.x; v < row_vecs; v += blockDim.x) {
        float acc[NE];
#pragma unroll
        for (int i = 0; i < NE; ++i) acc[i] = 0.0f;
        auto add = [&](const uint4 q) {
            float f[8];
            if constexpr (BF16) {
                unpack8(q, f);
            } else {
                f[0] = __uint_as_float(q.x);
                f[1] = __uint_as_float(q.y);
                f[2] = __uint_as_float(q.z);
                f[3] = __uint_as_float(q.w);
            }
#pragma unroll
            for (int i = 0; i < NE; ++i) acc[i] += f[i];
        };
        if (dout) add(dout[t * row_vecs + v]);
        if (dxs) add(dxs[t * row_vecs + v]);
        for (int j = 0; j < k; ++j) {
            add(dxp[(int64_t)rows[j] * row_vecs + v]);
            const float* e = E + (int64_t)ex[j] * d + v * NE;
#pragma unroll
            for (int i = 0; i < NE; i += 4) {
                const float4 q = *(const float4*)(e + i);
                acc[i] = __builtin_fmaf(w[j], q.x, acc[i]);
                acc[i + 1] = __builtin_fmaf(w[j], q.y, acc[i + 1]);
                acc[i + 2] = __builtin_fmaf(w[j], q.z, acc[i + 2]);
                acc[i + 3] = __builtin_fmaf(w[j], q.w, acc[i + 3]);
            }
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
        dx[t * row_vecs + v] = o;
    }
}

hipError_t launch_input_grad(const moe_cfg& c, const void* dout, const void* dx_shared,
                             const void* dx_perm, const int32_t* dst_row, const float* dz,
                             const int32_t* idx, const float* centroids, void* dx,
                             hipStream_t st) {
    const int64_t T = c.tokens;
    if (T == 0) return hipSuccess;
    const int64_t esz = c.act_dtype == MOE_BF16 ? 2 : 4;
    const int64_t row_vecs = c.hidden * esz / 16;
    const int threads = (int)(row_vecs >= 1024 ? 1024 : (row_vecs + 63) / 64 * 64);
    if (c.act_dtype == MOE_BF16)
        input_grad_kernel<true><<<dim3((unsigned)T), threads, 0, st>>>(
            (const uint4*)dout, (const uint4*)dx_shared, (const uint4*)dx_perm, dst_row, dz, idx,
            centroids, (uint4*)dx, (int)c.top_k, row_vecs, c.hidden);
    else
        input_grad_kernel<false><<<dim3((unsigned)T), threads, 0, st>>>(
            (const uint4*)dout, (const uint4*)dx_shared, (const uint4*)dx_perm, dst_row, dz, idx,
            centroids, (uint4*)dx, (int)c.top_k, row_vecs, c.hidden);
    return hipGetLastError();
}

}  // namespace moe
