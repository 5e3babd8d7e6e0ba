// permute.hip -- dispatch of token rows to experts: a stable counting sort of
// the T*k (token, slot) pairs by expert, and the row gather that feeds the
// grouped expert GEMMs.  (The pages show dispatch only as the cross-node
// all-to-all of the DeepSeek-V3 training setup; on one GPU it is this
// permutation.)
//
// Row of pair (t, j) with expert e = idx[t, j]:
//   offsets[e] + #{pairs (t', j') with idx = e and t' < t}
// (a token's k experts are distinct, so ties inside a token cannot occur).
// Computed without order-dependent atomics:
//   1. rank:    per block of PERM_TB tokens, one wavefront walks the tokens in
//               order with LDS counters -> block-local rank and block histogram
//   2. bscan:   per expert, exclusive prefix of its block histogram over blocks
//   3. offsets: exclusive prefix of the per-expert totals
//   4. scatter: dst_row, src_token, and the row copy x[t] -> x_perm[row] for
//               each of the token's k rows (FP8: quantise the row's 1x128 tiles
//               into x_q, x_s first, then copy codes and scales).  Without
//               x_perm (the expert GEMM gathers the rows itself through
//               src_token) only the indices (and for FP8 x_q, x_s) are written.
#include <mutex>

#include "moe_internal.h"

namespace moe {

struct PermWs {
    int32_t* local_rank;  // [T*k]
    int32_t* blk;         // [nblk][N]: block histogram, then prefix over blocks
    int32_t* totals;      // [N]
};

static int64_t align256(int64_t b) { return (b + 255) & ~int64_t(255); }

size_t permute_workspace_bytes(const moe_cfg& c) {
    const int64_t TK = c.tokens * c.top_k, nblk = cdiv(c.tokens, PERM_TB);
    return (size_t)(align256(TK * 4) + align256(nblk * c.n_experts * 4) +
                    align256(c.n_experts * 4));
}

static PermWs carve(const moe_cfg& c, void* ws) {
    const int64_t TK = c.tokens * c.top_k, nblk = cdiv(c.tokens, PERM_TB);
    char* p = (char*)ws;
    PermWs w;
    w.local_rank = (int32_t*)p;
    p += align256(TK * 4);
    w.blk = (int32_t*)p;
    p += align256(nblk * c.n_experts * 4);
    w.totals = (int32_t*)p;
    return w;
}

// 1. one wavefront per block of PERM_TB tokens
__global__ void __launch_bounds__(64) perm_rank_kernel(const int32_t* __restrict__ idx,
                                                       int32_t* __restrict__ local_rank,
                                                       int32_t* __restrict__ blk, int64_t T,
                                                       int k, int N) {
    __shared__ int32_t cnt[1024];
    const int lane = threadIdx.x;
    for (int e = lane; e < N; e += 64) cnt[e] = 0;
    __syncthreads();
    const int64_t t0 = (int64_t)blockIdx.x * PERM_TB;
    const int64_t t1 = min(t0 + PERM_TB, T);
    for (int64_t t = t0; t < t1; ++t) {
        // lanes j < k handle slot j; the k experts of a token are distinct, so
        // the read-modify-writes below touch distinct counters
        if (lane < k) {
            const int e = idx[t * k + lane];
            const int r = cnt[e];
            cnt[e] = r + 1;
            local_rank[t * k + lane] = r;
        }
        __syncthreads();  // the next token's reads see these updates
    }
    int32_t* out = blk + (int64_t)blockIdx.x * N;
    for (int e = lane; e < N; e += 64) out[e] = cnt[e];
}

// 2. one 256-thread block per expert: exclusive prefix over the blocks
__global__ void __launch_bounds__(256) perm_bscan_kernel(int32_t* __restrict__ blk,
                                                         int32_t* __restrict__ totals,
                                                         int64_t nblk, int N) {
    __shared__ int32_t sh_wave[4];
    __shared__ int32_t sh_carry;
    const int e = blockIdx.x;
    if (threadIdx.x == 0) sh_carry = 0;
    __syncthreads();
    for (int64_t b0 = 0; b0 < nblk; b0 += 256) {
        const int64_t b = b0 + threadIdx.x;
        const int32_t v = b < nblk ? blk[b * N + e] : 0;
        const int32_t incl = block_incl_scan_256(v, sh_wave);
        const int32_t carry = sh_carry;
        if (b < nblk) blk[b * N + e] = carry + incl - v;
        __syncthreads();
        if (threadIdx.x == 255) sh_carry = carry + incl;
        __syncthreads();
    }
    if (threadIdx.x == 0) totals[e] = sh_carry;
}

// 3. offsets = exclusive prefix of the totals (one 256-thread block)
__global__ void __launch_bounds__(256) perm_offsets_kernel(const int32_t* __restrict__ totals,
                                                           int32_t* __restrict__ offsets,
                                                           int N) {
    __shared__ int32_t sh_wave[4];
    __shared__ int32_t sh_carry;
    if (threadIdx.x == 0) sh_carry = 0;
    __syncthreads();
    for (int e0 = 0; e0 < N; e0 += 256) {
        const int e = e0 + threadIdx.x;
        const int32_t v = e < N ? totals[e] : 0;
        const int32_t incl = block_incl_scan_256(v, sh_wave);
        const int32_t carry = sh_carry;
        if (e < N) offsets[e] = carry + incl - v;
        __syncthreads();
        if (threadIdx.x == 255) sh_carry = carry + incl;
        __syncthreads();
    }
    if (threadIdx.x == 0) offsets[N] = sh_carry;
}

// 4a. rows of 16-byte vectors (bf16 or fp32): one 128-thread block per token
__global__ void __launch_bounds__(128) perm_scatter_kernel(
    const uint4* __restrict__ x, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ local_rank, const int32_t* __restrict__ blk,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ src_token,
    int32_t* __restrict__ dst_row, uint4* __restrict__ x_perm, int k, int N, int64_t row_vecs) {
    __shared__ int32_t rows[64];
    const int64_t t = blockIdx.x;
    if (threadIdx.x < k) {
        const int j = threadIdx.x;
        const int e = idx[t * k + j];
        const int32_t row = offsets[e] + blk[(t / PERM_TB) * N + e] + local_rank[t * k + j];
        rows[j] = row;
        dst_row[t * k + j] = row;
        src_token[row] = (int32_t)t;
    }
    __syncthreads();
    const uint4* src = x + t * row_vecs;
    for (int64_t v = threadIdx.x; v < row_vecs; v += blockDim.x) {
        const uint4 val = src[v];
        // the permuted rows are written once here and read back by the expert
        // GEMMs long after: non-temporal stores (measured faster)
        for (int j = 0; j < k; ++j)
            __builtin_nontemporal_store(u32x4_t{val.x, val.y, val.z, val.w},
                                        (u32x4_t*)(x_perm + (int64_t)rows[j] * row_vecs + v));
    }
}

// 4c. indices only (no row copy): one thread per (token, slot) pair
__global__ void __launch_bounds__(256) perm_index_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ local_rank,
    const int32_t* __restrict__ blk, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ src_token, int32_t* __restrict__ dst_row, int64_t T, int k, int N) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= T * k) return;
    const int64_t t = i / k;
    const int e = idx[i];
    const int32_t row = offsets[e] + blk[(t / PERM_TB) * N + e] + local_rank[i];
    dst_row[i] = row;
    src_token[row] = (int32_t)t;
}

// threads per token block of the FP8 scatter (up to 2 row vectors each: more
// blocks resident than with one 896-thread block per V3 token, 69 -> 62 us
// per permute call)
#ifndef MOE_F8SC_T
#define MOE_F8SC_T 512
#endif
// 4b. FP8: one 128-thread block per token; 16 lanes per 1x128 tile, 8 values
// per lane.  scale = amax/448 (fp32 divide); codes are nearest-even E4M3 of
// clamp(v/scale, +-448); all-zero tile -> scale 0, codes 0.
__global__ void __launch_bounds__(1024) perm_scatter_fp8_kernel(
    const uint4* __restrict__ x, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ local_rank, const int32_t* __restrict__ blk,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ src_token,
    int32_t* __restrict__ dst_row, uint2* __restrict__ x_perm, float* __restrict__ x_perm_scale,
    uint2* __restrict__ x_q, float* __restrict__ x_s, int k, int N, int64_t d) {
    __shared__ int32_t rows[64];
    const int64_t t = blockIdx.x;
    if (threadIdx.x < k) {
        const int j = threadIdx.x;
        const int e = idx[t * k + j];
        const int32_t row = offsets[e] + blk[(t / PERM_TB) * N + e] + local_rank[t * k + j];
        rows[j] = row;
        dst_row[t * k + j] = row;
        src_token[row] = (int32_t)t;
    }
    // the token's rows are needed only to scatter into x_perm; the codes of x
    // itself do not wait for the index loads
    if (x_perm != nullptr) __syncthreads();
    const int64_t vecs = d / 8;     // 8 bf16 per 16-byte vector
    const int64_t tiles = d / 128;
    const uint4* src = x + t * vecs;
    // blockDim.x (a multiple of 64) threads = blockDim.x/16 tiles per pass;
    // every lane of a 16-lane group belongs to the same tile, and a pass is
    // entered by the whole block (uniform trip count)
#pragma unroll 4
    for (int64_t v0 = 0; v0 < vecs; v0 += blockDim.x) {
        const int64_t v = v0 + threadIdx.x;
        const bool valid = v < vecs;
        uint4 val = valid ? src[v] : make_uint4(0, 0, 0, 0);
        float f[8];
        const uint32_t w[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
        const float scale = amax / 448.0f;
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) lo |= quant_e4m3(f[i], scale) << (8 * i);
#pragma unroll
        for (int i = 0; i < 4; ++i) hi |= quant_e4m3(f[4 + i], scale) << (8 * i);
        if (valid) {
            const uint2 q = make_uint2(lo, hi);
            x_q[t * vecs + v] = q;
            if (x_perm != nullptr)  // (without it the GEMM gathers from x_q)
                for (int j = 0; j < k; ++j)  // written once, read by the GEMMs later
                    __builtin_nontemporal_store(u32x2_t{lo, hi},
                                                (u32x2_t*)(x_perm + (int64_t)rows[j] * vecs + v));
            if ((threadIdx.x & 15) == 0) {
                const int64_t tile = v / 16;
                x_s[t * tiles + tile] = scale;
                if (x_perm != nullptr)
                    for (int j = 0; j < k; ++j) x_perm_scale[(int64_t)rows[j] * tiles + tile] = scale;
            }
        }
    }
}

// ---------------------------------------------------------------- no-allocation variant
//
// moe_permute_noalloc's scratch: the same ranks and block histograms as the
// caller's workspace of moe_permute, held in this file-scope device array
// (every GPU the library runs on holds its own copy until the process ends).
// In host code `scratch` names a host-side stand-in, not a device address, so
// the kernels get the address hipGetSymbolAddress returns for the current
// device, looked up once per device and kept.  Every element the permutation
// reads is written earlier in the same call, so nothing is cleared; calls that
// overlap on one GPU (two streams) share the array and race.
static __device__ __align__(256) uint8_t scratch[PERM_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t permute_scratch(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_permute(const moe_cfg& c, const void* x, const int32_t* idx,
                          int32_t* offsets, int32_t* src_token, int32_t* dst_row, void* x_perm,
                          float* x_perm_scale, uint8_t* x_q, float* x_s, void* ws,
                          hipStream_t st) {
    const int64_t T = c.tokens, N = c.n_experts;
    const int k = (int)c.top_k;
    const int64_t nblk = cdiv(T, PERM_TB);
    PermWs w = carve(c, ws);
    if (T > 0) {
        perm_rank_kernel<<<dim3((unsigned)nblk), 64, 0, st>>>(idx, w.local_rank, w.blk, T, k,
                                                              (int)N);
    }
    perm_bscan_kernel<<<dim3((unsigned)N), 256, 0, st>>>(w.blk, w.totals, nblk, (int)N);
    perm_offsets_kernel<<<1, 256, 0, st>>>(w.totals, offsets, (int)N);
    if (T > 0) {
        if (x_perm == nullptr && c.gemm_dtype != MOE_FP8_E4M3) {
            perm_index_kernel<<<dim3((unsigned)cdiv(T * k, 256)), 256, 0, st>>>(
                idx, w.local_rank, w.blk, offsets, src_token, dst_row, T, k, (int)N);
        } else if (c.gemm_dtype == MOE_FP8_E4M3) {
            const int64_t vecs = c.hidden / 8;
            const int threads = (int)(vecs >= MOE_F8SC_T ? MOE_F8SC_T : (vecs + 63) / 64 * 64);
            perm_scatter_fp8_kernel<<<dim3((unsigned)T), threads, 0, st>>>(
                (const uint4*)x, idx, w.local_rank, w.blk, offsets, src_token, dst_row,
                (uint2*)x_perm, x_perm_scale, (uint2*)x_q, x_s, k, (int)N, c.hidden);
        } else {
            const int64_t esz = c.act_dtype == MOE_BF16 ? 2 : 4;
            perm_scatter_kernel<<<dim3((unsigned)T), 128, 0, st>>>(
                (const uint4*)x, idx, w.local_rank, w.blk, offsets, src_token, dst_row,
                (uint4*)x_perm, k, (int)N, c.hidden * esz / 16);
        }
    }
    return hipGetLastError();
}

}  // namespace moe
