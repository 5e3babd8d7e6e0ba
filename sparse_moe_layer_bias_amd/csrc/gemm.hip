// gemm.hip -- grouped SwiGLU expert FFN (routed experts + the shared expert in
// the same launches) for bf16 and fp32 storage.
//
// DeepSeek-V3 report reading guide (xyznot.com/de), "Methode" item 2: each
// token's routed experts FFN^(r)_i and the shared expert FFN^(s) are applied to
// u_t.  FFN_i is read as SwiGLU without biases: W2 (silu(W1 u) * (W3 u)).
//
// Two launches per step:
//   gate/up:  h[r, :] = silu(x[r] W1^T) * (x[r] W3^T)    (SwiGLU fused in the epilogue)
//   down:     y[r, :] = h[r] W2^T
// Each launch walks a device-side tile list built from the expert offsets
// (ffn_tile_map), so the ragged per-expert row counts never reach the host.
//
// bf16 kernel (gfx950 MFMA v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//   workgroup tile 128 rows x 128 weight rows, K step 64, LDS double buffer
//   with an XOR swizzle of 16-byte chunks; 4 wavefronts in 2x2, 64x64 each.
//   gate/up: the 128 weight rows of a tile are W1 and W3 rows of the same 64
//   h columns, arranged so that each wavefront holds a and b of the same
//   (row, column) in the same accumulator slot.
//   Tile order is XCD-aware: consecutive tiles of one expert land on one XCD,
//   so its activation rows and weight panels are shared through that L2.
#include "moe_internal.h"

namespace moe {

static int64_t align256(int64_t b) { return (b + 255) & ~int64_t(255); }

constexpr int BF_BM = 128;   // rows (tokens) per tile
constexpr int BF_BN = 128;   // weight rows per tile
constexpr int BF_BK = 64;    // contraction step
constexpr int F32_BM = 64;   // fp32 path

// ---------------------------------------------------------------- tile map

// groups 0..N-1 are routed experts (rows offsets[g]..offsets[g+1]), group N is
// the shared expert (rows 0..T-1) when present.  Output: tiles[i] = (group, m0)
// and *n_tiles.
__global__ void __launch_bounds__(256) ffn_tile_map_kernel(const int32_t* __restrict__ offsets,
                                                           int N, int64_t T, int has_shared,
                                                           int BM, int2* __restrict__ tiles,
                                                           int32_t* __restrict__ n_tiles) {
    __shared__ int32_t sh_wave[4];
    __shared__ int32_t sh_carry;
    const int ng = N + (has_shared ? 1 : 0);
    if (threadIdx.x == 0) sh_carry = 0;
    __syncthreads();
    for (int g0 = 0; g0 < ng; g0 += 256) {
        const int g = g0 + threadIdx.x;
        int64_t M = 0;
        if (g < N)
            M = offsets[g + 1] - offsets[g];
        else if (g < ng)
            M = T;
        const int32_t nt = (int32_t)((M + BM - 1) / BM);
        const int32_t incl = block_incl_scan_256(nt, sh_wave);
        const int32_t start = sh_carry + incl - nt;
        for (int32_t i = 0; i < nt; ++i) tiles[start + i] = make_int2(g, i * BM);
        __syncthreads();
        if (threadIdx.x == 255) sh_carry = sh_carry + incl;
        __syncthreads();
    }
    if (threadIdx.x == 0) *n_tiles = sh_carry;
}

struct GemmParams {
    const int2* tiles;
    const int32_t* n_tiles;
    const int32_t* offsets;
    int N;          // routed experts
    int ntn;        // n-tiles per m-tile in the grid (max over groups)
    int64_t T;
    int64_t K_r, K_s;        // contraction length, routed / shared
    int64_t Nout_r, Nout_s;  // output columns, routed / shared
    const void* A_r;         // routed rows  [TK, K_r]
    const void* A_s;         // shared rows  [T, K_s]
    const void* B_r;         // per-expert weights
    const void* B_s;
    void* C_r;               // [TK, Nout_r]
    void* C_s;               // [T, Nout_s]
};

struct Work {
    int64_t m0, M, K, Nout, nt;
    const char* A;
    const char* B;
    char* C;
};

// decode the workgroup's (tile, n-tile); returns false when there is no work.
// Work units are numbered u = mt * ntn + nt; unit u goes to blockIdx
// (u % per) * 8 + u / per with per = ceil(units / 8), so that XCD x (which is
// handed blockIdx x, x+8, ...) runs the contiguous unit range [x*per, (x+1)*per).
template <int MODE, int ESZ>
__device__ __forceinline__ bool decode_work(const GemmParams& p, int cols_per_tile, Work& w) {
    const int64_t units = (int64_t)(*p.n_tiles) * p.ntn;
    const int64_t per = (units + 7) / 8;
    const int64_t L = blockIdx.x;
    if (L >= 8 * per) return false;
    const int64_t u = (L % 8) * per + L / 8;
    if (u >= units) return false;
    const int64_t mt = u / p.ntn;
    w.nt = u % p.ntn;
    const int2 t = p.tiles[mt];
    const int g = t.x;
    w.m0 = t.y;
    int64_t rowbase;
    if (g < p.N) {
        rowbase = p.offsets[g];
        w.M = p.offsets[g + 1] - rowbase;
        w.K = p.K_r;
        w.Nout = p.Nout_r;
        w.A = (const char*)p.A_r + rowbase * w.K * ESZ;
        const int64_t wrows = MODE == 0 ? 2 * w.Nout : w.Nout;
        w.B = (const char*)p.B_r + (int64_t)g * wrows * w.K * ESZ;
        w.C = (char*)p.C_r + rowbase * w.Nout * ESZ;
    } else {
        w.M = p.T;
        w.K = p.K_s;
        w.Nout = p.Nout_s;
        w.A = (const char*)p.A_s;
        w.B = (const char*)p.B_s;
        w.C = (char*)p.C_s;
    }
    return w.nt * cols_per_tile < w.Nout;
}

// ---------------------------------------------------------------- bf16 MFMA

__device__ __forceinline__ float silu_f(float a) { return a / (1.0f + __expf(-a)); }

// LDS element offset of (row, 16-byte chunk) in a [128][64] bf16 tile
__device__ __forceinline__ int swz(int row, int ch) { return row * 64 + ((ch ^ (row & 7)) << 3); }

template <int MODE>
__global__ void __launch_bounds__(256, 2) ffn_gemm_bf16_kernel(GemmParams p) {
    Work w;
    constexpr int COLS = MODE == 0 ? 64 : 128;  // output columns per tile
    if (!decode_work<MODE, 2>(p, COLS, w)) return;

    __shared__ __attribute__((aligned(16))) uint16_t As[2][BF_BM * BF_BK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BF_BN * BF_BK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t K = w.K;
    const int64_t valid_rows = w.M - w.m0;  // >= 1

    // global source rows of this thread's 4 A chunks and 4 B chunks
    const uint16_t* a_src[4];
    const uint16_t* b_src[4];
    int lds_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = tid + 256 * i;
        const int row = c >> 3, ch = c & 7;
        int64_t ar = w.m0 + row;
        if (ar >= w.M) ar = w.M - 1;  // clamp to a valid row; never stored
        a_src[i] = (const uint16_t*)w.A + ar * K + ch * 8;
        int64_t br;
        if (MODE == 0) {
            const int half = (row >> 5) & 1, wn_ = row >> 6, j = row & 31;
            br = (half ? w.Nout : 0) + w.nt * 64 + wn_ * 32 + j;
        } else {
            br = w.nt * 128 + row;
        }
        b_src[i] = (const uint16_t*)w.B + br * K + ch * 8;
        lds_off[i] = swz(row, ch);
    }

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    uint4 ra[4], rb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ra[i] = *(const uint4*)(a_src[i]);
        rb[i] = *(const uint4*)(b_src[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        *(uint4*)(&As[0][lds_off[i]]) = ra[i];
        *(uint4*)(&Bs[0][lds_off[i]]) = rb[i];
    }
    __syncthreads();

    const bool blk_on[2] = {wm * 64 < valid_rows, wm * 64 + 32 < valid_rows};
    const int nk = (int)(K / BF_BK);
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            const int64_t koff = (int64_t)(kt + 1) * BF_BK;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ra[i] = *(const uint4*)(a_src[i] + koff);
                rb[i] = *(const uint4*)(b_src[i] + koff);
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int ch = 2 * s + (lane >> 5);
            bf16x8_t af[2], bfr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = wm * 64 + i * 32 + (lane & 31);
                af[i] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(&As[buf][swz(r, ch)]));
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int r = wn * 64 + j * 32 + (lane & 31);
                bfr[j] = __builtin_bit_cast(bf16x8_t, *(const uint4*)(&Bs[buf][swz(r, ch)]));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                if (!blk_on[i]) continue;
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j],
                                                                         0, 0, 0);
            }
        }
        if (more) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                *(uint4*)(&As[buf ^ 1][lds_off[i]]) = ra[i];
                *(uint4*)(&Bs[buf ^ 1][lds_off[i]]) = rb[i];
            }
        }
        __syncthreads();
    }

    // epilogue.  32x32 accumulator layout: lane l holds column l%32 and rows
    // 8*(v/4) + 4*(l/32) + v%4 for v = 0..15.
    uint16_t* C = (uint16_t*)w.C;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        if (!blk_on[i]) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int64_t r = w.m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            if (r >= w.M) continue;
            if (MODE == 0) {
                const int64_t c = w.nt * 64 + wn * 32 + (lane & 31);
                const float a = acc[i][0][v], b = acc[i][1][v];
                C[r * w.Nout + c] = f32_to_bf16(silu_f(a) * b);
            } else {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int64_t c = w.nt * 128 + wn * 64 + j * 32 + (lane & 31);
                    C[r * w.Nout + c] = f32_to_bf16(acc[i][j][v]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------- fp32 path
// Plain VALU kernel for fp32 storage (small layers): 64 rows x 64 columns per
// 256-thread block; thread = (row tid%64, 16 columns (tid/64)*16..+15).
template <int MODE>
__global__ void __launch_bounds__(256) ffn_gemm_f32_kernel(GemmParams p) {
    Work w;
    if (!decode_work<MODE, 4>(p, 64, w)) return;
    const int tid = threadIdx.x;
    const int64_t r = w.m0 + (tid & 63);
    if (r >= w.M) return;
    const float* a = (const float*)w.A + r * w.K;
    const float* B = (const float*)w.B;
    float* C = (float*)w.C;
    const int64_t c0 = w.nt * 64 + (tid >> 6) * 16;
    for (int jj = 0; jj < 16; ++jj) {
        const int64_t c = c0 + jj;
        if (c >= w.Nout) break;
        if (MODE == 0) {
            const float* w1 = B + c * w.K;
            const float* w3 = B + (w.Nout + c) * w.K;
            float sa = 0.0f, sb = 0.0f;
            for (int64_t k = 0; k < w.K; ++k) {
                sa = __builtin_fmaf(a[k], w1[k], sa);
                sb = __builtin_fmaf(a[k], w3[k], sb);
            }
            C[r * w.Nout + c] = sa / (1.0f + expf(-sa)) * sb;
        } else {
            const float* w2 = B + c * w.K;
            float s = 0.0f;
            for (int64_t k = 0; k < w.K; ++k) s = __builtin_fmaf(a[k], w2[k], s);
            C[r * w.Nout + c] = s;
        }
    }
}

// ---------------------------------------------------------------- launch

struct FfnWs {
    int2* tiles;
    int32_t* n_tiles;
    void* h_r;   // [TK, I]
    void* h_s;   // [T, Is]
    float* hs_r; // FP8 scales [TK, I/128]
    float* hs_s; // FP8 scales [T, Is/128]
};

static int ffn_bm(const moe_cfg& c) {
    return c.act_dtype == MOE_F32 ? F32_BM : BF_BM;
}

static int64_t ffn_max_tiles(const moe_cfg& c) {
    const int64_t BM = ffn_bm(c), TK = c.tokens * c.top_k;
    return TK / BM + c.n_experts + 1 + cdiv(c.tokens, BM) + 1;
}

static int64_t h_elem_bytes(const moe_cfg& c) {
    return c.gemm_dtype == MOE_FP8_E4M3 ? 1 : (c.act_dtype == MOE_BF16 ? 2 : 4);
}

size_t ffn_workspace_bytes(const moe_cfg& c) {
    const int64_t TK = c.tokens * c.top_k, T = c.tokens;
    const int64_t eb = h_elem_bytes(c);
    int64_t b = align256(ffn_max_tiles(c) * 8) + 256;
    b += align256(TK * c.inter * eb) + align256(T * c.inter_shared * eb);
    if (c.gemm_dtype == MOE_FP8_E4M3)
        b += align256(TK * (c.inter / 128) * 4) + align256(T * (c.inter_shared / 128) * 4);
    return (size_t)b;
}

static FfnWs carve_ffn(const moe_cfg& c, void* ws) {
    const int64_t TK = c.tokens * c.top_k, T = c.tokens;
    const int64_t eb = h_elem_bytes(c);
    char* p = (char*)ws;
    FfnWs w{};
    w.tiles = (int2*)p;
    p += align256(ffn_max_tiles(c) * 8);
    w.n_tiles = (int32_t*)p;
    p += 256;
    w.h_r = p;
    p += align256(TK * c.inter * eb);
    w.h_s = p;
    p += align256(T * c.inter_shared * eb);
    if (c.gemm_dtype == MOE_FP8_E4M3) {
        w.hs_r = (float*)p;
        p += align256(TK * (c.inter / 128) * 4);
        w.hs_s = (float*)p;
    }
    return w;
}

hipError_t launch_expert_ffn_fp8(const moe_cfg& c, const FfnArgs& a, const int2* tiles,
                                 const int32_t* n_tiles, void* h_r, void* h_s, float* hs_r,
                                 float* hs_s, int64_t max_tiles, hipStream_t st);

hipError_t launch_expert_ffn(const moe_cfg& c, const FfnArgs& a, void* ws, hipStream_t st) {
    const int64_t T = c.tokens, TK = T * c.top_k;
    const bool has_shared = c.inter_shared > 0 && T > 0;
    if (TK == 0) return hipSuccess;
    FfnWs w = carve_ffn(c, ws);
    const int BM = ffn_bm(c);
    const int64_t max_tiles = ffn_max_tiles(c);
    ffn_tile_map_kernel<<<1, 256, 0, st>>>(a.offsets, (int)c.n_experts, T, has_shared ? 1 : 0,
                                           BM, w.tiles, w.n_tiles);
    if (c.gemm_dtype == MOE_FP8_E4M3)
        return launch_expert_ffn_fp8(c, a, w.tiles, w.n_tiles, w.h_r, w.h_s, w.hs_r, w.hs_s,
                                     max_tiles, st);

    GemmParams p{};
    p.tiles = w.tiles;
    p.n_tiles = w.n_tiles;
    p.offsets = a.offsets;
    p.N = (int)c.n_experts;
    p.T = has_shared ? T : 0;
    const int64_t Imax = c.inter > c.inter_shared ? c.inter : c.inter_shared;

    // gate/up: A = x rows, B = W13, C = h
    p.K_r = c.hidden;
    p.K_s = c.hidden;
    p.Nout_r = c.inter;
    p.Nout_s = c.inter_shared;
    p.A_r = a.x_perm;
    p.A_s = a.x_sh;
    p.B_r = a.w13;
    p.B_s = a.ws13;
    p.C_r = w.h_r;
    p.C_s = w.h_s;
    if (c.act_dtype == MOE_BF16) {
        p.ntn = (int)(Imax / 64);
        ffn_gemm_bf16_kernel<0><<<dim3((unsigned)(max_tiles * p.ntn)), 256, 0, st>>>(p);
    } else {
        p.ntn = (int)cdiv(Imax, 64);
        ffn_gemm_f32_kernel<0><<<dim3((unsigned)(max_tiles * p.ntn)), 256, 0, st>>>(p);
    }
    // down: A = h, B = W2, C = y
    p.K_r = c.inter;
    p.K_s = c.inter_shared;
    p.Nout_r = c.hidden;
    p.Nout_s = c.hidden;
    p.A_r = w.h_r;
    p.A_s = w.h_s;
    p.B_r = a.w2;
    p.B_s = a.ws2;
    p.C_r = a.y_perm;
    p.C_s = a.y_shared;
    if (c.act_dtype == MOE_BF16) {
        p.ntn = (int)(c.hidden / 128);
        ffn_gemm_bf16_kernel<1><<<dim3((unsigned)(max_tiles * p.ntn)), 256, 0, st>>>(p);
    } else {
        p.ntn = (int)cdiv(c.hidden, 64);
        ffn_gemm_f32_kernel<1><<<dim3((unsigned)(max_tiles * p.ntn)), 256, 0, st>>>(p);
    }
    return hipGetLastError();
}

}  // namespace moe
