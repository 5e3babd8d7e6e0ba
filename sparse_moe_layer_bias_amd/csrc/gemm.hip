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
// Tile order is XCD-aware (see decode_v2): consecutive work units of one
// expert land on one XCD so its token rows or weight panel are shared in L2.
#include "moe_internal.h"

namespace moe {

static int64_t align256(int64_t b) { return (b + 255) & ~int64_t(255); }

constexpr int BF_BM = 320;   // token rows per tile, bf16 / FP8 MFMA kernels
constexpr int F32_BM = 64;   // fp32 path

// ---------------------------------------------------------------- tile map

// Token tiles: routed expert g (rows offsets[g]..offsets[g+1]) gets
// ceil(M_g / BM) tiles, written first; the shared expert (rows 0..T-1) gets
// ceil(T / BM) tiles after them.  tiles[i] = (group, first row); group N is
// the shared expert.  counts[0] = routed tiles, counts[1] = shared tiles.
__global__ void __launch_bounds__(256) ffn_tile_map_kernel(const int32_t* __restrict__ offsets,
                                                           int N, int64_t T, int has_shared,
                                                           int BM, int2* __restrict__ tiles,
                                                           int32_t* __restrict__ counts) {
    __shared__ int32_t sh_wave[4];
    __shared__ int32_t sh_carry;
    if (threadIdx.x == 0) sh_carry = 0;
    __syncthreads();
    for (int g0 = 0; g0 < N; g0 += 256) {
        const int g = g0 + threadIdx.x;
        const int64_t M = g < N ? offsets[g + 1] - offsets[g] : 0;
        const int32_t nt = (int32_t)((M + BM - 1) / BM);
        const int32_t incl = block_incl_scan_256(nt, sh_wave);
        const int32_t start = sh_carry + incl - nt;
        for (int32_t i = 0; i < nt; ++i) tiles[start + i] = make_int2(g, i * BM);
        __syncthreads();
        if (threadIdx.x == 255) sh_carry = sh_carry + incl;
        __syncthreads();
    }
    const int32_t nr = sh_carry;
    const int32_t ns = has_shared ? (int32_t)((T + BM - 1) / BM) : 0;
    for (int32_t i = threadIdx.x; i < ns; i += blockDim.x) tiles[nr + i] = make_int2(N, i * BM);
    if (threadIdx.x == 0) {
        counts[0] = nr;
        counts[1] = ns;
    }
}

// ---------------------------------------------------------------- bf16 MFMA
//
// Workgroup = 8 wavefronts; tile = 256 weight rows x up to 320 token rows,
// i.e. one weight panel against ALL rows of an expert (routed experts get
// ~T*k/N rows), so every weight byte streams from HBM exactly once and the
// MFMA work follows the expert's real row count in steps of 32.
// MFMA v_mfma_f32_32x32x16_bf16 with the weight rows as the A operand:
// D[w][t] = sum_k W[w][k] X[t][k].  Wave (wg = wave%4, tg = wave/4) owns weight
// rows wg*64..+63 (two 32-row blocks) and token rows tg*160..+159 (five blocks).
// K step 64; the next step's operands are copied global -> LDS directly
// (global_load_lds_dwordx4) while the current step is multiplied; two LDS
// stages (2 x 72 KB).  LDS rows are 128 B (8 chunks of 16 B); chunk c of row r
// sits at slot c ^ (r & 7), so the 32 lanes reading one chunk of 32
// consecutive rows hit distinct banks.
// gate/up: the 64 weight rows of a wave are W1 rows n..n+31 (block 0) and W3
// rows n..n+31 (block 1): a and b of one (token, column) share a register slot
// and SwiGLU is applied in registers.

constexpr int G_WR = 256;      // weight rows per tile
constexpr int G_TR = 320;      // token rows per tile
constexpr int G_BK = 64;       // contraction step
constexpr int G_THREADS = 512;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ lds_void* to_lds(void* p) { return (lds_void*)p; }

struct GemmParamsV2 {
    const int2* tiles;     // routed tiles [0, n_r), shared tiles [n_r, n_r + n_s)
    const int32_t* counts; // [0] = routed tiles, [1] = shared tiles
    const int32_t* offsets;
    int N;
    int ntn_r, ntn_s;      // weight tiles per token tile, routed / shared
    int64_t T;
    int64_t K_r, K_s;
    int64_t Nout_r, Nout_s;
    const void* A_r;       // token rows
    const void* A_s;
    const void* B_r;       // weights
    const void* B_s;
    void* C_r;
    void* C_s;
};

struct WorkV2 {
    int64_t m0, M, K, Nout, wt;
    const char* X;   // token rows of the group
    const char* W;   // weights of the group
    char* C;         // output rows of the group
};

// Units: routed (tile, wt) tile-major -- the weight tiles of one expert run
// next to each other and share its token rows in L2; shared (wt, tile)
// wt-major -- the token chunks of one weight panel run next to each other and
// share it.  Unit u runs on blockIdx (u % per) * 8 + u / per, per = ceil(units/8),
// so each XCD (blockIdx x, x+8, ...) gets a contiguous unit range.
template <int ESZ>
__device__ __forceinline__ bool decode_v2(const GemmParamsV2& p, int mode, WorkV2& w) {
    const int64_t nr = p.counts[0], ns = p.counts[1];
    const int64_t ur = nr * p.ntn_r, units = ur + ns * p.ntn_s;
    const int64_t per = (units + 7) / 8;
    const int64_t L = blockIdx.x;
    if (L >= 8 * per) return false;
    const int64_t u = (L % 8) * per + L / 8;
    if (u >= units) return false;
    int64_t tile;
    if (u < ur) {
        tile = u / p.ntn_r;
        w.wt = u % p.ntn_r;
    } else {
        const int64_t v = u - ur;
        w.wt = v / ns;
        tile = nr + v % ns;
    }
    const int2 t = p.tiles[tile];
    const int g = t.x;
    w.m0 = t.y;
    if (g < p.N) {
        const int64_t rowbase = p.offsets[g];
        w.M = p.offsets[g + 1] - rowbase;
        w.K = p.K_r;
        w.Nout = p.Nout_r;
        w.X = (const char*)p.A_r + rowbase * w.K * ESZ;
        const int64_t wrows = mode == 0 ? 2 * w.Nout : w.Nout;
        w.W = (const char*)p.B_r + (int64_t)g * wrows * w.K * ESZ;
        w.C = (char*)p.C_r + rowbase * w.Nout * ESZ;
    } else {
        w.M = p.T;
        w.K = p.K_s;
        w.Nout = p.Nout_s;
        w.X = (const char*)p.A_s;
        w.W = (const char*)p.B_s;
        w.C = (char*)p.C_s;
    }
    return true;
}

__device__ __forceinline__ float silu_f(float a) { return a / (1.0f + __expf(-a)); }

template <int MODE>
__global__ void __launch_bounds__(G_THREADS, 1) ffn_gemm_bf16_kernel(GemmParamsV2 p) {
    WorkV2 w;
    if (!decode_v2<2>(p, MODE, w)) return;
    const uint16_t* Wp = (const uint16_t*)w.W;
    const uint16_t* Xp = (const uint16_t*)w.X;

    __shared__ __attribute__((aligned(1024))) uint16_t Aw0[G_WR * G_BK];
    __shared__ __attribute__((aligned(1024))) uint16_t Xt0[G_TR * G_BK];
    __shared__ __attribute__((aligned(1024))) uint16_t Aw1[G_WR * G_BK];
    __shared__ __attribute__((aligned(1024))) uint16_t Xt1[G_TR * G_BK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wg = wave & 3, tg = wave >> 2;
    const int64_t K = w.K;
    const int64_t mc = w.M - w.m0 < G_TR ? w.M - w.m0 : G_TR;  // token rows in this tile, >= 1

    // weight rows of this tile that exist (MODE 1 may end inside a tile)
    const int64_t wbase = MODE == 0 ? w.wt * 128 : w.wt * 256;
    // per-lane global sources for the 4 weight-chunk and 5 token-chunk copies
    const uint16_t* wsrc[4];
    const uint16_t* xsrc[5];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int slot = (wave * 4 + i) * 64 + lane;
        const int r = slot >> 3, c = (slot & 7) ^ (r & 7);
        int64_t wr;
        if (MODE == 0) {
            const int g4 = r >> 6, half = (r >> 5) & 1, j = r & 31;
            wr = (half ? w.Nout : 0) + wbase + g4 * 32 + j;
        } else {
            wr = wbase + r;
            if (wr >= w.Nout) wr = w.Nout - 1;  // clamp; never stored
        }
        wsrc[i] = Wp + wr * K + c * 8;
    }
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const int slot = (wave * 5 + i) * 64 + lane;
        const int r = slot >> 3, c = (slot & 7) ^ (r & 7);
        int64_t tr = w.m0 + (r < mc ? r : mc - 1);  // clamp; never stored
        xsrc[i] = Xp + tr * K + c * 8;
    }

    auto issue = [&](int64_t k0, uint16_t* Aw, uint16_t* Xt) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(wsrc[i] + k0),
                                             to_lds(Aw + (wave * 4 + i) * 512), 16, 0, 0);
#pragma unroll
        for (int i = 0; i < 5; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(xsrc[i] + k0),
                                             to_lds(Xt + (wave * 5 + i) * 512), 16, 0, 0);
    };

    f32x16_t acc[2][5];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 5; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // which 32-row blocks of this wave carry real rows (wave-uniform)
    bool t_on[5];
#pragma unroll
    for (int j = 0; j < 5; ++j) t_on[j] = tg * 160 + j * 32 < mc;
    const bool w_on = MODE == 0 ? true : (wbase + wg * 64 < w.Nout);

    const int nk = (int)(K / G_BK);
    issue(0, Aw0, Xt0);
    for (int kt = 0; kt < nk; ++kt) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();  // stage kt is in LDS; everyone is done with stage kt-1
        uint16_t* Aw = (kt & 1) ? Aw1 : Aw0;
        uint16_t* Xt = (kt & 1) ? Xt1 : Xt0;
        if (kt + 1 < nk) {
            if (kt & 1)
                issue((int64_t)(kt + 1) * G_BK, Aw0, Xt0);
            else
                issue((int64_t)(kt + 1) * G_BK, Aw1, Xt1);
        }
        if (w_on) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int ch = 2 * s + (lane >> 5);
                bf16x8_t af[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int r = wg * 64 + i * 32 + (lane & 31);
                    af[i] = __builtin_bit_cast(
                        bf16x8_t, *(const uint4*)(Aw + r * 64 + ((ch ^ (r & 7)) << 3)));
                }
#pragma unroll
                for (int j = 0; j < 5; ++j) {
                    if (!t_on[j]) continue;
                    const int r = tg * 160 + j * 32 + (lane & 31);
                    const bf16x8_t xf = __builtin_bit_cast(
                        bf16x8_t, *(const uint4*)(Xt + r * 64 + ((ch ^ (r & 7)) << 3)));
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], xf, acc[i][j],
                                                                             0, 0, 0);
                }
            }
        }
    }

    // epilogue.  32x32 accumulator layout: lane l holds column (token) l%32 and
    // rows (weight rows) 8*(v/4) + 4*(l/32) + v%4, v = 0..15.
    if (!w_on) return;
#pragma unroll
    for (int j = 0; j < 5; ++j) {
        if (!t_on[j]) continue;
        const int64_t t = w.m0 + tg * 160 + j * 32 + (lane & 31);
        if (t >= w.M) continue;
        uint16_t* crow = (uint16_t*)w.C + t * w.Nout;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int rr = 8 * g + 4 * (lane >> 5);
            if (MODE == 0) {
                const int64_t n = wbase + wg * 32 + rr;
                float h[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    h[q] = silu_f(acc[0][j][4 * g + q]) * acc[1][j][4 * g + q];
                *(uint2*)(crow + n) = make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
            } else {
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int64_t n = wbase + wg * 64 + i * 32 + rr;
                    *(uint2*)(crow + n) =
                        make_uint2(pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]),
                                   pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]));
                }
            }
        }
    }
}

// ---------------------------------------------------------------- fp32 path
// Plain VALU kernel for fp32 storage (small layers): 64 token rows x 64 output
// columns per 256-thread block; thread = (row tid%64, columns (tid/64)*16..+15).
template <int MODE>
__global__ void __launch_bounds__(256) ffn_gemm_f32_kernel(GemmParamsV2 p) {
    WorkV2 w;
    if (!decode_v2<4>(p, MODE, w)) return;
    const int tid = threadIdx.x;
    const int64_t r = w.m0 + (tid & 63);
    if (r >= w.M) return;
    const float* a = (const float*)w.X + r * w.K;
    const float* B = (const float*)w.W;
    float* C = (float*)w.C;
    const int64_t c0 = w.wt * 64 + (tid >> 6) * 16;
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
    int32_t* counts;  // [2]
    void* h_r;        // [TK, I]
    void* h_s;        // [T, Is]
    float* hs_r;      // FP8 scales [TK, I/128]
    float* hs_s;      // FP8 scales [T, Is/128]
};

static int ffn_bm(const moe_cfg& c) { return c.act_dtype == MOE_F32 ? F32_BM : BF_BM; }

static int64_t ffn_max_routed_tiles(const moe_cfg& c) {
    return c.tokens * c.top_k / ffn_bm(c) + c.n_experts;
}
static int64_t ffn_max_shared_tiles(const moe_cfg& c) { return cdiv(c.tokens, ffn_bm(c)); }

static int64_t h_elem_bytes(const moe_cfg& c) {
    return c.gemm_dtype == MOE_FP8_E4M3 ? 1 : (c.act_dtype == MOE_BF16 ? 2 : 4);
}

size_t ffn_workspace_bytes(const moe_cfg& c) {
    const int64_t TK = c.tokens * c.top_k, T = c.tokens;
    const int64_t eb = h_elem_bytes(c);
    int64_t b = align256((ffn_max_routed_tiles(c) + ffn_max_shared_tiles(c)) * 8) + 256;
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
    p += align256((ffn_max_routed_tiles(c) + ffn_max_shared_tiles(c)) * 8);
    w.counts = (int32_t*)p;
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
                                 const int32_t* counts, void* h_r, void* h_s, float* hs_r,
                                 float* hs_s, int64_t max_r, int64_t max_s, hipStream_t st);

hipError_t launch_expert_ffn(const moe_cfg& c, const FfnArgs& a, void* ws, hipStream_t st) {
    const int64_t T = c.tokens, TK = T * c.top_k;
    const bool has_shared = c.inter_shared > 0 && T > 0;
    if (TK == 0) return hipSuccess;
    FfnWs w = carve_ffn(c, ws);
    const int BM = ffn_bm(c);
    const int64_t max_r = ffn_max_routed_tiles(c);
    const int64_t max_s = has_shared ? ffn_max_shared_tiles(c) : 0;
    ffn_tile_map_kernel<<<1, 256, 0, st>>>(a.offsets, (int)c.n_experts, T, has_shared ? 1 : 0,
                                           BM, w.tiles, w.counts);
    if (c.gemm_dtype == MOE_FP8_E4M3)
        return launch_expert_ffn_fp8(c, a, w.tiles, w.counts, w.h_r, w.h_s, w.hs_r, w.hs_s,
                                     max_r, max_s, st);

    GemmParamsV2 p{};
    p.tiles = w.tiles;
    p.counts = w.counts;
    p.offsets = a.offsets;
    p.N = (int)c.n_experts;
    p.T = has_shared ? T : 0;
    const bool bf = c.act_dtype == MOE_BF16;

    // gate/up: token rows x W13 -> h  (bf16: 128 h columns per weight tile)
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
    const int cols0 = bf ? 128 : 64;
    p.ntn_r = (int)cdiv(c.inter, cols0);
    p.ntn_s = has_shared ? (int)cdiv(c.inter_shared, cols0) : 0;
    // every unit index the XCD mapping can produce must have a block: round
    // the bound on units up to a multiple of 8
    unsigned grid = (unsigned)(8 * cdiv(max_r * p.ntn_r + max_s * p.ntn_s, 8));
    if (bf)
        ffn_gemm_bf16_kernel<0><<<grid, G_THREADS, 0, st>>>(p);
    else
        ffn_gemm_f32_kernel<0><<<grid, 256, 0, st>>>(p);

    // down: h x W2 -> y  (bf16: 256 output columns per weight tile)
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
    const int cols1 = bf ? 256 : 64;
    p.ntn_r = (int)cdiv(c.hidden, cols1);
    p.ntn_s = has_shared ? (int)cdiv(c.hidden, cols1) : 0;
    grid = (unsigned)(8 * cdiv(max_r * p.ntn_r + max_s * p.ntn_s, 8));
    if (bf)
        ffn_gemm_bf16_kernel<1><<<grid, G_THREADS, 0, st>>>(p);
    else
        ffn_gemm_f32_kernel<1><<<grid, 256, 0, st>>>(p);
    return hipGetLastError();
}

}  // namespace moe
