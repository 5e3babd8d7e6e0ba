// gemm_fp8.hip -- FP8 E4M3 grouped SwiGLU expert FFN (routed experts + the
// shared expert in the same launches).
//
// DeepSeek-V3 report reading guide (xyznot.com/de), "Kernideen", FP8 bullet:
// E4M3 operands with 1x128 activation tiles and 128x128 weight blocks, and the
// partial sums moved to FP32 every N_c = 128 accumulation steps.  Here every
// 128-wide contraction block k_b contributes P_b = sum_{k in k_b} qx*qw from
// two v_mfma_f32_32x32x64_f8f6f4, scaled by s_x[row, k_b] * s_w[block, k_b] in
// fp32 -- the block scales are arbitrary fp32 values (amax/448), which the
// hardware's power-of-two block scales cannot express.
// gate/up: h = silu(a) * b is quantised in the epilogue per 1x128 tile: a
// workgroup computes exactly 128 h columns (one tile) for each of its rows, so
// the tile amax is a reduction over the workgroup's 4 weight-row waves.
//
// Tiles: 256 weight rows x up to 320 token rows -- one weight panel against
// all rows of an expert, as in the bf16 kernel -- with 8 wavefronts (wg =
// wave%4 owns 64 weight rows = two 32-row blocks, tg = wave/4 owns 160 token
// rows = five blocks).  K step 128 = one scale block; two LDS stages of
// 32 KB weight codes + 40 KB token codes + 1.25 KB token scales, copied
// global -> LDS directly.  LDS rows are 128 bytes (the 128 codes of a K step)
// with the bf16 kernel's chunk swizzle; weights are pre-packed in that order.
//
// Promotion in place: with sc_b = s_x[row, b] * s_w[block, b] the accumulator
// holds R_b = S_b / sc_b, i.e. R_b = R_{b-1} * (sc_{b-1} / sc_b) + P_b, where the
// MFMAs add P_b directly into R.  The result is S = R_last * sc_last.  A zero
// scale (an all-zero tile or block, whose codes are all zero, so P_b = 0)
// keeps the previous scale.  This keeps one register set per output block
// (no separate partials), which is what lets a wave hold 5 token blocks.
#include "gemm_common.h"

namespace moe {

constexpr int F8_TR = 320;                 // token rows per tile
constexpr int F8_BK = 128;                 // contraction step = scale block = LDS row (bytes)
constexpr int F8_WAVES = 8;
constexpr int F8_THREADS = 64 * F8_WAVES;
constexpr int F8_A = G_WR_PACK * F8_BK;    // bytes per stage: weight codes
constexpr int F8_X = F8_TR * F8_BK;        // token codes
constexpr int F8_S = F8_TR * 4;            // token scales
constexpr int F8_STAGE = F8_A + F8_X + F8_S;

struct Fp8Params {
    GemmParamsV2 g;        // A: token codes, B: packed weight codes, C: h codes / y bf16
    const float* xs_r;     // token tile scales [rows][K/128], routed / shared
    const float* xs_s;
    const float* ws_r;     // weight block scales [mats][rows/128][K/128]
    const float* ws_s;
    float* hs_r;           // gate/up: h tile scales [rows][I/128]
    float* hs_s;
};

// Pack FP8 weight codes [n_mats][rows][K] into the kernel's LDS image order:
// out[mat][wt][kt][slot] (16-byte chunks), kt = 128-wide contraction step,
// slot = r*8 + pc holding logical chunk sub_chunk8(r, pc) of packed row r.
template <int MODE>
__global__ void __launch_bounds__(256) pack_weights_fp8_kernel(const uint4* __restrict__ w,
                                                               uint4* __restrict__ out,
                                                               int64_t n_mats, int64_t Nout,
                                                               int64_t K, int64_t ntn) {
    const int64_t nkt = K / F8_BK;
    const int64_t per_mat = ntn * nkt * G_WR_PACK * 8;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_mats * per_mat) return;
    const int64_t mat = i / per_mat;
    int64_t rem = i % per_mat;
    const int64_t wt = rem / (nkt * G_WR_PACK * 8);
    rem %= nkt * G_WR_PACK * 8;
    const int64_t kt = rem / (G_WR_PACK * 8);
    const int slot = (int)(rem % (G_WR_PACK * 8));
    const int r = slot >> 3, c = sub_chunk8(r, slot & 7);
    const int64_t src = packed_row_source<MODE>(wt, r, Nout);
    const int64_t rows = MODE == 0 ? 2 * Nout : Nout;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (src >= 0) v = w[((mat * rows + src) * K + kt * F8_BK + c * 16) / 16];
    out[i] = v;
}

// 32 codes of one 128-byte LDS row for k-half q: logical chunks 4q + 2*(lane/32), +1
__device__ __forceinline__ i32x8_t ld_frag32(const uint8_t* rowp, int r, int c0) {
    const uint4 lo = *(const uint4*)(rowp + sub_chunk8(r, c0) * 16);
    const uint4 hi = *(const uint4*)(rowp + sub_chunk8(r, c0 + 1) * 16);
    i32x8_t v;
    v[0] = (int)lo.x; v[1] = (int)lo.y; v[2] = (int)lo.z; v[3] = (int)lo.w;
    v[4] = (int)hi.x; v[5] = (int)hi.y; v[6] = (int)hi.z; v[7] = (int)hi.w;
    return v;
}

template <int MODE, int NB>
__device__ __forceinline__ void gemm_fp8_body(const Fp8Params& P, const WorkV2& w,
                                              uint8_t* smem) {
    constexpr int NA = F8_A / 1024, NX = F8_X / 1024;  // 1 KB copies per stage
    constexpr int PA = NA / F8_WAVES, PX = (NX + F8_WAVES - 1) / F8_WAVES;
    constexpr int NSC = F8_TR / 64;                      // dword copies for the scales
    constexpr int NBB = NB > 0 ? NB : 1;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wg = wave & 3, tg = wave >> 2;
    const int64_t K = w.K;
    const int64_t nkb = K / F8_BK;
    const int64_t mc = w.M - w.m0 < F8_TR ? w.M - w.m0 : F8_TR;
    const int nk = (int)nkb;
    const bool shared = w.g >= P.g.N;
    const int64_t gi = shared ? 0 : w.g;
    const float* xs = (shared ? P.xs_s : P.xs_r) + (w.rowbase + w.m0) * nkb;
    const float* wsc = shared ? P.ws_s : P.ws_r;
    const int64_t wrows = MODE == 0 ? 2 * w.Nout : w.Nout;
    const int64_t wrb = wrows / 128;  // 128-row scale blocks per expert matrix

    const char* wstage0 = w.W + w.wt * (int64_t)nk * F8_A;
    const uint32_t woff = lane * 16;
    const char* xbase = w.X + w.m0 * K;

    // token code copies: block b = 8 rows (one 128-byte line each); the blocks
    // holding real rows are the prefix b < nxe
    const int nxe = (int)((mc + 7) / 8);
    uint32_t xoff[PX];
#pragma unroll
    for (int j = 0; j < PX; ++j) {
        const int b = wave + F8_WAVES * j;
        const int r = b * 8 + (lane >> 3), c = sub_chunk8(r, lane & 7);
        const int64_t tr = r < mc ? r : mc - 1;
        xoff[j] = (uint32_t)(tr * K + c * 16);
    }
    // token scale copies (dwords): wave s < NSC copies rows s*64 .. +63
    const int64_t srow = wave * 64 + lane < mc ? wave * 64 + lane : mc - 1;
    const float* ssrc0 = xs + srow * nkb;

    auto stage = [&](int s) { return smem + s * F8_STAGE; };
    auto issue = [&](int kt, int s) {
        uint8_t* As = stage(s);
        uint8_t* Xs = As + F8_A;
        uint8_t* Ss = Xs + F8_X;
        const char* wsrc = wstage0 + (int64_t)kt * F8_A;
        const char* xsrc = xbase + (int64_t)kt * F8_BK;
#pragma unroll
        for (int j = 0; j < PA; ++j) {
            const int b = wave + F8_WAVES * j;
            __builtin_amdgcn_global_load_lds((const void*)(wsrc + b * 1024 + woff),
                                             to_lds(As + b * 1024), 16, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < PX; ++j) {
            const int b = wave + F8_WAVES * j;
            if (b < nxe)
                __builtin_amdgcn_global_load_lds((const void*)(xsrc + xoff[j]),
                                                 to_lds(Xs + b * 1024), 16, 0, 0);
        }
        if (wave < NSC)
            __builtin_amdgcn_global_load_lds((const void*)(ssrc0 + kt), to_lds(Ss + wave * 256),
                                             4, 0, 0);
    };

    f32x16_t acc[2][NBB];
    float cur[2][NBB];  // the scale the accumulator is currently expressed in
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NBB; ++j) {
            cur[i][j] = 1.0f;
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
        }

    // weight-scale block of each of this wave's two 32-row blocks
    int64_t wblk[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        if (MODE == 0)
            wblk[i] = (i ? w.Nout / 128 : 0) + w.wt;  // W1 rows, then the W3 rows
        else
            wblk[i] = w.wt * 2 + (wg >> 1);
    }

    issue(0, 0);
    for (int kt = 0; kt < nk; ++kt) {
        vm_wait_n(0);
        __syncthreads();  // stage kt landed for every wave; stage kt-1 is free
        if (kt + 1 < nk) issue(kt + 1, (kt + 1) & 1);
        if constexpr (NB > 0) {
            __builtin_amdgcn_iglp_opt(1);
            const uint8_t* As = stage(kt & 1);
            const uint8_t* Xs = As + F8_A;
            const float* Ss = (const float*)(Xs + F8_X);
            float sw[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) sw[i] = wsc[(gi * wrb + wblk[i]) * nkb + kt];
            i32x8_t af[2][2];
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int r = (wg * 2 + i) * 32 + (lane & 31);
                    af[q][i] = ld_frag32(As + r * F8_BK, r, 4 * q + 2 * (lane >> 5));
                }
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int r = tg * 160 + j * 32 + (lane & 31);
                const i32x8_t x0 = ld_frag32(Xs + r * F8_BK, r, 2 * (lane >> 5));
                const i32x8_t x1 = ld_frag32(Xs + r * F8_BK, r, 4 + 2 * (lane >> 5));
                const float sx = Ss[r];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const float sc = sw[i] * sx;
                    const float nw = sc == 0.0f ? cur[i][j] : sc;
                    const float ratio = cur[i][j] / nw;
                    cur[i][j] = nw;
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[i][j][v] *= ratio;
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[0][i], x0, acc[i][j],
                                                                                0, 0, 0, 0, 0, 0);
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[1][i], x1, acc[i][j],
                                                                                0, 0, 0, 0, 0, 0);
                }
            }
        }
    }
    // back to absolute values
    if constexpr (NB > 0) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] *= cur[i][j];
    }

    // epilogue.  32x32 accumulator layout: lane l holds column (token) l%32 and
    // rows (weight rows) 8*(v/4) + 4*(l/32) + v%4, v = 0..15.
    __syncthreads();  // every wave is done with the stage buffers
    if (MODE == 0) {
        // h = silu(a) * b for the tile's 128 columns, then 1x128 quantisation:
        // amax over the 4 weight-row waves through LDS
        float* red = (float*)smem;  // [F8_TR rows][4 waves]
        float hv[NBB][16];
#pragma unroll
        for (int j = 0; j < NBB; ++j) {
            float m = 0.0f;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                hv[j][v] = NB > 0 ? silu_f(acc[0][j][v]) * acc[1][j][v] : 0.0f;
                m = fmaxf(m, fabsf(hv[j][v]));
            }
            m = fmaxf(m, __shfl_xor(m, 32, 64));
            if (NB > 0 && lane < 32) red[(tg * 160 + j * 32 + lane) * 4 + wg] = m;
        }
        __syncthreads();
        if constexpr (NB > 0) {
            uint8_t* hq = (uint8_t*)(shared ? P.g.C_s : P.g.C_r);
            float* hsc = shared ? P.hs_s : P.hs_r;
            const int64_t ntile = w.Nout / 128;
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int rr = tg * 160 + j * 32 + (lane & 31);
                const int64_t t = w.m0 + rr;
                if (t >= w.M) continue;
                const float4 mm = *(const float4*)(red + rr * 4);
                const float amax = fmaxf(fmaxf(mm.x, mm.y), fmaxf(mm.z, mm.w));
                const float scale = amax / 448.0f;
                const int64_t row = w.rowbase + t;
                uint8_t* hrow = hq + row * w.Nout + w.wt * 128 + wg * 32;
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    uint32_t q = 0;
#pragma unroll
                    for (int u = 0; u < 4; ++u) q |= quant_e4m3(hv[j][4 * g4 + u], scale) << (8 * u);
                    *(uint32_t*)(hrow + 8 * g4 + 4 * (lane >> 5)) = q;
                }
                if (wg == 0 && lane < 32) hsc[row * ntile + w.wt] = scale;
            }
        }
    } else {
        // y (bf16) through LDS in two token halves, stored as 16-byte row chunks
        constexpr int OSTR = 256 + 8;  // padded row (elements)
        uint16_t* ot = (uint16_t*)smem;
        uint16_t* y = (uint16_t*)(shared ? P.g.C_s : P.g.C_r) + w.rowbase * w.Nout;
        const int64_t wbase = w.wt * 256;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            if (half == 1) __syncthreads();
            if constexpr (NB > 0) {
                if (tg == half) {
#pragma unroll
                    for (int j = 0; j < NB; ++j) {
                        const int row = j * 32 + (lane & 31);
#pragma unroll
                        for (int g4 = 0; g4 < 4; ++g4) {
                            const int rr = 8 * g4 + 4 * (lane >> 5);
#pragma unroll
                            for (int i = 0; i < 2; ++i)
                                *(uint2*)(ot + row * OSTR + (wg * 2 + i) * 32 + rr) = make_uint2(
                                    pack_bf16x2(acc[i][j][4 * g4], acc[i][j][4 * g4 + 1]),
                                    pack_bf16x2(acc[i][j][4 * g4 + 2], acc[i][j][4 * g4 + 3]));
                        }
                    }
                }
            }
            __syncthreads();
            const int nrows = (int)(mc - half * 160 < 160 ? mc - half * 160 : 160);
            for (int q = threadIdx.x; q < nrows * 32; q += F8_THREADS) {
                const int rr = q / 32, ch = q % 32;
                const int64_t col = wbase + ch * 8;
                if (col < w.Nout)
                    *(uint4*)(y + (w.m0 + half * 160 + rr) * w.Nout + col) =
                        *(const uint4*)(ot + rr * OSTR + ch * 8);
            }
        }
    }
}

template <int MODE>
__global__ void __launch_bounds__(F8_THREADS, 1) ffn_gemm_fp8_kernel(Fp8Params P) {
    WorkV2 w;
    if (!decode_v2<1>(P.g, MODE, w)) return;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * F8_STAGE];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wg = wave & 3, tg = wave >> 2;
    const int64_t mc = w.M - w.m0 < F8_TR ? w.M - w.m0 : F8_TR;
    int64_t nb = (mc - tg * 160 + 31) / 32;
    nb = nb < 0 ? 0 : (nb > 5 ? 5 : nb);
    if (MODE == 1 && w.wt * 256 + wg * 64 >= w.Nout) nb = 0;
    switch (nb) {
        case 5: gemm_fp8_body<MODE, 5>(P, w, smem); break;
        case 4: gemm_fp8_body<MODE, 4>(P, w, smem); break;
        case 3: gemm_fp8_body<MODE, 3>(P, w, smem); break;
        case 2: gemm_fp8_body<MODE, 2>(P, w, smem); break;
        case 1: gemm_fp8_body<MODE, 1>(P, w, smem); break;
        default: gemm_fp8_body<MODE, 0>(P, w, smem); break;
    }
}

// ---------------------------------------------------------------- launch

size_t packed_weight_bytes_fp8(const moe_cfg& c, int which) {
    const bool routed = which == 0 || which == 1;
    const int64_t n = routed ? c.n_experts : 1;
    const int64_t I = routed ? c.inter : c.inter_shared;
    if (which == 0 || which == 2) return (size_t)(n * cdiv(I, 128) * G_WR_PACK * c.hidden);
    return (size_t)(n * cdiv(c.hidden, 256) * G_WR_PACK * I);
}

hipError_t launch_pack_weights_fp8(const moe_cfg& c, int which, const void* w, void* out,
                                   hipStream_t st) {
    const bool routed = which == 0 || which == 1;
    const int64_t n = routed ? c.n_experts : 1;
    const int64_t I = routed ? c.inter : c.inter_shared;
    const bool up = which == 0 || which == 2;
    const int64_t Nout = up ? I : c.hidden, K = up ? c.hidden : I;
    const int64_t ntn = up ? cdiv(I, 128) : cdiv(c.hidden, 256);
    const int64_t total = n * ntn * (K / F8_BK) * G_WR_PACK * 8;
    if (total == 0) return hipSuccess;
    const unsigned blocks = (unsigned)cdiv(total, 256);
    if (up)
        pack_weights_fp8_kernel<0><<<blocks, 256, 0, st>>>((const uint4*)w, (uint4*)out, n, Nout,
                                                           K, ntn);
    else
        pack_weights_fp8_kernel<1><<<blocks, 256, 0, st>>>((const uint4*)w, (uint4*)out, n, Nout,
                                                           K, ntn);
    return hipGetLastError();
}

hipError_t launch_expert_ffn_fp8(const moe_cfg& c, const FfnArgs& a, const int2* tiles,
                                 const int32_t* counts, void* h_r, void* h_s, float* hs_r,
                                 float* hs_s, int64_t max_r, int64_t max_s, hipStream_t st) {
    const int64_t T = c.tokens;
    const bool has_shared = c.inter_shared > 0 && T > 0;
    Fp8Params P{};
    P.g.tiles = tiles;
    P.g.counts = counts;
    P.g.offsets = a.offsets;
    P.g.N = (int)c.n_experts;
    P.g.T = has_shared ? T : 0;

    // gate/up: token codes x W13 codes -> h codes + h tile scales
    P.g.K_r = c.hidden;
    P.g.K_s = c.hidden;
    P.g.Nout_r = c.inter;
    P.g.Nout_s = c.inter_shared;
    P.g.A_r = a.x_perm;
    P.g.A_s = a.x_sh;
    P.g.B_r = a.w13;
    P.g.B_s = a.ws13;
    P.g.C_r = h_r;
    P.g.C_s = h_s;
    P.xs_r = a.x_perm_scale;
    P.xs_s = a.x_sh_scale;
    P.ws_r = a.w13_scale;
    P.ws_s = a.ws13_scale;
    P.hs_r = hs_r;
    P.hs_s = hs_s;
    P.g.ntn_r = (int)(c.inter / 128);
    P.g.ntn_s = has_shared ? (int)(c.inter_shared / 128) : 0;
    unsigned grid = (unsigned)(8 * cdiv(max_r * P.g.ntn_r + max_s * P.g.ntn_s, 8));
    ffn_gemm_fp8_kernel<0><<<grid, F8_THREADS, 0, st>>>(P);

    // down: h codes x W2 codes -> y (bf16)
    P.g.K_r = c.inter;
    P.g.K_s = c.inter_shared;
    P.g.Nout_r = c.hidden;
    P.g.Nout_s = c.hidden;
    P.g.A_r = h_r;
    P.g.A_s = h_s;
    P.g.B_r = a.w2;
    P.g.B_s = a.ws2;
    P.g.C_r = a.y_perm;
    P.g.C_s = a.y_shared;
    P.xs_r = hs_r;
    P.xs_s = hs_s;
    P.ws_r = a.w2_scale;
    P.ws_s = a.ws2_scale;
    P.hs_r = nullptr;
    P.hs_s = nullptr;
    P.g.ntn_r = (int)cdiv(c.hidden, 256);
    P.g.ntn_s = has_shared ? (int)cdiv(c.hidden, 256) : 0;
    grid = (unsigned)(8 * cdiv(max_r * P.g.ntn_r + max_s * P.g.ntn_s, 8));
    ffn_gemm_fp8_kernel<1><<<grid, F8_THREADS, 0, st>>>(P);
    return hipGetLastError();
}

}  // namespace moe
