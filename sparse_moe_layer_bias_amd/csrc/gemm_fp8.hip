// gemm_fp8.hip -- FP8 E4M3 grouped SwiGLU expert FFN (routed experts + the
// shared expert in the same launches).
//
// DeepSeek-V3 report reading guide (xyznot.com/de), "Kernideen", FP8 bullet:
// E4M3 operands with 1x128 activation tiles and 128x128 weight blocks, and the
// partial sums moved to FP32 every N_c = 128 accumulation steps.  Here every
// 128-wide contraction block k_b contributes P_b = sum_{k in k_b} qx*qw from
// two v_mfma_scale_f32_32x32x64_f8f6f4, scaled by s_x[row, k_b] *
// s_w[block, k_b] in fp32.  The block scales are arbitrary fp32 values
// (amax/448): the MFMA's power-of-two block-scale operands take their
// exponents and the VALU their significands (promotion, below).
// gate/up: h = silu(a) * b is quantised in the epilogue per 1x128 tile: a
// workgroup computes exactly 128 h columns (one tile) for each of its rows, so
// the tile amax is a reduction over the workgroup's 4 weight-row waves.
//
// Tiles: 256 weight rows x up to 320 token rows -- one weight panel against
// all rows of an expert, as in the bf16 kernel -- with 8 wavefronts (wg =
// wave%4 owns 64 weight rows = two 32-row blocks, tg = wave/4 owns 160 token
// rows = five blocks).  The contraction runs in steps of 128 (one scale
// block) through two LDS stages of 32 KB weight codes + 40 KB token codes +
// 1.25 KB token scales, copied global -> LDS directly.  LDS rows are 128 bytes
// with the chunk swizzle c ^ ((r >> 1) & 7); the weights are pre-packed in that
// order.
//
// Promotion: with the K block's scale split as sc_b = s_x * s_w =
// 2^(E_b) * m_b (E_b from the E8M0 codes of s_x and s_w, m_b the product of
// their significands, in [1, 4)), the accumulator holds R_b = S_b / m_b:
// R_b = R_{b-1} * (m_{b-1} / m_b) + 2^(E_b) * P_b.  The MFMA applies 2^(E_b)
// through its block-scale operands and adds into R directly; the VALU only
// rescales by the mantissa ratio, which stays within [1/4, 4], so no range is
// lost whatever the spread of the block scales.  S = R_last * m_last.  A zero
// scale (an all-zero tile or block: its codes are all zero) keeps the unit.
// One register set per output block (no separate partials) lets a wave hold
// five token blocks.
#include "gemm_common.h"

namespace moe {

constexpr int F8_TR = 320;                 // token rows per tile
constexpr int F8_KB = 128;                 // scale block along the contraction
constexpr int F8_BK = 128;                 // contraction step per stage = LDS row (bytes)
constexpr int F8_NS = 2;                   // LDS stages
constexpr int F8_WAVES = 8;
constexpr int F8_THREADS = 64 * F8_WAVES;
constexpr int F8_A = G_WR_PACK * F8_BK;    // bytes per stage: weight codes
constexpr int F8_X = F8_TR * F8_BK;        // token codes
constexpr int F8_S = F8_TR * 4;            // token scales of the step's scale block
static_assert(F8_BK == F8_KB, "one scale block per step");
constexpr int F8_STAGE = F8_A + F8_X + F8_S;

struct Fp8Params {
    GemmParamsV2 g;        // A: token codes, B: packed weight codes, C: h codes / y bf16
    const float* xs_r;     // token tile scales [rows][K/128], routed / shared
    const float* xs_s;
    const float* ws_r;     // weight block scales [mats][rows/128][K/128]
    const float* ws_s;
    float* hs_r;           // gate/up: h tile scales [rows][I/128]
    float* hs_s;
    int ws_t;              // weight scales indexed [mats][K/128][rows/128] (the
                           // block grid of the untransposed matrix: dgrad GEMMs)
    void* hb_r;            // modes 2 and 4: h in bf16 [rows][Nout]; a, b go to g.E
    void* hb_s;
    float* hf_r;           // modes 0 and 4, optional: h in fp32 before quantisation
    float* hf_s;
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

// LDS reads of 16-byte MFMA operand pieces by 32-bit LDS address
typedef __attribute__((address_space(3))) const i32x4_t lds_i32x4_t;

// A non-negative scale s as m * 2^(e8 - 127): e8 is s's biased exponent (the
// E8M0 code) and m in [1, 2) its significand; for s below 2^-126 (zero or
// subnormal) e8 = 0 and m = s * 2^127 in [0, 2), exact.
__device__ __forceinline__ void split_scale(float s, int& e8, float& m) {
    const uint32_t b = __float_as_uint(s);
    e8 = (int)(b >> 23);
    m = e8 ? __uint_as_float((b & 0x7fffffu) | 0x3f800000u) : s * 0x1p127f;
}

template <int MODE, int NB>
__device__ __forceinline__ void gemm_fp8_body(const Fp8Params& P, const WorkV2& w,
                                              uint8_t* smem) {
    constexpr int NA = F8_A / 1024, NX = F8_X / 1024;  // 1 KB copies per stage
    constexpr int PA = NA / F8_WAVES, PX = (NX + F8_WAVES - 1) / F8_WAVES;
    constexpr int NSC = F8_TR / 64;                      // dword copies for the scales
    constexpr int NBB = NB > 0 ? NB : 1;
    static_assert(NA % F8_WAVES == 0, "weight copies split evenly over the waves");

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wg = wave & 3, tg = wave >> 2;
    const int64_t K = w.K;
    const int64_t nkb = K / F8_KB;  // scale blocks
    const int nk = (int)(K / F8_BK);  // steps
    const int64_t mc = w.M - w.m0 < F8_TR ? w.M - w.m0 : F8_TR;
    const bool shared = w.g >= P.g.N;
    const int64_t gi = shared ? 0 : w.g;
    // with a gather list (inference forward) the routed rows are rows of the
    // shared expert's x codes and scales, found through src_token
    const int32_t* gat = w.gather;
    const float* xs = gat ? P.xs_r : (shared ? P.xs_s : P.xs_r) + (w.rowbase + w.m0) * nkb;
    const float* wsc = shared ? P.ws_s : P.ws_r;
    constexpr bool GU = MODE != 1;  // gate/up-shaped tile (modes 0 and 2)
    const int64_t wrows = GU ? 2 * w.Nout : w.Nout;
    const int64_t wrb = wrows / 128;  // 128-row scale blocks per expert matrix

    // Copies: global_load_lds from a wave-uniform base plus 32-bit lane
    // offsets, every address in bounds (token rows past the tile's last are
    // clamped to it): the tile's weight panel, the expert's token rows and
    // their scales.  (The compiler's own waits for these copies stay at the
    // step boundaries.  The buffer form of the instruction, as a builtin, made
    // it wait for every copy in flight before the first LDS read; written as
    // inline asm instead it measured 1% slower than this.)
    const char* wpanel = w.W + w.wt * (int64_t)nk * F8_A;
    const char* xbase = gat ? w.X : w.X + w.m0 * K;

    // token code copies: block b = 8 rows (128-byte lines); the blocks holding
    // real rows are the prefix b < nxe; rows past the last one repeat it
    const int nxe = (int)((mc + 7) / 8);
    uint32_t xoff[PX];
#pragma unroll
    for (int j = 0; j < PX; ++j) {
        const int b = wave + F8_WAVES * j;
        const int r = b * 8 + (lane >> 3), c = sub_chunk8(r, lane & 7);
        const int64_t tr = r < mc ? r : mc - 1;
        const int64_t sr = gat ? (int64_t)gat[w.m0 + tr] : tr;
        xoff[j] = (uint32_t)(sr * K + c * 16);
    }
    // token scale copies (dwords): wave s < NSC copies rows s*64 .. +63
    const int64_t srow0 = wave * 64 + lane < mc ? wave * 64 + lane : mc - 1;
    const int64_t srow = gat ? (int64_t)gat[w.m0 + srow0] : srow0;
    const uint32_t soff = (uint32_t)(srow * nkb * 4);

    auto stage = [&](int s) { return smem + s * F8_STAGE; };
    // this wave's copies for step kt into buffer s: weight blocks, token
    // blocks, then the token scales of the step's scale block
    auto issue = [&](int kt, int s) {
        uint8_t* As = stage(s);
        uint8_t* Xs = As + F8_A;
        uint8_t* Ss = Xs + F8_X;
        const char* wsrc = wpanel + (int64_t)kt * F8_A;
        const char* xsrc = xbase + (int64_t)kt * F8_BK;
#pragma unroll
        for (int c = 0; c < PA; ++c) {
            const int b = wave + F8_WAVES * c;
            __builtin_amdgcn_global_load_lds((const void*)(wsrc + b * 1024 + lane * 16),
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
            __builtin_amdgcn_global_load_lds((const void*)((const char*)xs + soff + kt * 4),
                                             to_lds(Ss + wave * 256), 4, 0, 0);
    };

    f32x16_t acc[2][NBB];
    float cur[2][NBB];  // the significand unit the accumulator is expressed in
    int ew[2], ex[NBB];  // E8M0 codes of the current scale block (weights, tokens)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NBB; ++j) {
            cur[i][j] = 1.0f;
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
        }

    // The weight block scales of the tile's two 128-row blocks for every K
    // block, staged in LDS once per tile.  (A global load per step would make
    // the step wait for the next stage's copies as well: vmcnt counts both.)
    // gate/up: block 0 = the W1 rows, block 1 = the W3 rows; down: the tile's
    // rows 0..127 and 128..255 (a wave's 64 rows lie in block wg/2).
    float* swl = (float*)(smem + F8_NS * F8_STAGE);
    {
        const int64_t b0 = GU ? w.wt : 2 * w.wt;
        const int64_t b1 = GU ? w.Nout / 128 + w.wt : 2 * w.wt + 1;
        for (int t = threadIdx.x; t < 2 * nkb; t += F8_THREADS) {
            const int64_t blk = t < nkb ? b0 : b1, kb = t < nkb ? t : t - nkb;
            swl[t] = blk < wrb ? wsc[P.ws_t ? (gi * nkb + kb) * wrb + blk : (gi * wrb + blk) * nkb + kb]
                               : 0.0f;
        }
    }

    // A 32x32x64 operand fragment: lane l holds 32 codes of row l % 32 of a
    // 32-row block, logical chunks 4q + 2h and 4q + 2h + 1 for K half q, with
    // h = l / 32.  Fragment rows are a multiple of 32 plus l % 32, so a row's
    // chunk swizzle (bits 1..3 of the row) is the lane's own: the byte offset
    // of each chunk is a per-lane constant, and every fragment read is a
    // stage base plus that offset plus an immediate.
    const int l32 = lane & 31;
    uint32_t co[2][2];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int b = 0; b < 2; ++b)
            co[q][b] = (uint32_t)(l32 * F8_BK + sub_chunk8(l32, 4 * q + 2 * (lane >> 5) + b) * 16);
    // p[q][b]: the lane's chunk in the stage's first fragment row block; a
    // block RB rows further is RB * F8_BK bytes on, an immediate offset
    auto frag = [&](const uint32_t (&p)[2][2], int q, int rowblk) {
        const i32x4_t lo = *(lds_i32x4_t*)(uintptr_t)(p[q][0] + rowblk * F8_BK);
        const i32x4_t hi = *(lds_i32x4_t*)(uintptr_t)(p[q][1] + rowblk * F8_BK);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };

    issue(0, 0);
    for (int kt = 0; kt < nk; ++kt) {
        vm_wait_n(0);
        __syncthreads();  // stage kt landed for every wave; stage kt-1 is free
        if (kt + 1 < nk) issue(kt + 1, (kt + 1) & 1);
        if constexpr (NB > 0) {
            const uint8_t* As = stage(kt & 1);
            const uint8_t* Xs = As + F8_A;
            const float* Ss = (const float*)(Xs + F8_X);
            // per-lane addresses, opaque to the compiler so that it keeps the
            // row block in the reads' immediate offsets
            const uint32_t la = (uint32_t)(uintptr_t)to_lds(As) + (wg * 2) * 32 * F8_BK;
            const uint32_t lx = (uint32_t)(uintptr_t)to_lds(Xs) + (tg * 160) * F8_BK;
            uint32_t pa[2][2], px[2][2];
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    pa[q][b] = la + co[q][b];
                    px[q][b] = lx + co[q][b];
                    asm volatile("" : "+v"(pa[q][b]), "+v"(px[q][b]));
                }
            // the two 64-wide K halves one after the other; the rescale to this
            // block's unit comes before the first half's MFMA
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                i32x8_t af[2];
                float mw[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    af[i] = frag(pa, q, i * 32);
                    if (q == 0) split_scale(swl[(GU ? i : wg >> 1) * nkb + kt], ew[i], mw[i]);
                }
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const int r = tg * 160 + j * 32 + l32;
                    const i32x8_t xf = frag(px, q, j * 32);
                    if (q == 0) {
                        float mx;
                        split_scale(Ss[r], ex[j], mx);
#pragma unroll
                        for (int i = 0; i < 2; ++i) {
                            const float mn = mw[i] * mx;
                            const float nw = mn == 0.0f ? cur[i][j] : mn;
                            const float ratio = cur[i][j] * __builtin_amdgcn_rcpf(nw);
                            cur[i][j] = nw;
#pragma unroll
                            for (int v = 0; v < 16; ++v) acc[i][j][v] *= ratio;
                        }
                    }
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            af[i], xf, acc[i][j], 0, 0, 0, ew[i], 0, ex[j]);
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
    if (MODE == 2 || MODE == 4) {
        // kept for the backward (mode 2: the backward's recompute; mode 4: the
        // training forward, which also quantises h below): a and b rounded to
        // bf16 into E ([rows][2 Nout], a row is [a | b]) and h = silu(a) * b
        // rounded to bf16 into hb ([rows][Nout]), straight from the
        // accumulators (4 columns per store)
        if constexpr (NB > 0) {
            uint16_t* hb = (uint16_t*)(shared ? P.hb_s : P.hb_r) + (w.rowbase + w.m0) * w.Nout;
            uint16_t* eb = (uint16_t*)(shared ? P.g.E_s : P.g.E_r) + (w.rowbase + w.m0) * 2 * w.Nout;
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int64_t rr = tg * 160 + j * 32 + (lane & 31);
                if (rr < mc) {
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const int64_t col = w.wt * 128 + wg * 32 + 8 * g4 + 4 * (lane >> 5);
                        float a[4], b[4];
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            a[v] = acc[0][j][4 * g4 + v];
                            b[v] = acc[1][j][4 * g4 + v];
                        }
                        *(uint2*)(eb + rr * 2 * w.Nout + col) =
                            make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
                        *(uint2*)(eb + rr * 2 * w.Nout + w.Nout + col) =
                            make_uint2(pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3]));
                        *(uint2*)(hb + rr * w.Nout + col) = make_uint2(
                            pack_bf16x2(silu_f(a[0]) * b[0], silu_f(a[1]) * b[1]),
                            pack_bf16x2(silu_f(a[2]) * b[2], silu_f(a[3]) * b[3]));
                    }
                }
            }
        }
    }
    if (MODE == 0 || MODE == 4) {
        // h = silu(a) * b for the tile's 128 columns, then 1x128 quantisation:
        // the tile amax is reduced over the 4 weight-row waves through LDS;
        // codes are staged in LDS and stored as whole 128-byte rows
        float* red = (float*)smem;          // [F8_TR rows][4 waves]
        constexpr int HST = 128 + 16;       // padded code row (bytes)
        uint8_t* hcodes = smem + F8_TR * 16;  // [F8_TR rows][HST]
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
        float* hf = shared ? P.hf_s : P.hf_r;
        if (hf != nullptr) {
            // the fp32 h values the quantisation below starts from (for checks
            // of the codes against an independent quantiser); 4 columns per store
            if constexpr (NB > 0) {
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const int64_t rr = tg * 160 + j * 32 + (lane & 31);
                    if (rr < mc) {
                        float* hrow = hf + (w.rowbase + w.m0 + rr) * w.Nout + w.wt * 128 + wg * 32 +
                                      4 * (lane >> 5);
#pragma unroll
                        for (int g4 = 0; g4 < 4; ++g4)
                            *(float4*)(hrow + 8 * g4) =
                                make_float4(hv[j][4 * g4], hv[j][4 * g4 + 1], hv[j][4 * g4 + 2],
                                            hv[j][4 * g4 + 3]);
                    }
                }
            }
        }
        __syncthreads();
        float* hsc = shared ? P.hs_s : P.hs_r;
        const int64_t ntile = w.Nout / 128;
        if constexpr (NB > 0) {
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int rr = tg * 160 + j * 32 + (lane & 31);
                const float4 mm = *(const float4*)(red + rr * 4);
                const float amax = fmaxf(fmaxf(mm.x, mm.y), fmaxf(mm.z, mm.w));
                const float scale = amax / 448.0f;
                // codes of clamp(h / scale) with the IEEE fp32 divide, as for
                // every other activation tile; an all-zero tile (scale 0) gets
                // codes 0
                float t[16];
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    t[v] = scale > 0.0f ? fminf(fmaxf(hv[j][v] / scale, -448.0f), 448.0f) : 0.0f;
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4)
                    *(uint32_t*)(hcodes + rr * HST + wg * 32 + 8 * g4 + 4 * (lane >> 5)) =
                        e4m3_encode4(t[4 * g4], t[4 * g4 + 1], t[4 * g4 + 2], t[4 * g4 + 3]);
                if (wg == 0 && lane < 32 && rr < mc) hsc[(w.rowbase + w.m0 + rr) * ntile + w.wt] = scale;
            }
        }
        __syncthreads();
        uint8_t* hq = (uint8_t*)(shared ? P.g.C_s : P.g.C_r) + (w.rowbase + w.m0) * w.Nout + w.wt * 128;
        for (int q = threadIdx.x; q < mc * 8; q += F8_THREADS) {
            const int rr = q >> 3, ch = q & 7;
            *(uint4*)(hq + rr * w.Nout + ch * 16) = *(const uint4*)(hcodes + rr * HST + ch * 16);
        }
    } else if (MODE == 1) {
        // y (bf16) through LDS in two token halves, stored as 16-byte row chunks
        constexpr int OSTR = 256 + 8;  // padded row (elements)
        uint16_t* ot = (uint16_t*)smem;
        uint16_t* y = (uint16_t*)(shared ? P.g.C_s : P.g.C_r) + w.rowbase * w.Nout;
        const int64_t wbase = w.wt * 256;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            if (half == 1) lds_barrier();  // the first half is read out of LDS
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
            lds_barrier();
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
    __shared__ __attribute__((aligned(1024))) uint8_t smem[F8_NS * F8_STAGE + 2 * 4 * FP8_MAX_KB];
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

// Pack the TRANSPOSE of FP8 weight codes [n_mats][K][Nout] (the forward's
// matrix, read column-wise) in the down-projection order of
// pack_weights_fp8_kernel<1>: packed row r of tile wt is column wt*256 + r.
// For the data-gradient GEMMs (W2^T: rows I, K = d; [W1; W3]^T: rows d,
// K = 2I); a one-off preparation, so the 16 codes of a chunk are gathered
// byte by byte.
__global__ void __launch_bounds__(256) pack_weights_fp8_t_kernel(const uint8_t* __restrict__ w,
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
    const int64_t src = packed_row_source<1>(wt, r, Nout);
    uint32_t v[4] = {0u, 0u, 0u, 0u};
    if (src >= 0) {
        const uint8_t* col = w + (mat * K + kt * F8_BK + c * 16) * Nout + src;
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e >> 2] |= (uint32_t)col[e * Nout] << (8 * (e & 3));
    }
    out[i] = make_uint4(v[0], v[1], v[2], v[3]);
}

// ---------------------------------------------------------------- launch

// which: 0/2 W13 and 1/3 W2 (routed / shared) for the forward; 4/6 [W1; W3]^T
// (rows d, K = 2I) and 5/7 W2^T (rows I, K = d) for the backward, packed from
// the forward's codes
static void fp8_pack_dims(const moe_cfg& c, int which, int64_t& n, int64_t& Nout, int64_t& K) {
    const bool routed = which == 0 || which == 1 || which == 4 || which == 5;
    n = routed ? c.n_experts : 1;
    const int64_t I = routed ? c.inter : c.inter_shared;
    if (which == 0 || which == 2) { Nout = I; K = c.hidden; }
    else if (which == 1 || which == 3) { Nout = c.hidden; K = I; }
    else if (which == 4 || which == 6) { Nout = c.hidden; K = 2 * I; }
    else { Nout = I; K = c.hidden; }
}

size_t packed_weight_bytes_fp8(const moe_cfg& c, int which) {
    int64_t n, Nout, K;
    fp8_pack_dims(c, which, n, Nout, K);
    if (which == 0 || which == 2) return (size_t)(n * cdiv(Nout, 128) * G_WR_PACK * K);
    return (size_t)(n * cdiv(Nout, 256) * G_WR_PACK * K);
}

hipError_t launch_pack_weights_fp8(const moe_cfg& c, int which, const void* w, void* out,
                                   hipStream_t st) {
    if (which >= 4) {
        int64_t n, Nout, K;
        fp8_pack_dims(c, which, n, Nout, K);
        const int64_t ntn = cdiv(Nout, 256);
        const int64_t total = n * ntn * (K / F8_BK) * G_WR_PACK * 8;
        if (total == 0) return hipSuccess;
        pack_weights_fp8_t_kernel<<<(unsigned)cdiv(total, 256), 256, 0, st>>>(
            (const uint8_t*)w, (uint4*)out, n, Nout, K, ntn);
        return hipGetLastError();
    }
    const bool routed = which == 0 || which == 1;
    const int64_t n = routed ? c.n_experts : 1;
    const int64_t I = routed ? c.inter : c.inter_shared;
    const bool up = which == 0 || which == 2;
    const int64_t Nout = up ? I : c.hidden, K = up ? c.hidden : I;
    const int64_t ntn = up ? cdiv(I, 128) : cdiv(c.hidden, 256);
    const int64_t total = n * ntn * (K / F8_BK) * G_WR_PACK * (F8_BK / 16);
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
                                 const int32_t* counts, const int32_t* order, void* h_r, void* h_s, float* hs_r,
                                 float* hs_s, int64_t max_r, int64_t max_s, hipStream_t st,
                                 const SavedActs* sv, float* hf_r, float* hf_s) {
    const int64_t T = c.tokens;
    const bool has_shared = c.inter_shared > 0 && T > 0;
    Fp8Params P{};
    P.g.tiles = tiles;
    P.g.counts = counts;
    P.g.order = order;
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
    P.g.gather_r = a.gather;  // inference forward, optional: routed rows = x_q[src_token]
    P.ws_r = a.w13_scale;
    P.ws_s = a.ws13_scale;
    P.hs_r = hs_r;
    P.hs_s = hs_s;
    P.hf_r = hf_r;
    P.hf_s = has_shared ? hf_s : nullptr;
    P.g.ntn_r = (int)(c.inter / 128);
    P.g.ntn_s = has_shared ? (int)(c.inter_shared / 128) : 0;
    unsigned grid = (unsigned)ffn_grid_blocks(max_r, P.g.ntn_r, max_s, P.g.ntn_s);
    if (sv) {  // training forward: also a, b and h in bf16 for the backward
        P.g.E_r = sv->ab_r;
        P.g.E_s = sv->ab_s;
        P.hb_r = sv->h_r;
        P.hb_s = sv->h_s;
        ffn_gemm_fp8_kernel<4><<<grid, F8_THREADS, 0, st>>>(P);
        P.g.E_r = P.g.E_s = P.hb_r = P.hb_s = nullptr;
    } else {
        ffn_gemm_fp8_kernel<0><<<grid, F8_THREADS, 0, st>>>(P);
    }

    // down: h codes x W2 codes -> y (bf16)
    P.g.gather_r = nullptr;
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
    P.hf_r = P.hf_s = nullptr;
    P.g.ntn_r = (int)cdiv(c.hidden, 256);
    P.g.ntn_s = has_shared ? (int)cdiv(c.hidden, 256) : 0;
    grid = (unsigned)ffn_grid_blocks(max_r, P.g.ntn_r, max_s, P.g.ntn_s);
    ffn_gemm_fp8_kernel<1><<<grid, F8_THREADS, 0, st>>>(P);
    return hipGetLastError();
}

hipError_t launch_fp8_gemm(const Fp8Gemm& op, const int2* tiles, const int32_t* counts,
                           const int32_t* order, const int32_t* offsets, int N, int64_t T_shared,
                           int64_t max_r, int64_t max_s, hipStream_t st) {
    Fp8Params P{};
    P.g.tiles = tiles;
    P.g.counts = counts;
    P.g.order = order;
    P.g.offsets = offsets;
    P.g.N = N;
    P.g.T = T_shared;
    P.g.K_r = op.K_r;
    P.g.K_s = op.K_s;
    P.g.Nout_r = op.Nout_r;
    P.g.Nout_s = op.Nout_s;
    P.g.A_r = op.A_r;
    P.g.A_s = op.A_s;
    P.g.B_r = op.B_r;
    P.g.B_s = op.B_s;
    P.g.C_r = op.C_r;
    P.g.C_s = op.C_s;
    P.g.E_r = op.E_r;
    P.g.E_s = op.E_s;
    P.xs_r = op.as_r;
    P.xs_s = op.as_s;
    P.ws_r = op.bs_r;
    P.ws_s = op.bs_s;
    P.ws_t = op.bs_t;
    const int cols = op.mode == 1 ? 256 : 128;
    P.g.ntn_r = (int)cdiv(op.Nout_r, cols);
    P.g.ntn_s = T_shared > 0 ? (int)cdiv(op.Nout_s, cols) : 0;
    const unsigned grid = (unsigned)ffn_grid_blocks(max_r, P.g.ntn_r, max_s, P.g.ntn_s);
    if (op.mode == 2) {
        P.g.C_r = P.g.C_s = nullptr;
        P.hb_r = op.C_r;
        P.hb_s = op.C_s;
        ffn_gemm_fp8_kernel<2><<<grid, F8_THREADS, 0, st>>>(P);
    }
    else
        ffn_gemm_fp8_kernel<1><<<grid, F8_THREADS, 0, st>>>(P);
    return hipGetLastError();
}

}  // namespace moe
