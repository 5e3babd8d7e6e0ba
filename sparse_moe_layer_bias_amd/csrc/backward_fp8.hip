// backward_fp8.hip -- FP8 E4M3 backward of the grouped SwiGLU experts.
//
// DeepSeek-V3 report reading guide (xyznot.com/de), "Kernideen", FP8 bullet:
// E4M3 for all tensors, 1x128 activation tiles, 128x128 weight blocks, FP32
// promotion every 128 accumulation steps.  Applied to the backward GEMMs, each
// operand is quantised along that GEMM's contraction:
//   dh  = dY W2            dY in 1x128 row tiles x W2's blocks (transposed pack)
//   da, db from dh and the recomputed a, b (bf16), then [da db] in 1x128 tiles
//   dX  = [da db] [W1; W3]  on the forward's FP8 kernel (mode 1, transposed pack)
//   dW2 = dY^T h,  dW13 = [da db]^T X: contraction over an expert's rows, so
//         dY, h, [da db] and X are quantised in 128x1 tiles down the rows (128
//         consecutive rows of one expert from its first, the last partial)
// a, b and h come from an FP8 gate/up recompute (mode 2), kept in bf16; dh, da,
// db and every output are rounded to bf16.
//
// The row-direction tiles are written transposed and block-major: the codes of
// 128-row block pb (blocks numbered along poff = prefix of the groups' row
// counts rounded up to 128, the shared expert last) are [pb][feature][128], so
// that the weight-gradient GEMM reads each operand tile of a block as one
// contiguous run of 128-byte rows along its contraction.
#include "gemm_common.h"

namespace moe {

static int64_t a256(int64_t b) { return (b + 255) & ~int64_t(255); }
static int64_t r128(int64_t b) { return (b + 127) & ~int64_t(127); }

// ---------------------------------------------------------------- row tiles

// bf16 rows [rows][C] -> E4M3 codes [rows][C] + 1x128 scales [rows][C/128];
// 16 lanes per tile, 8 values per lane
__global__ void __launch_bounds__(256) quant_rows_bf16_kernel(const uint4* __restrict__ x,
                                                              int64_t rows, int64_t C,
                                                              uint2* __restrict__ q,
                                                              float* __restrict__ s) {
    const int64_t tiles = C / 128;
    const int64_t tile = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int l = threadIdx.x & 15;
    const bool valid = tile < rows * tiles;  // uniform over each 16-lane group
    const int64_t v = (valid ? tile : 0) * 16 + l;  // 8-element vector index
    const uint4 val = valid ? x[v] : make_uint4(0, 0, 0, 0);
    const uint32_t w[4] = {val.x, val.y, val.z, val.w};
    float f[8];
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
        q[v] = make_uint2(lo, hi);
        if (l == 0) s[tile] = scale;
    }
}

// SwiGLU backward of rows [rows] with I columns: from dh [rows][I] and the
// recompute's [a | b] [rows][2I] (bf16), da = dh b s (1 + a (1 - s)) and
// db = dh a s (s = sigmoid(a)) rounded to bf16 into dab = [da | db]
// [rows][2I], and the 1x128 tiles of those bf16 values: codes [rows][2I],
// scales [rows][2I/128].  16 lanes per (row, 128-column block of I): the da
// tile and the db tile of the same columns.
__global__ void __launch_bounds__(256) swiglu_bwd_fp8_kernel(
    const uint4* __restrict__ dh, const uint4* __restrict__ ab, int64_t rows, int64_t I,
    uint4* __restrict__ dab, uint2* __restrict__ q, float* __restrict__ s) {
    const int64_t nj = I / 128;
    const int64_t unit = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int l = threadIdx.x & 15;
    const bool valid = unit < rows * nj;
    const int64_t u = valid ? unit : 0;
    const int64_t r = u / nj, j = u % nj;
    const int64_t vh = (r * I + j * 128) / 8 + l;            // dh vector
    const int64_t va = (r * 2 * I + j * 128) / 8 + l;        // a vector; b at + I/8
    const uint4 qh = dh[vh], qa = ab[va], qb = ab[va + I / 8];
    const uint32_t wh[4] = {qh.x, qh.y, qh.z, qh.w};
    const uint32_t wa[4] = {qa.x, qa.y, qa.z, qa.w};
    const uint32_t wb[4] = {qb.x, qb.y, qb.z, qb.w};
    float da[8], db[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int k = i >> 1;
        const uint32_t sh = (i & 1) ? 0 : 16;
        const uint32_t mk = 0xffff0000u;
        const float h = __uint_as_float((wh[k] << sh) & mk);
        const float a = __uint_as_float((wa[k] << sh) & mk);
        const float b = __uint_as_float((wb[k] << sh) & mk);
        const float sg = 1.0f / (1.0f + expf(-a));
        // rounded to bf16 here: the tiles quantise the stored values
        da[i] = bf16_to_f32(f32_to_bf16(h * b * sg * (1.0f + a * (1.0f - sg))));
        db[i] = bf16_to_f32(f32_to_bf16(h * a * sg));
    }
    float ma = 0.0f, mb = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        ma = fmaxf(ma, fabsf(da[i]));
        mb = fmaxf(mb, fabsf(db[i]));
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
        ma = fmaxf(ma, __shfl_xor(ma, m, 64));
        mb = fmaxf(mb, __shfl_xor(mb, m, 64));
    }
    const float sa = ma / 448.0f, sb = mb / 448.0f;
    uint32_t ca[2] = {0u, 0u}, cb[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        ca[i >> 2] |= quant_e4m3(da[i], sa) << (8 * (i & 3));
        cb[i >> 2] |= quant_e4m3(db[i], sb) << (8 * (i & 3));
    }
    if (valid) {
        dab[va] = make_uint4(pack_bf16x2(da[0], da[1]), pack_bf16x2(da[2], da[3]),
                             pack_bf16x2(da[4], da[5]), pack_bf16x2(da[6], da[7]));
        dab[va + I / 8] = make_uint4(pack_bf16x2(db[0], db[1]), pack_bf16x2(db[2], db[3]),
                                     pack_bf16x2(db[4], db[5]), pack_bf16x2(db[6], db[7]));
        const int64_t qv = (r * 2 * I + j * 128) / 8 + l;
        q[qv] = make_uint2(ca[0], ca[1]);
        q[qv + I / 8] = make_uint2(cb[0], cb[1]);
        if (l == 0) {
            s[r * 2 * nj + j] = sa;
            s[r * 2 * nj + nj + j] = sb;
        }
    }
}

// ---------------------------------------------------------------- row-direction tiles

// poff[g] = sum over g' < g of roundup(M_g', 128), g = 0..N (N = the shared
// expert with S rows), poff[N+1] = the total.  One workgroup: thread t holds
// the padded counts of groups PO_E t .. PO_E t + PO_E - 1 (zero past N), and a
// scan of the per-thread sums gives each thread its starting offset.
constexpr int PO_T = 256, PO_E = 5;
static_assert(PO_T * PO_E >= 1024 + 1, "covers the largest expert count and the shared expert");
__global__ void __launch_bounds__(PO_T) pad_offsets_kernel(const int32_t* __restrict__ offsets,
                                                           int N, int64_t S,
                                                           int32_t* __restrict__ poff) {
    __shared__ int64_t part[PO_T];
    const int t = threadIdx.x;
    int64_t v[PO_E];
    int64_t sum = 0;
#pragma unroll
    for (int e = 0; e < PO_E; ++e) {
        const int g = t * PO_E + e;
        const int64_t M = g < N ? offsets[g + 1] - offsets[g] : (g == N ? S : 0);
        v[e] = (M + 127) & ~int64_t(127);
        sum += v[e];
    }
    part[t] = sum;
    __syncthreads();
    for (int o = 1; o < PO_T; o <<= 1) {  // inclusive scan of the per-thread sums
        const int64_t add = t >= o ? part[t - o] : 0;
        __syncthreads();
        part[t] += add;
        __syncthreads();
    }
    int64_t acc = t > 0 ? part[t - 1] : 0;
#pragma unroll
    for (int e = 0; e < PO_E; ++e) {
        const int g = t * PO_E + e;
        if (g <= N) poff[g] = (int32_t)acc;
        acc += v[e];
    }
    if (t == PO_T - 1) poff[N + 1] = (int32_t)part[PO_T - 1];
}

struct ColQuant {
    const uint16_t* src_r;     // routed rows [T*k][ld_r] (bf16), or x [T][ld_r] with gather
    const uint16_t* src_s;     // shared rows [S][ld_s]
    const int32_t* gather;     // routed row -> source row (nullptr: identity)
    const int32_t* offsets;
    const int32_t* poff;
    int N;
    int64_t S;                 // shared rows (0: none)
    int64_t C_r, C_s;          // features (columns) of routed / shared rows
    int64_t ld_r, ld_s;
    uint8_t* out;              // [block][F][128] codes
    float* out_s;              // [block][F] scales
    int64_t F;                 // features per block in out (>= C_r, C_s)
};

// One 128-row block of one group x QC_CHUNKS * 64 features, 64 at a time: the
// column amax over the block's real rows, the codes of every real row
// (padding rows get code 0), written transposed (64 output rows of 128 codes
// per chunk).  The block's group and source rows are looked up once (a chain
// of dependent loads: the group search, the group's first row, the gather
// list) and serve every chunk; the next chunk's rows are loaded while this
// one is quantised.  The grid is one-dimensional with the feature chunk
// varying fastest, so consecutive workgroups read neighbouring pieces of the
// same rows.
constexpr int QC_CHUNKS = 4;

__global__ void __launch_bounds__(256) quant_cols_t_kernel(ColQuant p) {
    __shared__ float tile[128][65];
    __shared__ float red[4][64];
    const int64_t cm = p.C_r > p.C_s ? p.C_r : p.C_s;
    const int64_t nfc = (cm + 64 * QC_CHUNKS - 1) / (64 * QC_CHUNKS);  // feature chunks
    const int64_t row0 = ((int64_t)blockIdx.x / nfc) * 128;  // position on the padded axis
    const int32_t total = p.poff[p.N + 1];
    if (row0 >= total) return;
    int lo = 0, hi = p.N;  // group g: poff[g] <= row0 < poff[g+1]
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (p.poff[mid] <= row0) lo = mid; else hi = mid - 1;
    }
    const int g = lo;
    const bool routed = g < p.N;
    const int64_t C = routed ? p.C_r : p.C_s;  // a multiple of 64
    const int64_t cbase = ((int64_t)blockIdx.x % nfc) * 64 * QC_CHUNKS;
    if (cbase >= C) return;
    const int nch = (int)((C - cbase) / 64 < QC_CHUNKS ? (C - cbase) / 64 : QC_CHUNKS);
    const int64_t r0 = row0 - p.poff[g];  // first row of the block within the group
    const int64_t M = routed ? p.offsets[g + 1] - p.offsets[g] : p.S;
    const int valid = (int)(M - r0 < 128 ? M - r0 : 128);  // >= 1: the block holds rows
    const int t = threadIdx.x;
    // the 4 passes' rows (rows past the group's last read its last row and
    // are stored as zeros)
    int64_t sr[4];
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
        const int row = pass * 32 + (t >> 3);
        const int64_t rc = r0 + (row < valid ? row : valid - 1);
        if (routed) {
            const int64_t rr = p.offsets[g] + rc;
            sr[pass] = p.gather ? (int64_t)p.gather[rr] : rr;
        } else {
            sr[pass] = rc;
        }
    }
    const uint16_t* base = routed ? p.src_r : p.src_s;
    const int64_t ld = routed ? p.ld_r : p.ld_s;
    const int cc = (t & 7) * 8;
    const int col = t & 63, part = t >> 6;
    auto load = [&](int64_t c0, uint4 (&v)[4]) {
#pragma unroll
        for (int pass = 0; pass < 4; ++pass) v[pass] = *(const uint4*)(base + sr[pass] * ld + c0 + cc);
    };
    uint4 v[4];
    load(cbase, v);
    for (int ch = 0; ch < nch; ++ch) {
        const int64_t c0 = cbase + (int64_t)ch * 64;
        if (ch > 0) __syncthreads();  // the previous chunk's tile and red are read
#pragma unroll
        for (int pass = 0; pass < 4; ++pass) {
            const int row = pass * 32 + (t >> 3);
            const uint32_t w[4] = {v[pass].x, v[pass].y, v[pass].z, v[pass].w};
            float f[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f[2 * i] = row < valid ? __uint_as_float(w[i] << 16) : 0.0f;
                f[2 * i + 1] = row < valid ? __uint_as_float(w[i] & 0xffff0000u) : 0.0f;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) tile[row][cc + i] = f[i];
        }
        if (ch + 1 < nch) load(c0 + 64, v);  // in flight while this chunk is quantised
        __syncthreads();
        float m = 0.0f;
        for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(tile[part * 32 + i][col]));
        red[part][col] = m;
        __syncthreads();
        const float amax = fmaxf(fmaxf(red[0][col], red[1][col]), fmaxf(red[2][col], red[3][col]));
        const float scale = amax / 448.0f;
        // rows past the group's last hold zeros and encode as code 0
        uint32_t code[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            uint32_t wv = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                wv |= quant_e4m3(tile[part * 32 + 4 * k + e][col], scale) << (8 * e);
            code[k] = wv;
        }
        uint8_t* o = p.out + ((row0 / 128) * p.F + c0 + col) * 128 + part * 32;
        *(uint4*)o = make_uint4(code[0], code[1], code[2], code[3]);
        *(uint4*)(o + 16) = make_uint4(code[4], code[5], code[6], code[7]);
        if (part == 0) p.out_s[(row0 / 128) * p.F + c0 + col] = scale;
    }
}

// ---------------------------------------------------------------- weight gradients

struct WgFp8 {
    const uint8_t* At;  // [block][FA][128] codes (A^T: output rows along the contraction)
    const float* AtS;   // [block][FA]
    const uint8_t* Bt;  // [block][FB][128]
    const float* BtS;
    const int32_t* poff;
    int64_t FA, FB;     // features per block of At, Bt
    int N;
    int has_shared;
    int64_t rowsA_r, rowsB_r, rowsA_s, rowsB_s;
    uint16_t* out_r;    // [N][rowsA_r][rowsB_r] bf16
    uint16_t* out_s;    // [rowsA_s][rowsB_s]
};

// out[n][c] = sum over the group's 128-row blocks u of
//   (sA[n,u] sB[c,u]) * sum_{rows of u} qA[n,row] qB[c,row]
// One workgroup (8 waves) = one 128 x 128 output tile of one group.  The
// gradients are written once and never read here, so the kernel is bound by
// those writes: short workgroups that end right after their stores let the
// next ones start while the stores drain (vmcnt counts loads and stores in
// issue order, so a workgroup that waited for new copies after a store would
// wait for the store too), and two of them share a CU.  A block's operands
// (16 KB of A^T and 16 KB of B^T codes, their scales) are copied global ->
// LDS by buffer DMA into one of 2 stages, all blocks up front when the group
// has at most two (the swizzle goes through the source addresses).
//
// Wave (wa, wb) owns rows wa*32.. and columns wb*64.. of the tile as 2 x 4
// blocks of 16x16x128 MFMAs with the B^T rows as the first operand, so that a
// lane holds one output row n and 4 consecutive columns per block.  One such
// MFMA takes a whole 128-row block (its code products, scale operands 1.0),
// whose result is promoted into the fp32 sum right away with the product of
// the two fp32 scales; no partial sum is carried between instructions, so a
// wave needs under 128 registers and four waves share a SIMD.  The finished
// tile is staged through LDS so that every output row leaves as one
// contiguous 256-byte run: stores straight from the MFMA layout would write
// 32-byte pieces of 16 rows per instruction, which the non-temporal path
// writes to HBM as partial lines.
//
// Tile order: with N a multiple of 8, routed expert g's tiles go to XCD g % 8
// (block b runs on XCD b % 8) one expert after another, so the expert's
// operand tiles are shared in that XCD's L2; the shared expert's tiles come
// last.  Within a group the tiles go in bands of 8 column tiles, row tile by
// row tile, so that the ~64 workgroups an XCD holds at once read 8 A^T and 8
// B^T tiles between them.
constexpr int WT_THREADS = 512;
constexpr int WT_A = 128 * 128, WT_B = 128 * 128;
constexpr int WT_STAGE = WT_A + WT_B + 4 * 256;
constexpr int WT_BAND = 8;

__global__ void __launch_bounds__(WT_THREADS, 4) wgrad_fp8_kernel(WgFp8 p) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * WT_STAGE];
    const int64_t upg = (p.rowsA_r / 128) * (p.rowsB_r / 128);  // tiles per routed expert
    const int64_t b = blockIdx.x;
    int g;
    int64_t t, rowsA, rowsB;
    uint16_t* out;
    if (b < (int64_t)p.N * upg) {
        if (p.N % 8 == 0) {
            const int64_t s = b >> 3;
            g = (int)((s / upg) * 8 + (b & 7));
            t = s % upg;
        } else {
            g = (int)(b / upg);
            t = b % upg;
        }
        rowsA = p.rowsA_r;
        rowsB = p.rowsB_r;
        out = p.out_r + (int64_t)g * rowsA * rowsB;
    } else {
        g = p.N;
        t = b - (int64_t)p.N * upg;
        rowsA = p.rowsA_s;
        rowsB = p.rowsB_s;
        if (!p.has_shared || t >= (rowsA / 128) * (rowsB / 128)) return;
        out = p.out_s;
    }
    // bands of WT_BAND column tiles, row tile by row tile within a band
    const int64_t nta = rowsA / 128, ntb = rowsB / 128;
    const int64_t band = t / (nta * WT_BAND), bw = min((int64_t)WT_BAND, ntb - band * WT_BAND);
    const int64_t in_band = t - band * nta * WT_BAND;
    const int64_t ta = in_band / bw, tb = band * WT_BAND + in_band % bw;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wa = wave & 3, wb = wave >> 2;
    const int64_t P0 = p.poff[g];
    const int nb = (int)((p.poff[g + 1] - P0) / 128);
    const int64_t pb0 = P0 / 128;  // the group's first block
    uint16_t* tile = out + ta * 128 * rowsB + tb * 128;

    if (nb == 0) {  // an expert without rows: zero gradient
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int idx = tid + WT_THREADS * k, row = idx >> 4, c16 = idx & 15;
            *(uint4*)(tile + row * rowsB + c16 * 8) = make_uint4(0, 0, 0, 0);
        }
        return;
    }

    // buffer descriptors over the group's blocks
    const i32x4_t rA = make_rsrc(p.At + pb0 * p.FA * 128, (int64_t)nb * p.FA * 128);
    const i32x4_t rB = make_rsrc(p.Bt + pb0 * p.FB * 128, (int64_t)nb * p.FB * 128);
    const i32x4_t rAs = make_rsrc(p.AtS + pb0 * p.FA, (int64_t)nb * p.FA * 4);
    const i32x4_t rBs = make_rsrc(p.BtS + pb0 * p.FB, (int64_t)nb * p.FB * 4);
    const int cnt = 2 + 2 + (wave < 4 ? 1 : 0);  // copies per wave and stage
    // one block's copies: 1 KB copies of 8 rows of 128 bytes (lane l fills
    // row 8k + l/8, slot l%8, with the logical chunk that the swizzle puts
    // there); waves 0-1 also copy the A scales, waves 2-3 the B scales.  The
    // offsets are recomputed at every call (the empty asm hides that they do
    // not change): kept live through the loop they would push the MFMA loop's
    // registers past the 128 of four waves a SIMD.
    auto issue = [&](int u, int buf) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int crow = ln >> 3, cslot = ln & 7;
        uint8_t* st = smem + buf * WT_STAGE;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int k = wave + 8 * j, r = 8 * k + crow;
            const uint32_t voff = (uint32_t)((ta * 128 + r) * 128 + sub_chunk8(r, cslot) * 16);
            dma_to_lds<16>(rA, st + k * 1024, voff, (uint32_t)(u * p.FA * 128));
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int k = wave + 8 * j, r = 8 * k + crow;
            const uint32_t voff = (uint32_t)((tb * 128 + r) * 128 + sub_chunk8(r, cslot) * 16);
            dma_to_lds<16>(rB, st + WT_A + k * 1024, voff, (uint32_t)(u * p.FB * 128));
        }
        float* sc = (float*)(st + WT_A + WT_B);
        if (wave < 2)
            dma_to_lds<4>(rAs, sc + wave * 64, (uint32_t)((ta * 128 + wave * 64 + ln) * 4),
                          (uint32_t)(u * p.FA * 4));
        else if (wave < 4)
            dma_to_lds<4>(rBs, sc + 128 + (wave - 2) * 64,
                          (uint32_t)((tb * 128 + (wave - 2) * 64 + ln) * 4),
                          (uint32_t)(u * p.FB * 4));
    };
    // A / B fragment of a 16x16x128 MFMA: lane l holds row r = l%16 of the
    // operand block and its 32 codes 32 (l/16) .. +31 of the 128-row block
    auto frag = [&](const uint8_t* base, int r) {
        const int c = 2 * (lane >> 4);
        const uint4 lo = *(const uint4*)(base + r * 128 + sub_chunk8(r, c) * 16);
        const uint4 hi = *(const uint4*)(base + r * 128 + sub_chunk8(r, c + 1) * 16);
        return i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                       (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };

    f32x4_t acc[2][4];  // [A block i][B block j]; lane: row n, 4 columns c
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    issue(0, 0);
    if (nb > 1) issue(1, 1);
    for (int u = 0; u < nb; ++u) {
        vm_wait_n(u + 1 < nb ? cnt : 0);  // block u landed (u + 1 may be in flight)
        lds_barrier();
        const uint8_t* sA = smem + (u & 1) * WT_STAGE;
        const uint8_t* sB = sA + WT_A;
        const float* scA = (const float*)(sB + WT_B);
        const float* scB = scA + 128;
        i32x8_t af[2];
        float sa[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            af[i] = frag(sA, wa * 32 + i * 16 + (lane & 15));
            sa[i] = scA[wa * 32 + i * 16 + (lane & 15)];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const i32x8_t bf = frag(sB, wb * 64 + j * 16 + (lane & 15));
            const float4 sb = *(const float4*)(scB + wb * 64 + j * 16 + 4 * (lane >> 4));
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                // lane holds output row n = lane%16 of A block i and columns
                // 4 (lane/16) .. +3 of B block j
                const f32x4_t part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    bf, af[i], f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, 127, 0, 127);
                acc[i][j][0] += part[0] * (sa[i] * sb.x);
                acc[i][j][1] += part[1] * (sa[i] * sb.y);
                acc[i][j][2] += part[2] * (sa[i] * sb.z);
                acc[i][j][3] += part[3] * (sa[i] * sb.w);
            }
        }
        if (u + 2 < nb) {
            lds_barrier();  // every wave is done with this stage
            issue(u + 2, u & 1);
        }
    }
    // store: staged through the LDS stages as padded bf16 rows, then each
    // output row leaves as one contiguous 256-byte run; non-temporal: the
    // gradients are not read here
    constexpr int SP = 128 + 8;  // padded staging row (elements)
    static_assert(128 * SP * 2 <= 2 * WT_STAGE, "the staged tile fits in the stages");
    uint16_t* stg = (uint16_t*)smem;
    lds_barrier();  // every wave is done with the last stage
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = wa * 32 + i * 16 + (lane & 15);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = wb * 64 + j * 16 + 4 * (lane >> 4);
            *(uint2*)(stg + row * SP + col) = make_uint2(pack_bf16x2(acc[i][j][0], acc[i][j][1]),
                                                         pack_bf16x2(acc[i][j][2], acc[i][j][3]));
        }
    }
    lds_barrier();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int idx = tid + WT_THREADS * k, row = idx >> 4, c16 = idx & 15;
        __builtin_nontemporal_store(*(const u32x4_t*)(stg + row * SP + c16 * 8),
                                    (u32x4_t*)(tile + row * rowsB + c16 * 8));
    }
}

// ---------------------------------------------------------------- driver

struct BwdFp8Ws {
    int2* tiles;
    int32_t* counts;
    int32_t* order;
    int32_t* keys;
    int32_t* poff;
    void *ab_r, *h_r, *ab_s, *h_s;      // recompute (bf16)
    uint8_t *gq_r, *gq_s;               // dY row tiles
    float *gs_r, *gs_s;
    void *dh_r, *dh_s;                  // dh (bf16)
    void *dab_r, *dab_s;                // [da | db] (bf16)
    uint8_t *tq_r, *tq_s;               // [da | db] row tiles
    float *ts_r, *ts_s;
    uint8_t *gT, *hT, *tT, *xT;         // row-direction tiles, transposed
    float *gTs, *hTs, *tTs, *xTs;
    int64_t P_ld;
};

static int64_t bwd_fp8_max_r(const moe_cfg& c) { return c.tokens * c.top_k / FP8_BM + c.n_experts; }
static int64_t bwd_fp8_max_s(const moe_cfg& c) { return cdiv(c.tokens, FP8_BM); }

static BwdFp8Ws carve_bwd_fp8(const moe_cfg& c, void* ws, size_t* bytes) {
    const int64_t R = c.tokens * c.top_k, T = c.tokens, d = c.hidden, I = c.inter;
    const int64_t Is = c.inter_shared, S = Is > 0 ? T : 0, N = c.n_experts;
    const int64_t Im = I > Is ? I : Is;
    BwdFp8Ws w{};
    w.P_ld = r128(R + 128 * N + S + 128);
    char* base = (char*)ws;
    int64_t o = 0;
    auto take = [&](int64_t n) {
        char* q = base ? base + o : nullptr;
        o += a256(n);
        return q;
    };
    w.tiles = (int2*)take((bwd_fp8_max_r(c) + bwd_fp8_max_s(c)) * 8);
    w.counts = (int32_t*)take(8);
    w.order = (int32_t*)take(bwd_fp8_max_r(c) * 4);
    w.keys = (int32_t*)take(bwd_fp8_max_r(c) * 4);
    w.poff = (int32_t*)take((N + 2) * 4);
    w.ab_r = take(R * 2 * I * 2);
    w.h_r = take(R * I * 2);
    w.ab_s = take(S * 2 * Is * 2);
    w.h_s = take(S * Is * 2);
    w.gq_r = (uint8_t*)take(R * d);
    w.gs_r = (float*)take(R * (d / 128) * 4);
    w.gq_s = (uint8_t*)take(S * d);
    w.gs_s = (float*)take(S * (d / 128) * 4);
    w.dh_r = take(R * I * 2);
    w.dh_s = take(S * Is * 2);
    w.dab_r = take(R * 2 * I * 2);
    w.dab_s = take(S * 2 * Is * 2);
    w.tq_r = (uint8_t*)take(R * 2 * I);
    w.ts_r = (float*)take(R * (2 * I / 128) * 4);
    w.tq_s = (uint8_t*)take(S * 2 * Is);
    w.ts_s = (float*)take(S * (2 * Is / 128) * 4);
    const int64_t sl = w.P_ld / 128;
    w.gT = (uint8_t*)take(d * w.P_ld);
    w.gTs = (float*)take(d * sl * 4);
    w.hT = (uint8_t*)take(Im * w.P_ld);
    w.hTs = (float*)take(Im * sl * 4);
    w.tT = (uint8_t*)take(2 * Im * w.P_ld);
    w.tTs = (float*)take(2 * Im * sl * 4);
    w.xT = (uint8_t*)take(d * w.P_ld);
    w.xTs = (float*)take(d * sl * 4);
    if (bytes) *bytes = (size_t)o;
    return w;
}

void ffn_backward_fp8_offsets(const moe_cfg& c, size_t off[25]) {
    char* base = (char*)(uintptr_t)4096;  // any aligned base: only differences are used
    const BwdFp8Ws w = carve_bwd_fp8(c, base, nullptr);
    auto o = [&](const void* p) { return (size_t)((const char*)p - base); };
    const void* ptrs[25] = {w.gq_r, w.gs_r, w.gq_s, w.gs_s, w.dh_r, w.dh_s, w.dab_r, w.dab_s,
                            w.tq_r, w.ts_r, w.tq_s, w.ts_s, w.gT, w.gTs, w.hT, w.hTs, w.tT,
                            w.tTs, w.xT, w.xTs, w.poff, w.ab_r, w.h_r, w.ab_s, w.h_s};
    for (int i = 0; i < 25; ++i) off[i] = o(ptrs[i]);
}

size_t ffn_backward_fp8_workspace_bytes(const moe_cfg& c) {
    size_t b = 0;
    carve_bwd_fp8(c, nullptr, &b);
    return b;
}

static hipError_t quant_rows(const void* x, int64_t rows, int64_t C, uint8_t* q, float* s,
                             hipStream_t st) {
    const int64_t tiles = rows * (C / 128);
    if (tiles == 0) return hipSuccess;
    quant_rows_bf16_kernel<<<(unsigned)cdiv(tiles, 16), 256, 0, st>>>((const uint4*)x, rows, C,
                                                                       (uint2*)q, s);
    return hipGetLastError();
}

static hipError_t swiglu_bwd(const void* dh, const void* ab, int64_t rows, int64_t I, void* dab,
                             uint8_t* q, float* s, hipStream_t st) {
    const int64_t units = rows * (I / 128);
    if (units == 0) return hipSuccess;
    swiglu_bwd_fp8_kernel<<<(unsigned)cdiv(units, 16), 256, 0, st>>>(
        (const uint4*)dh, (const uint4*)ab, rows, I, (uint4*)dab, (uint2*)q, s);
    return hipGetLastError();
}

hipError_t launch_expert_ffn_backward_fp8(const moe_cfg& c, const FfnBwdFp8Args& a, void* ws,
                                          hipStream_t st, const void* saved) {
    const int64_t T = c.tokens, R = T * c.top_k, d = c.hidden, I = c.inter;
    const int64_t Is = c.inter_shared, N = c.n_experts;
    const bool has_shared = Is > 0 && T > 0;
    const int64_t S = has_shared ? T : 0;
    const int64_t Im = I > Is ? I : Is;
    BwdFp8Ws w = carve_bwd_fp8(c, ws, nullptr);
    if (saved) {  // a, b, h kept by the training forward (moe_expert_ffn_train_fp8)
        const SavedActs sv = carve_saved(c, const_cast<void*>(saved));
        w.ab_r = sv.ab_r;
        w.h_r = sv.h_r;
        w.ab_s = sv.ab_s;
        w.h_s = sv.h_s;
    }
    const int64_t max_r = bwd_fp8_max_r(c), max_s = has_shared ? bwd_fp8_max_s(c) : 0;
    hipError_t e;
    if (R > 0) {
        launch_tile_map(a.offsets, (int)N, T, has_shared, FP8_BM, w.tiles, w.counts, w.order,
                        w.keys, st);
        // 1. a, b, h of every row (FP8 gate/up, as in the forward), unless kept
        Fp8Gemm g{};
        g.mode = 2;
        g.K_r = g.K_s = d;
        g.Nout_r = I;
        g.Nout_s = Is;
        g.A_r = a.x_perm_q;
        g.A_s = a.x_q;
        g.as_r = a.x_perm_s;
        g.as_s = a.x_s;
        g.B_r = a.w13;
        g.B_s = a.ws13;
        g.bs_r = a.w13_s;
        g.bs_s = a.ws13_s;
        g.C_r = w.h_r;
        g.C_s = w.h_s;
        g.E_r = w.ab_r;
        g.E_s = w.ab_s;
        if (!saved && (e = launch_fp8_gemm(g, w.tiles, w.counts, w.order, a.offsets, (int)N, S,
                                           max_r, max_s, st)) != hipSuccess)
            return e;
        // 2. dY row tiles, dh = dY W2
        if ((e = quant_rows(a.dy_perm, R, d, w.gq_r, w.gs_r, st)) != hipSuccess) return e;
        if (has_shared && (e = quant_rows(a.dy_sh, S, d, w.gq_s, w.gs_s, st)) != hipSuccess)
            return e;
        g = Fp8Gemm{};
        g.mode = 1;
        g.K_r = g.K_s = d;
        g.Nout_r = I;
        g.Nout_s = Is;
        g.A_r = w.gq_r;
        g.A_s = w.gq_s;
        g.as_r = w.gs_r;
        g.as_s = w.gs_s;
        g.B_r = a.w2t;
        g.B_s = a.ws2t;
        g.bs_r = a.w2_s;
        g.bs_s = a.ws2_s;
        g.bs_t = 1;
        g.C_r = w.dh_r;
        g.C_s = w.dh_s;
        if ((e = launch_fp8_gemm(g, w.tiles, w.counts, w.order, a.offsets, (int)N, S, max_r,
                                 max_s, st)) != hipSuccess)
            return e;
        // 3. da, db and their row tiles
        if ((e = swiglu_bwd(w.dh_r, w.ab_r, R, I, w.dab_r, w.tq_r, w.ts_r, st)) != hipSuccess)
            return e;
        if (has_shared &&
            (e = swiglu_bwd(w.dh_s, w.ab_s, S, Is, w.dab_s, w.tq_s, w.ts_s, st)) != hipSuccess)
            return e;
        // 4. dX = [da db] [W1; W3]
        g = Fp8Gemm{};
        g.mode = 1;
        g.K_r = 2 * I;
        g.K_s = 2 * Is;
        g.Nout_r = g.Nout_s = d;
        g.A_r = w.tq_r;
        g.A_s = w.tq_s;
        g.as_r = w.ts_r;
        g.as_s = w.ts_s;
        g.B_r = a.w13t;
        g.B_s = a.ws13t;
        g.bs_r = a.w13_s;
        g.bs_s = a.ws13_s;
        g.bs_t = 1;
        g.C_r = a.dx_perm;
        g.C_s = a.dx_sh;
        if ((e = launch_fp8_gemm(g, w.tiles, w.counts, w.order, a.offsets, (int)N, S, max_r,
                                 max_s, st)) != hipSuccess)
            return e;
    }
    // 5. row-direction tiles of dY, h, [da db] and X (empty groups: nothing)
    pad_offsets_kernel<<<1, PO_T, 0, st>>>(a.offsets, (int)N, S, w.poff);
    const unsigned pblocks = (unsigned)(w.P_ld / 128);
    auto cols = [&](const void* sr, const void* ss, const int32_t* gather, int64_t Cr,
                    int64_t Cs, int64_t ldr, int64_t lds, int64_t F, uint8_t* out,
                    float* outs) {
        ColQuant p{};
        p.src_r = (const uint16_t*)sr;
        p.src_s = (const uint16_t*)ss;
        p.gather = gather;
        p.offsets = a.offsets;
        p.poff = w.poff;
        p.N = (int)N;
        p.S = S;
        p.C_r = Cr;
        p.C_s = Cs;
        p.ld_r = ldr;
        p.ld_s = lds;
        p.out = out;
        p.out_s = outs;
        p.F = F;
        const int64_t cm = Cr > Cs ? Cr : Cs;
        const int64_t nblk = cdiv(cm, 64 * QC_CHUNKS) * (int64_t)pblocks;
        if (nblk > 0) quant_cols_t_kernel<<<dim3((unsigned)nblk), 256, 0, st>>>(p);
    };
    if (R + S > 0) {
        cols(a.dy_perm, a.dy_sh, nullptr, d, d, d, d, d, w.gT, w.gTs);
        cols(w.h_r, w.h_s, nullptr, I, Is, I, Is, Im, w.hT, w.hTs);
        cols(w.dab_r, w.dab_s, nullptr, 2 * I, 2 * Is, 2 * I, 2 * Is, 2 * Im, w.tT, w.tTs);
        cols(a.x, a.x, a.src_token, d, d, d, d, d, w.xT, w.xTs);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // 6. dW2 = dY^T h and dW13 = [da db]^T X for every expert (zeros without rows)
    auto wgrad = [&](const uint8_t* At, const float* AtS, int64_t FA, const uint8_t* Bt,
                     const float* BtS, int64_t FB, int64_t rAr, int64_t rBr, int64_t rAs,
                     int64_t rBs, void* outr, void* outs) {
        WgFp8 p{};
        p.At = At;
        p.AtS = AtS;
        p.Bt = Bt;
        p.BtS = BtS;
        p.poff = w.poff;
        p.FA = FA;
        p.FB = FB;
        p.N = (int)N;
        p.has_shared = has_shared ? 1 : 0;
        p.rowsA_r = rAr;
        p.rowsB_r = rBr;
        p.rowsA_s = rAs;
        p.rowsB_s = rBs;
        p.out_r = (uint16_t*)outr;
        p.out_s = (uint16_t*)outs;
        const int64_t units = N * (rAr / 128) * (rBr / 128) +
                              (has_shared ? (rAs / 128) * (rBs / 128) : 0);
        if (units > 0) wgrad_fp8_kernel<<<(unsigned)units, WT_THREADS, 0, st>>>(p);
    };
    wgrad(w.gT, w.gTs, d, w.hT, w.hTs, Im, d, I, d, Is, a.dw2, a.dws2);
    wgrad(w.tT, w.tTs, 2 * Im, w.xT, w.xTs, d, 2 * I, d, 2 * Is, d, a.dw13, a.dws13);
    return hipGetLastError();
}

}  // namespace moe
