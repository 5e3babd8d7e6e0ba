// gemm_bwd.hip -- backward of the grouped SwiGLU expert FFN (routed experts and
// the shared expert), bf16 and fp32 storage.
//
// Forward (DeepSeek-V3 report reading guide, xyznot.com/de, "Methode" item 2,
// FFN read as SwiGLU without biases): for the rows X of one expert,
//   a = X W1^T, b = X W3^T, h = silu(a) * b, y = h W2^T.
// Given dY = dL/dy, the chain rule gives five grouped GEMMs:
//   recompute  a, b (stored), h (stored)       X [M,d]    x W13 [2I,d]^T
//   dgrad down dh = dY W2, then in the epilogue da = dh b silu'(a), db = dh silu(a)
//                                              dY [M,d]   x W2 [d,I]
//   dgrad up   dX = [da db] W13                [M,2I]     x W13 [2I,d]
//   wgrad down dW2 = dY^T h                    contraction over the M rows
//   wgrad up   dW13 = [da db]^T X              contraction over the M rows
// silu'(a) = sig(a) (1 + a (1 - sig(a))).
//
// bf16: the first three run on the forward's streaming kernel (gemm.hip, modes
// 2, 3 and 1) with the weights packed for it -- W13 as in the forward, W13 and
// W2 transposed for the dgrads.  The weight gradients contract over token rows,
// so both operands are stored against the MFMA's operand order; they run
// here: one 256 x 256 tile of dW per workgroup, 8 wavefronts of 64 x 128 on
// v_mfma_f32_16x16x32_bf16 (a tile contracts over only ~T*k/N rows, so a big
// tile gets the most MFMA work out of each round trip to memory).  The rows
// are copied global -> LDS as they are stored (4 stages of 32 rows, copies
// 3 stages ahead, no staging registers), and gfx950's transposing LDS load
// turns them into MFMA operands.
// fp32: plain VALU kernels for all five (small layers).
#include "gemm_common.h"

namespace moe {

enum BwdOp { OP_RECOMP = 0, OP_DGRAD_DOWN = 1, OP_DGRAD_UP = 2, OP_WGRAD_DOWN = 3, OP_WGRAD_UP = 4 };

struct BwdParams {
    const int32_t* offsets;
    int N;
    int has_shared;
    // weight gradients: tiles per group and column tiles per row of tiles,
    // routed experts and the shared expert
    int64_t ntn_r, ntc_r, ntn_s, ntc_s;
    int64_t T, TK, d, I_r, I_s;
    const void* x_perm;
    const void* x;
    const void* dy_perm;
    const void* dy_s;
    const void* w13;
    const void* w2;
    const void* ws13;
    const void* ws2;
    void* ab_r;
    void* ab_s;
    void* h_r;
    void* h_s;
    void* dab_r;
    void* dab_s;
    void* dx_perm;
    void* dx_s;
    void* dw13;
    void* dw2;
    void* dws13;
    void* dws2;
};

// One group's view: routed expert g < N over its rows of the permuted arrays,
// or the shared expert (g == N) over all T tokens.
template <typename E>
struct Grp {
    int64_t M, I;
    const E* X;
    const E* dY;
    const E* W13;
    const E* W2;
    E* ab;    // [M][2I]: a in columns 0..I-1, b in I..2I-1
    E* h;     // [M][I]
    E* dab;   // [M][2I]: da, db
    E* dX;    // [M][d]
    E* dW13;  // [2I][d]
    E* dW2;   // [d][I]
};

template <typename E>
__device__ __forceinline__ void group_view(const BwdParams& p, int g, Grp<E>& v) {
    const int64_t d = p.d;
    if (g < p.N) {
        const int64_t rb = p.offsets[g];
        const int64_t I = p.I_r;
        v.M = p.offsets[g + 1] - rb;
        v.I = I;
        v.X = (const E*)p.x_perm + rb * d;
        v.dY = (const E*)p.dy_perm + rb * d;
        v.W13 = (const E*)p.w13 + (int64_t)g * 2 * I * d;
        v.W2 = (const E*)p.w2 + (int64_t)g * d * I;
        v.ab = (E*)p.ab_r + rb * 2 * I;
        v.h = (E*)p.h_r + rb * I;
        v.dab = (E*)p.dab_r + rb * 2 * I;
        v.dX = (E*)p.dx_perm + rb * d;
        v.dW13 = (E*)p.dw13 + (int64_t)g * 2 * I * d;
        v.dW2 = (E*)p.dw2 + (int64_t)g * d * I;
    } else {
        v.M = p.T;
        v.I = p.I_s;
        v.X = (const E*)p.x;
        v.dY = (const E*)p.dy_s;
        v.W13 = (const E*)p.ws13;
        v.W2 = (const E*)p.ws2;
        v.ab = (E*)p.ab_s;
        v.h = (E*)p.h_s;
        v.dab = (E*)p.dab_s;
        v.dX = (E*)p.dx_s;
        v.dW13 = (E*)p.dws13;
        v.dW2 = (E*)p.dws2;
    }
}

// extents of C (rows, columns) and of the contraction for one group
template <int OP>
__device__ __forceinline__ void op_extents(int64_t M, int64_t I, int64_t d, int64_t& R,
                                           int64_t& C, int64_t& K) {
    if (OP == OP_RECOMP) { R = M; C = I; K = d; }             // C columns = h columns
    else if (OP == OP_DGRAD_DOWN) { R = M; C = I; K = d; }
    else if (OP == OP_DGRAD_UP) { R = M; C = d; K = 2 * I; }
    else if (OP == OP_WGRAD_DOWN) { R = d; C = I; K = M; }
    else { R = 2 * I; C = d; K = M; }
}

// Weight-gradient unit -> (group, first dW row, first dW column); false = no
// work.  The shared expert's tiles come first, dealt round-robin over the
// XCDs (block L runs on XCD L % 8): each contracts over all T tokens, so they
// are the longest units and are spread evenly.  Then XCD x takes the routed
// experts x, x+8, x+16, ... one after the other, so the ~M rows of the expert
// its CUs are working on stay in that XCD's L2.
__device__ __forceinline__ bool wgrad_unit(const BwdParams& p, int64_t L, int& g, int64_t& r0,
                                           int64_t& c0, int CT) {
    const int64_t S = p.has_shared ? p.ntn_s : 0;
    int64_t rem, ntc;
    if (L < S) {
        g = p.N;
        rem = L;
        ntc = p.ntc_s;
    } else {
        const int64_t Lp = L - S, x = Lp % 8, i = Lp / 8;
        const int64_t gi = (i / p.ntn_r) * 8 + x;
        if (gi >= p.N) return false;
        g = (int)gi;
        rem = i % p.ntn_r;
        ntc = p.ntc_r;
    }
    r0 = (rem / ntc) * CT;
    c0 = (rem % ntc) * CT;
    return true;
}

// ---------------------------------------------------------------- bf16 MFMA

constexpr int BT = 256;       // dW tile rows and columns
constexpr int BBK = 32;       // contraction rows (token rows) per LDS stage
constexpr int NSTG = 4;       // LDS stages: loads run 3 stages ahead
constexpr int BW_WAVES = 8;   // 4 x 2 wavefronts of 64 x 128
constexpr int BW_THREADS = 64 * BW_WAVES;
constexpr int WG_DMA = 4;     // global -> LDS copies per wavefront per stage

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// LDS holds each operand stage in its memory order, [32 contraction rows][256
// columns], 512-byte rows of 16 segments of 32 bytes; segment s of row k is
// stored at slot s ^ wg_seg(k).  The MFMA operands are read with the
// transposing LDS load (ds_read_b64_tr_b16): a group of 16 lanes names 16
// pieces of 8 bytes, pieces 4e..4e+3 form row e of a 4 x 16 block, and lane i
// receives element i of each of the 4 rows -- here one column and 4
// consecutive contraction rows.  One such read touches rows 8g + e (+4) for
// g, e < 4 in a single segment; wg_seg gives those 16 rows 8 distinct bank
// groups (2 passes for 512 bytes, the minimum).
__device__ __forceinline__ int wg_seg(int k) { return (k & 3) | (((k >> 3) & 1) << 2); }

template <int OP>
__global__ void __launch_bounds__(BW_THREADS, 1) wgrad_bf16_kernel(BwdParams p) {
    static_assert(OP == OP_WGRAD_DOWN || OP == OP_WGRAD_UP, "weight gradients only");
    int g;
    int64_t r0, c0;
    if (!wgrad_unit(p, blockIdx.x, g, r0, c0, BT)) return;
    Grp<uint16_t> v;
    group_view(p, g, v);
    const int64_t d = p.d, I = v.I;
    int64_t R, C, K;
    op_extents<OP>(v.M, I, d, R, C, K);
    if (r0 >= R || c0 >= C) return;

    // C[r][c] = sum_m A[m][r0 + r] B[m][c0 + c]
    const uint16_t* a_base;
    const uint16_t* b_base;
    int64_t a_ld, b_ld;
    uint16_t* Cp;
    int64_t ldc;
    if (OP == OP_WGRAD_DOWN) {  // dW2 [d][I] = dY^T h
        a_base = v.dY + r0; a_ld = d;
        b_base = v.h + c0; b_ld = I;
        Cp = v.dW2; ldc = I;
    } else {                    // dW13 [2I][d] = [da db]^T X
        a_base = v.dab + r0; a_ld = 2 * I;
        b_base = v.X + c0; b_ld = d;
        Cp = v.dW13; ldc = d;
    }

    __shared__ __attribute__((aligned(1024))) uint16_t smem[NSTG][2][BBK * BT];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 3, wn = wave >> 2;
    const int nk = (int)((K + BBK - 1) / BBK);

    // Copies: buffer descriptors over the operand rows 0..K-1 of the tile's
    // columns (range-checked: rows past K, and columns past the operand in its
    // last row, read as zeros).  Copy q (0..15) of a stage covers rows 2q,
    // 2q+1; wavefront w issues q = w and w + 8 for A and for B.  Lane l
    // fills LDS bytes 16l..16l+15 of the two rows: row 2q + l/32, slot
    // (l%32)/2, half l%2, which holds logical segment slot ^ wg_seg(row).
    const int64_t acols = R - r0 < BT ? R - r0 : BT, bcols = C - c0 < BT ? C - c0 : BT;
    const i32x4_t ra = make_rsrc(a_base, K > 0 ? ((K - 1) * a_ld + acols) * 2 : 0);
    const i32x4_t rb = make_rsrc(b_base, K > 0 ? ((K - 1) * b_ld + bcols) * 2 : 0);
    auto issue = [&](int kt, int s) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int q = wave + 8 * h;
            const int row = 2 * q + (lane >> 5);
            const int col = (((lane & 31) >> 1) ^ wg_seg(row)) * 16 + (lane & 1) * 8;
            const int64_t grow = (int64_t)kt * BBK + row;
            dma_to_lds<16>(ra, smem[s][0] + 2 * q * BT, (uint32_t)((grow * a_ld + col) * 2), 0);
            dma_to_lds<16>(rb, smem[s][1] + 2 * q * BT, (uint32_t)((grow * b_ld + col) * 2), 0);
        }
    };

    // MFMA: D rows = B columns (output columns), D columns = A columns (output
    // rows); wave (wm, wn) owns output rows wm*64 + 16i + 0..15 (i < 4) and
    // columns wn*128 + 16j + 0..15 (j < 8); lane holds
    // C[16-row block + l16][16-column block + 4 gq + 0..3]
    const int l16 = lane & 15, gq = lane >> 4;
    f32x4_t acc[8][4];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // fragment of columns cb..cb+15: lane (gq, l16) names piece l16 of rows
    // 8gq + l16/4 (+4): columns cb + 4 (l16 % 4) .. +3
    const int fk = 8 * gq + (l16 >> 2), fc = 4 * (l16 & 3);
    auto frag = [&](const uint16_t* buf, int cb) {
        const int s0 = ((cb >> 4) ^ wg_seg(fk)) * 16 + fc;
        const int s1 = ((cb >> 4) ^ wg_seg(fk + 4)) * 16 + fc;
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(to_lds(buf + fk * BT + s0)));
        const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(to_lds(buf + (fk + 4) * BT + s1)));
        return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    auto compute = [&](int st) {
        bf16x8_t af[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) af[i] = frag(smem[st][0], wm * 64 + i * 16);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bf16x8_t bf = frag(smem[st][1], wn * 128 + j * 16);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf, af[i], acc[j][i], 0, 0, 0);
        }
    };

    // Pipeline: stage kt waits for its copies (each wavefront's later stages
    // may stay in flight), a barrier makes it visible to all and frees stage
    // kt-1, whose buffer then takes stage kt+NSTG-1.  lds_barrier, not
    // __syncthreads: the copies in flight must not be waited for.
#pragma unroll
    for (int s = 0; s < NSTG - 1; ++s)
        if (s < nk) issue(s, s);
    for (int kt = 0; kt < nk; ++kt) {
        const int after = nk - 1 - kt < NSTG - 2 ? nk - 1 - kt : NSTG - 2;
        vm_wait_n(after * WG_DMA);
        lds_barrier();
        if (kt + NSTG - 1 < nk) issue(kt + NSTG - 1, (kt + NSTG - 1) % NSTG);
        compute(kt % NSTG);
    }
    lds_barrier();  // every wave is done with the stage buffers

    // Epilogue through LDS: the 256 x 256 bf16 tile, 16-byte chunk c of row r
    // at slot c ^ (r & 15), then whole 512-byte rows to global memory, 16
    // bytes per thread, as non-temporal stores (dW is written once and not
    // read back here; keeping it out of L2 leaves room for the operands;
    // measured faster).  A group without rows (K = 0) writes zeros.
    uint16_t* ot = &smem[0][0][0];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = wm * 64 + i * 16 + l16;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int col = wn * 128 + j * 16 + 4 * gq;
            *(uint2*)(ot + row * BT + (((col >> 3) ^ (row & 15)) << 3) + (col & 7)) =
                make_uint2(pack_bf16x2(acc[j][i][0], acc[j][i][1]),
                           pack_bf16x2(acc[j][i][2], acc[j][i][3]));
        }
    }
    __syncthreads();
    const int64_t rows = R - r0 < BT ? R - r0 : BT;
    const int64_t chunks = (C - c0 < BT ? C - c0 : BT) / 8;
    for (int q = tid; q < BT * (BT / 8); q += BW_THREADS) {
        const int row = q >> 5, c = q & 31;
        if (row < rows && c < chunks) {
            const uint4 q4 = *(const uint4*)(ot + row * BT + ((c ^ (row & 15)) << 3));
            __builtin_nontemporal_store(u32x4_t{q4.x, q4.y, q4.z, q4.w},
                                        (u32x4_t*)(Cp + (r0 + row) * ldc + c0 + c * 8));
        }
    }
}

// ---------------------------------------------------------------- fp32 path
// Plain VALU kernels for fp32 storage (small layers): one thread per output
// element, contraction in ascending order with fp32 FMAs.  Row-tiled GEMMs
// enumerate the TK routed rows then the T shared rows; weight gradients
// enumerate each group's R x C outputs.
template <int OP>
__global__ void __launch_bounds__(256) bwd_f32_kernel(BwdParams p, int64_t cols,
                                                      int64_t per_r, int64_t total) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= total) return;
    int g;
    int64_t m, n;
    if (OP <= OP_DGRAD_UP) {
        const int64_t row = e / cols;
        n = e % cols;
        if (row < p.TK) {
            int lo = 0, hi = p.N;  // largest g with offsets[g] <= row
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (p.offsets[mid] <= row) lo = mid; else hi = mid;
            }
            g = lo;
            m = row - p.offsets[g];
        } else {
            g = p.N;
            m = row - p.TK;
        }
    } else {
        if (e < (int64_t)p.N * per_r) {
            g = (int)(e / per_r);
            m = (e % per_r) / cols;
            n = (e % per_r) % cols;
        } else {
            g = p.N;
            const int64_t r = e - (int64_t)p.N * per_r;
            const int64_t cs = OP == OP_WGRAD_DOWN ? p.I_s : p.d;
            m = r / cs;
            n = r % cs;
        }
    }
    Grp<float> v;
    group_view(p, g, v);
    const int64_t d = p.d, I = v.I;
    int64_t R, C, K;
    op_extents<OP>(v.M, I, d, R, C, K);
    if (m >= R || n >= C) return;
    if (OP == OP_RECOMP) {
        float sa = 0.0f, sb = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            const float xv = v.X[m * d + k];
            sa = __builtin_fmaf(xv, v.W13[n * d + k], sa);
            sb = __builtin_fmaf(xv, v.W13[(I + n) * d + k], sb);
        }
        v.ab[m * 2 * I + n] = sa;
        v.ab[m * 2 * I + I + n] = sb;
        v.h[m * I + n] = sa / (1.0f + expf(-sa)) * sb;
    } else if (OP == OP_DGRAD_DOWN) {
        float dh = 0.0f;
        for (int64_t k = 0; k < K; ++k) dh = __builtin_fmaf(v.dY[m * d + k], v.W2[k * I + n], dh);
        const float a = v.ab[m * 2 * I + n], b = v.ab[m * 2 * I + I + n];
        const float sg = 1.0f / (1.0f + expf(-a));
        v.dab[m * 2 * I + n] = dh * b * sg * (1.0f + a * (1.0f - sg));
        v.dab[m * 2 * I + I + n] = dh * a * sg;
    } else if (OP == OP_DGRAD_UP) {
        float s = 0.0f;
        for (int64_t k = 0; k < K; ++k) s = __builtin_fmaf(v.dab[m * 2 * I + k], v.W13[k * d + n], s);
        v.dX[m * d + n] = s;
    } else if (OP == OP_WGRAD_DOWN) {
        float s = 0.0f;
        for (int64_t k = 0; k < K; ++k) s = __builtin_fmaf(v.dY[k * d + m], v.h[k * I + n], s);
        v.dW2[m * I + n] = s;
    } else {
        float s = 0.0f;
        for (int64_t k = 0; k < K; ++k) s = __builtin_fmaf(v.dab[k * 2 * I + m], v.X[k * d + n], s);
        v.dW13[m * d + n] = s;
    }
}

// ---------------------------------------------------------------- launch

struct BwdWs {
    void* tile_ws;
    void *ab_r, *ab_s, *h_r, *h_s, *dab_r, *dab_s;
};

static int64_t align256(int64_t b) { return (b + 255) & ~int64_t(255); }
static int64_t bwd_esz(const moe_cfg& c) { return c.act_dtype == MOE_BF16 ? 2 : 4; }
static int64_t imax(int64_t a, int64_t b) { return a > b ? a : b; }

size_t ffn_saved_bytes(const moe_cfg& c) {
    const int64_t TK = c.tokens * c.top_k, T = c.tokens, eb = bwd_esz(c);
    const int64_t I = c.inter, Is = c.inter_shared;
    return (size_t)(align256(TK * 2 * I * eb) + align256(TK * I * eb) +
                    align256(T * 2 * Is * eb) + align256(T * Is * eb));
}

SavedActs carve_saved(const moe_cfg& c, void* saved) {
    const int64_t TK = c.tokens * c.top_k, T = c.tokens, eb = bwd_esz(c);
    const int64_t I = c.inter, Is = c.inter_shared;
    char* q = (char*)saved;
    SavedActs s{};
    s.ab_r = q; q += align256(TK * 2 * I * eb);
    s.h_r = q; q += align256(TK * I * eb);
    s.ab_s = q; q += align256(T * 2 * Is * eb);
    s.h_s = q;
    return s;
}

size_t ffn_backward_workspace_bytes(const moe_cfg& c) {
    const int64_t TK = c.tokens * c.top_k, T = c.tokens, eb = bwd_esz(c);
    const int64_t I = c.inter, Is = c.inter_shared;
    int64_t b = align256((int64_t)ffn_bwd_tile_ws_bytes(c));
    b += 2 * align256(TK * 2 * I * eb) + align256(TK * I * eb);  // ab, dab, h routed
    b += 2 * align256(T * 2 * Is * eb) + align256(T * Is * eb);  // shared
    return (size_t)b;
}

static BwdWs carve_bwd(const moe_cfg& c, void* ws) {
    const int64_t TK = c.tokens * c.top_k, T = c.tokens, eb = bwd_esz(c);
    const int64_t I = c.inter, Is = c.inter_shared;
    char* q = (char*)ws;
    BwdWs w{};
    w.tile_ws = q;
    q += align256((int64_t)ffn_bwd_tile_ws_bytes(c));
    w.ab_r = q; q += align256(TK * 2 * I * eb);
    w.dab_r = q; q += align256(TK * 2 * I * eb);
    w.h_r = q; q += align256(TK * I * eb);
    w.ab_s = q; q += align256(T * 2 * Is * eb);
    w.dab_s = q; q += align256(T * 2 * Is * eb);
    w.h_s = q;
    return w;
}

template <int OP>
static void launch_wgrad_bf16(const BwdParams& p, int64_t units, hipStream_t st) {
    if (units > 0) wgrad_bf16_kernel<OP><<<dim3((unsigned)units), BW_THREADS, 0, st>>>(p);
}

template <int OP>
static void launch_bwd_f32(const BwdParams& p, int64_t cols, int64_t per_r, int64_t total,
                           hipStream_t st) {
    if (total > 0)
        bwd_f32_kernel<OP><<<dim3((unsigned)cdiv(total, 256)), 256, 0, st>>>(p, cols, per_r, total);
}

static BwdParams bwd_params(const moe_cfg& c) {
    const int64_t T = c.tokens;
    const bool has_shared = c.inter_shared > 0 && T > 0;
    BwdParams p{};
    p.N = (int)c.n_experts;
    p.has_shared = has_shared ? 1 : 0;
    p.T = has_shared ? T : 0;
    p.TK = T * c.top_k;
    p.d = c.hidden;
    p.I_r = c.inter;
    p.I_s = has_shared ? c.inter_shared : 0;
    return p;
}

hipError_t launch_ffn_save_f32(const moe_cfg& c, const void* x_perm, const void* x_sh,
                               const int32_t* offsets, const void* w13, const void* ws13,
                               void* saved, hipStream_t st) {
    BwdParams p = bwd_params(c);
    const SavedActs sv = carve_saved(c, saved);
    p.offsets = offsets;
    p.x_perm = x_perm;
    p.x = x_sh;
    p.w13 = w13;
    p.ws13 = ws13;
    p.ab_r = sv.ab_r;
    p.ab_s = sv.ab_s;
    p.h_r = sv.h_r;
    p.h_s = sv.h_s;
    const int64_t hcols = p.I_r > p.I_s ? p.I_r : p.I_s;
    launch_bwd_f32<OP_RECOMP>(p, hcols, 0, (p.TK + p.T) * hcols, st);
    return hipGetLastError();
}

hipError_t launch_expert_ffn_backward(const moe_cfg& c, const FfnBwdArgs& a, void* ws,
                                      hipStream_t st, const void* saved) {
    const int64_t T = c.tokens, TK = T * c.top_k, d = c.hidden, N = c.n_experts;
    const int64_t I = c.inter, Is = c.inter_shared;
    const bool has_shared = Is > 0 && T > 0;
    BwdWs w = carve_bwd(c, ws);
    if (saved) {
        // a, b and h from the training forward
        const SavedActs sv = carve_saved(c, (void*)saved);
        w.ab_r = sv.ab_r;
        w.ab_s = sv.ab_s;
        w.h_r = sv.h_r;
        w.h_s = sv.h_s;
    }
    BwdParams p = bwd_params(c);
    p.offsets = a.offsets;
    p.x_perm = a.x_perm;
    p.x = a.x_sh;
    p.dy_perm = a.dy_perm;
    p.dy_s = a.dy_sh;
    // fp32 layers: the "packed" weights are plain copies (W13 [2I][d], W2 [d][I])
    p.w13 = a.w13;
    p.w2 = a.w2t;
    p.ws13 = a.ws13;
    p.ws2 = a.ws2t;
    p.ab_r = w.ab_r;
    p.ab_s = w.ab_s;
    p.h_r = w.h_r;
    p.h_s = w.h_s;
    p.dab_r = w.dab_r;
    p.dab_s = w.dab_s;
    p.dx_perm = a.dx_perm;
    p.dx_s = a.dx_sh;
    p.dw13 = a.dw13;
    p.dw2 = a.dw2;
    p.dws13 = a.dws13;
    p.dws2 = a.dws2;
    const int64_t Ish = p.I_s;

    if (c.act_dtype == MOE_BF16) {
        if (TK > 0) {
            const hipError_t e = launch_ffn_bwd_dgrad_bf16(c, a, w.tile_ws, w.ab_r, w.ab_s, w.h_r,
                                                           w.h_s, w.dab_r, w.dab_s, !saved, st);
            if (e != hipSuccess) return e;
        }
        // weight gradients: every group, including experts without rows (zeros)
        auto units = [&]() {
            return (has_shared ? p.ntn_s : 0) + 8 * cdiv(N, 8) * p.ntn_r;
        };
        p.ntc_r = cdiv(I, BT);
        p.ntn_r = cdiv(d, BT) * p.ntc_r;
        p.ntc_s = cdiv(Ish, BT);
        p.ntn_s = cdiv(d, BT) * p.ntc_s;
        launch_wgrad_bf16<OP_WGRAD_DOWN>(p, units(), st);
        p.ntc_r = p.ntc_s = cdiv(d, BT);
        p.ntn_r = cdiv(2 * I, BT) * p.ntc_r;
        p.ntn_s = cdiv(2 * Ish, BT) * p.ntc_s;
        launch_wgrad_bf16<OP_WGRAD_UP>(p, units(), st);
    } else {
        const int64_t rows = TK + p.T;
        const int64_t hcols = imax(I, Ish);
        if (!saved) launch_bwd_f32<OP_RECOMP>(p, hcols, 0, rows * hcols, st);
        launch_bwd_f32<OP_DGRAD_DOWN>(p, hcols, 0, rows * hcols, st);
        launch_bwd_f32<OP_DGRAD_UP>(p, d, 0, rows * d, st);
        launch_bwd_f32<OP_WGRAD_DOWN>(p, I, d * I, N * d * I + (has_shared ? d * Is : 0), st);
        launch_bwd_f32<OP_WGRAD_UP>(p, d, 2 * I * d, N * 2 * I * d + (has_shared ? 2 * Is * d : 0), st);
    }
    return hipGetLastError();
}

}  // namespace moe
