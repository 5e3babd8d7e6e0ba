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
// Tile order is XCD-aware (see decode_v2): the units of one tile run on one
// XCD, back to back, so its token rows are shared in L2; tiles go to the XCDs
// round-robin so each gets an even share of routed and shared work.
//
// The same kernel serves three GEMMs of the backward (gemm_bwd.hip), by mode:
//   0  gate/up            h = silu(x W1^T) * (x W3^T)
//   1  down               y = h W2^T  (also the up-projection dgrad dX = [da db] W13,
//                         with the transposed W13 packed as the weights)
//   2  gate/up recompute  mode 0, also storing a and b for the backward
//   3  down dgrad         dh = dY W2 (transposed W2 packed as the weights), and
//                         in the epilogue da = dh b silu'(a), db = dh silu(a)
#include "gemm_common.h"

namespace moe {

static int64_t align256(int64_t b) { return (b + 255) & ~int64_t(255); }

constexpr int BF_BM = 320;      // token rows per tile, bf16 MFMA kernel
constexpr int F32_BM = 64;      // token rows per tile, fp32 path

// ---------------------------------------------------------------- tile map

// Token tiles: routed expert g (rows offsets[g]..offsets[g+1]) gets
// ceil(M_g / BM) tiles, written first; the shared expert (rows 0..T-1) gets
// ceil(T / BM) tiles after them.  tiles[i] = (group, first row); group N is
// the shared expert.  counts[0] = routed tiles, counts[1] = shared tiles.
// Tile list and order.  Routed tiles (expert g, first row m0) come expert by
// expert, then the shared expert's tiles.  `order` lists the routed tiles by
// row count, largest first (counting sort on the count; tiles with equal
// counts in any order -- the order only decides where a tile runs, never what
// it computes).  BM <= TM_MAXBM.
constexpr int TM_MAXBM = 512;
__global__ void __launch_bounds__(256) ffn_tile_map_kernel(const int32_t* __restrict__ offsets,
                                                           int N, int64_t T, int has_shared,
                                                           int BM, int2* __restrict__ tiles,
                                                           int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ order,
                                                           int32_t* __restrict__ keys) {
    __shared__ int32_t sh_wave[4];
    __shared__ int32_t sh_carry;
    __shared__ int32_t hist[TM_MAXBM + 1];
    for (int k = threadIdx.x; k <= BM; k += blockDim.x) hist[k] = 0;
    if (threadIdx.x == 0) sh_carry = 0;
    __syncthreads();
    for (int g0 = 0; g0 < N; g0 += 256) {
        const int g = g0 + threadIdx.x;
        const int64_t M = g < N ? offsets[g + 1] - offsets[g] : 0;
        const int32_t nt = (int32_t)((M + BM - 1) / BM);
        const int32_t incl = block_incl_scan_256(nt, sh_wave);
        const int32_t start = sh_carry + incl - nt;
        for (int32_t i = 0; i < nt; ++i) {
            const int32_t rows = (int32_t)(M - (int64_t)i * BM < BM ? M - (int64_t)i * BM : BM);
            tiles[start + i] = make_int2(g, i * BM);
            keys[start + i] = rows;
            atomicAdd(&hist[rows], 1);
        }
        __syncthreads();
        if (threadIdx.x == 255) sh_carry = sh_carry + incl;
        __syncthreads();
    }
    const int32_t nr = sh_carry;
    // first position of each row count in `order`, largest count first
    __syncthreads();
    if (threadIdx.x == 0) sh_carry = 0;
    __syncthreads();
    for (int k0 = 0; k0 <= BM; k0 += 256) {
        const int k = BM - (k0 + (int)threadIdx.x);  // descending counts
        const int32_t h = k >= 0 ? hist[k] : 0;
        const int32_t incl = block_incl_scan_256(h, sh_wave);
        const int32_t base = sh_carry;
        __syncthreads();
        if (k >= 0) hist[k] = base + incl - h;
        if (threadIdx.x == 255) sh_carry = base + incl;
        __syncthreads();
    }
    for (int32_t t = threadIdx.x; t < nr; t += blockDim.x) order[atomicAdd(&hist[keys[t]], 1)] = t;
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
// MFMA work follows the expert's real row count in steps of 16.
// MFMA v_mfma_f32_16x16x32_bf16 with the weight rows as the A operand:
// D[w][t] = sum_k W[w][k] X[t][k].  Wave (wr = wave%4, tg = wave/4) owns weight
// rows wr*64..+63 (four 16-row blocks) and token rows tg*160..+159 (ten
// blocks); only the blocks that hold real token rows are multiplied (the main
// loop is specialised on that count, so it is straight-line code).  The 16x16
// form rather than 32x32x16: on gfx950 it sustains a higher MFMA rate and slows
// the concurrent global -> LDS copies less (measured 2.8% faster here).
// LDS holds NS stages of BK contraction elements; a stage is a sequence of
// 64-wide sub-tiles, each [rows][8 chunks of 16 B] with chunk c of row r at
// slot c ^ ((r >> 1) & 7), so that the 16 lanes served together by a
// ds_read_b128 (one chunk of 16 consecutive rows) hit distinct banks.  Stages
// are filled by global_load_lds_dwordx4 copies issued NS-1 stages ahead.  The
// weights are pre-packed (pack_weights_kernel) in exactly this LDS image order,
// so a stage's weight copy is one contiguous 256*BK*2-byte read.
// gate/up: the 64 weight rows of a wave are W1 rows n..n+31 (blocks 0, 1) and
// W3 rows n..n+31 (blocks 2, 3): a and b of one (token, column) share a
// register slot and SwiGLU is applied in registers.

constexpr int G_WR = 256;      // weight rows per tile
constexpr int G_TR = 320;      // token rows per tile
// wavefronts per workgroup: 4 weight-row groups of 64 x 2 token halves
constexpr int G_WAVES = 8;
constexpr int G_THREADS = 64 * G_WAVES;
constexpr int G_WRG = G_WAVES / 2;        // weight-row groups
// contraction step and number of LDS stages in the copy pipeline
#ifndef MOE_GEMM_BK
#define MOE_GEMM_BK 64
#endif
#ifndef MOE_GEMM_NS
#define MOE_GEMM_NS 2
#endif
// token fragments read ahead of their MFMAs in the scheduled step sequence
#ifndef MOE_GEMM_LA
#define MOE_GEMM_LA 5
#endif
// contraction elements per LDS sub-tile: one step up to 64 (rows of 2*G_SUB
// bytes), and the 16-byte chunks per row with their bank-spreading swizzle
constexpr int G_SUB = MOE_GEMM_BK < 64 ? MOE_GEMM_BK : 64;
constexpr int G_CPR = G_SUB / 8;
static_assert(G_CPR == 4 || G_CPR == 8, "LDS rows of 64 or 128 bytes");
__device__ __forceinline__ int g_swz(int r, int c) {
    return G_CPR == 8 ? sub_chunk8(r, c) : sub_chunk(r, c);
}
constexpr int G_RPB = 1024 / (2 * G_SUB);  // rows per 1 KB copy

// Pack a stack of n_mats expert matrices into the GEMM's LDS image order:
// out[mat][wt][kc][slot] (16-byte chunks), kc = G_SUB-wide contraction block,
// slot = r*G_CPR + pc holding logical chunk g_swz(r, pc) of packed row r.
template <int MODE>
__global__ void __launch_bounds__(256) pack_weights_kernel(const uint4* __restrict__ w,
                                                           uint4* __restrict__ out,
                                                           int64_t n_mats, int64_t Nout,
                                                           int64_t K, int64_t ntn) {
    const int64_t nkc = K / G_SUB;
    const int64_t per_mat = ntn * nkc * G_WR * G_CPR;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_mats * per_mat) return;
    const int64_t mat = i / per_mat;
    int64_t rem = i % per_mat;
    const int64_t wt = rem / (nkc * G_WR * G_CPR);
    rem %= nkc * G_WR * G_CPR;
    const int64_t kc = rem / (G_WR * G_CPR);
    const int slot = (int)(rem % (G_WR * G_CPR));
    const int r = slot / G_CPR, c = g_swz(r, slot % G_CPR);
    const int64_t src = packed_row_source<MODE>(wt, r, Nout);
    const int64_t rows = MODE == 0 ? 2 * Nout : Nout;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (src >= 0) v = w[((mat * rows + src) * K + kc * G_SUB + c * 8) / 8];
    out[i] = v;
}

// Transposed packing, for the backward's dgrad GEMMs: packed row r of weight
// tile wt is column wt*256 + r of a matrix stored [K][Nout] (zero past Nout),
// in the same LDS image order as above.
__global__ void __launch_bounds__(256) pack_weights_t_kernel(const uint16_t* __restrict__ w,
                                                             uint4* __restrict__ out,
                                                             int64_t n_mats, int64_t Nout,
                                                             int64_t K, int64_t ntn) {
    const int64_t nkc = K / G_SUB;
    const int64_t per_mat = ntn * nkc * G_WR * G_CPR;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_mats * per_mat) return;
    const int64_t mat = i / per_mat;
    int64_t rem = i % per_mat;
    const int64_t wt = rem / (nkc * G_WR * G_CPR);
    rem %= nkc * G_WR * G_CPR;
    const int64_t kc = rem / (G_WR * G_CPR);
    const int slot = (int)(rem % (G_WR * G_CPR));
    const int r = slot / G_CPR, c = g_swz(r, slot % G_CPR);
    const int64_t col = wt * G_WR + r;
    uint32_t v[4] = {0, 0, 0, 0};
    if (col < Nout) {
        const uint16_t* src = w + (mat * K + kc * G_SUB + c * 8) * Nout + col;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            v[e] = (uint32_t)src[(2 * e) * Nout] | ((uint32_t)src[(2 * e + 1) * Nout] << 16);
    }
    out[i] = make_uint4(v[0], v[1], v[2], v[3]);
}

// 16-byte-per-lane global -> LDS copy (lane i's bytes land at lds + 16 i).
// Written as asm so that the compiler's waitcnt bookkeeping does not see it:
// a pending builtin LDS-DMA copy counts there as an LDS access of unknown
// order, after which every wait for an LDS fragment read becomes lgkmcnt(0),
// i.e. for all reads in flight, and reads cannot run ahead of the MFMAs.
// The caller waits for the copies itself (vmcnt), also before the LDS is
// reused.  Five wait states first: the M0 and address set-up just before may
// come from VALU-written SGPRs.
__device__ __forceinline__ void copy16_to_lds(const void* g, const void* lds) {
    const uint32_t m0 = (uint32_t)(uintptr_t)lds;
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(m0) : "memory");
}

template <int MODE, int BK, int NS, int NB>
__device__ __forceinline__ void gemm_bf16_body(const WorkV2& w, uint16_t* smem) {
    constexpr int NSUB = BK / G_SUB;
    constexpr int A_EL = G_WR * BK, X_EL = G_TR * BK;
    constexpr int NA = A_EL * 2 / 1024;         // 1 KB copies per stage (weights)
    constexpr int NX = X_EL * 2 / 1024;         // 1 KB copies per stage (tokens, at most)
    constexpr int PA = NA / G_WAVES, PX = (NX + G_WAVES - 1) / G_WAVES;
    constexpr int NBB = NB > 0 ? NB : 1;
    static_assert(NA % G_WAVES == 0, "weight copies split evenly over the waves");
    static_assert(BK % G_SUB == 0, "contraction step is a whole number of LDS sub-tiles");

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave % G_WRG, tg = wave / G_WRG;  // weight-row group, token half
    const int64_t K = w.K;
    const int64_t mc = w.M - w.m0 < G_TR ? w.M - w.m0 : G_TR;
    const int nk = (int)(K / BK);
    // uniform bases + 32-bit per-lane byte offsets (scalar-base addressing)
    const char* wstage0 = w.W + (w.wt * (int64_t)nk * A_EL) * 2;
    const uint32_t woff = lane * 16;
    // the tile's first token row; with a gather list the rows come from
    // anywhere in X and each lane's offset carries its row
    const char* xbase = w.gather ? w.X : w.X + w.m0 * K * 2;

    // Token copies: block b = G_RPB rows (rb = b / NSUB) of sub-tile q = b % NSUB,
    // each row one 2*G_SUB-byte line; the blocks holding real rows are the
    // prefix b < nxe.  Rows past the tile's last real row are never copied
    // (their LDS is never stored from).
    const int nxe = NSUB * (int)((mc + G_RPB - 1) / G_RPB);
    int cnt = PA;  // copies this wave issues per stage
    uint32_t xoff[PX];
#pragma unroll
    for (int j = 0; j < PX; ++j) {
        const int b = wave + G_WAVES * j;
        if (b < nxe) ++cnt;
        const int q = b % NSUB, rb = b / NSUB;
        const int r = rb * G_RPB + (int)((unsigned)lane / G_CPR), c = g_swz(r, (int)((unsigned)lane % G_CPR));
        const int64_t tr = r < mc ? r : mc - 1;  // clamp inside a partial block
        const int64_t sr = w.gather ? (int64_t)w.gather[w.m0 + tr] : tr;
        xoff[j] = (uint32_t)((sr * K + q * G_SUB + c * 8) * 2);
    }

    auto stage_a = [&](int s) { return smem + s * (A_EL + X_EL); };
    auto stage_x = [&](int s) { return smem + s * (A_EL + X_EL) + A_EL; };
    auto issue = [&](int kt, int s) {
        uint16_t* As = stage_a(s);
        uint16_t* Xs = stage_x(s);
        const char* wsrc = wstage0 + (int64_t)kt * A_EL * 2;
        const char* xsrc = xbase + (int64_t)kt * BK * 2;
#pragma unroll
        for (int j = 0; j < PA; ++j) {
            const int b = wave + G_WAVES * j;
            copy16_to_lds((const void*)(wsrc + b * 1024 + woff), As + b * 512);
        }
#pragma unroll
        for (int j = 0; j < PX; ++j) {
            const int b = wave + G_WAVES * j;
            if (b < nxe)
                copy16_to_lds((const void*)(xsrc + xoff[j]),
                              Xs + (b % NSUB) * G_TR * G_SUB + (b / NSUB) * 512);
        }
    };

    // 16x16x32 MFMAs: wave (wr, tg) owns weight rows wr*64 + 16i + 0..15
    // (i = 0..3) and token rows tg*160 + 16j + 0..15 (j < NB)
    f32x4_t acc[4][NBB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NBB; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const int l16 = lane & 15, g = lane >> 4;
    // rows 16k + l16 share l16's swizzle: chunk offsets are lane constants
    uint32_t coff[G_SUB / 32];
#pragma unroll
    for (int s = 0; s < G_SUB / 32; ++s) coff[s] = g_swz(l16, 4 * s + g) * 8;

    // One step as one scheduled sequence, weight-fragment-major: pass i of a
    // 32-wide substep multiplies weight fragment i with all NB token
    // fragments, so the first MFMA of a substep waits for two reads, not five.
    // Reads are held (sched_group_barrier) to [A0, X0..X(L-1), A1] up front,
    // then one per MFMA of pass 0 (X(L).., A2, A3); pass 3 of a substep
    // issues the next substep's first reads into the registers its own MFMAs
    // have just freed.  Each MFMA then waits only for the reads it uses
    // (partial lgkmcnt waits), and the other wave of the SIMD fills the rest.
    // The products and their order per accumulator are those of the plain
    // loop below (k ascending), so the results are the same bits.
    constexpr int LA = MOE_GEMM_LA;
    auto compute_seq = [&](auto sidx) {  // generic: instantiated only when NB >= LA
        constexpr int SUBS = BK / 32;
        const uint16_t* As = stage_a(sidx);
        const uint16_t* Xs = stage_x(sidx);
        bf16x8_t af[SUBS][4], xf[SUBS][NBB];
        auto rda = [&](int s, int i) {
            const int q = s / (G_SUB / 32);
            return __builtin_bit_cast(bf16x8_t, *(const uint4*)(As + q * G_WR * G_SUB +
                (wr * 64 + i * 16 + l16) * G_SUB + coff[s % (G_SUB / 32)]));
        };
        auto rdx = [&](int s, int j) {
            const int q = s / (G_SUB / 32);
            return __builtin_bit_cast(bf16x8_t, *(const uint4*)(Xs + q * G_TR * G_SUB +
                (tg * 160 + j * 16 + l16) * G_SUB + coff[s % (G_SUB / 32)]));
        };
#pragma unroll
        for (int s = 0; s < SUBS; ++s) {
            af[s][0] = rda(s, 0);
#pragma unroll
            for (int j = 0; j < LA; ++j) xf[s][j] = rdx(s, j);
            af[s][1] = rda(s, 1);
#pragma unroll
            for (int j = LA; j < NB; ++j) xf[s][j] = rdx(s, j);
            af[s][2] = rda(s, 2);
            af[s][3] = rda(s, 3);
        }
#pragma unroll
        for (int s = 0; s < SUBS; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s][i], xf[s][j], acc[i][j], 0, 0, 0);
        constexpr int R0 = LA + 2;       // reads before the first MFMA of a substep
        constexpr int RP = NB - LA + 2;  // reads of a substep during its pass 0
        __builtin_amdgcn_sched_group_barrier(0x100, R0, 0);  // 0x100: LDS reads
#pragma unroll
        for (int s = 0; s < SUBS; ++s) {
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 0x008: MFMA
                if (j < RP) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            if constexpr (RP > NB) __builtin_amdgcn_sched_group_barrier(0x100, RP - NB, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2 * NB, 0);
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (s + 1 < SUBS && j < R0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            if constexpr (R0 > NB)
                if (s + 1 < SUBS) __builtin_amdgcn_sched_group_barrier(0x100, R0 - NB, 0);
        }
    };
    auto compute = [&](int sidx) {
        if constexpr (NB >= LA) {
            compute_seq(sidx);
        } else if constexpr (NB > 0) {
            const uint16_t* As = stage_a(sidx);
            const uint16_t* Xs = stage_x(sidx);
#pragma unroll
            for (int s = 0; s < BK / 32; ++s) {
                const int q = s / (G_SUB / 32);
                const uint32_t co = coff[s % (G_SUB / 32)];
                bf16x8_t af[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    af[i] = __builtin_bit_cast(
                        bf16x8_t, *(const uint4*)(As + q * G_WR * G_SUB + (wr * 64 + i * 16 + l16) * G_SUB + co));
                const uint16_t* xrow = Xs + q * G_TR * G_SUB + (tg * 160 + l16) * G_SUB + co;
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const bf16x8_t xf = __builtin_bit_cast(bf16x8_t, *(const uint4*)(xrow + j * 16 * G_SUB));
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], xf, acc[i][j], 0, 0, 0);
                }
            }
        }
    };

#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
        if (s < nk) issue(s, s);
    for (int kt = 0; kt < nk; ++kt) {
        // copies issued by this wave after stage kt's may stay in flight:
        // later stages, cnt each
        const int after = nk - 1 - kt < NS - 2 ? nk - 1 - kt : NS - 2;
        vm_wait_n(after * cnt);
        // this wave's copies of stage kt have landed (its own vmcnt); the
        // barrier makes that true for every wave, and stage kt-1 is free
        lds_barrier();
        if (kt + NS - 1 < nk) issue(kt + NS - 1, (kt + NS - 1) % NS);
        compute(kt % NS);
    }

    // Epilogue.  The output tile goes through LDS so that global stores are
    // whole 16-byte row chunks: gate/up writes 128 h columns of every row at
    // once; down writes 256 y columns in two passes (token halves).  LDS rows
    // are padded by 16 bytes so the 16 rows written by a lane group hit
    // distinct banks.
    vm_wait<0>();     // no copy of this wave in flight (the asm copies are not tracked)
    __syncthreads();  // every wave is done with the stage buffers
    constexpr bool GU = MODE == 0 || MODE == 2;  // gate/up-shaped tile
    constexpr int OCOLS = GU ? 128 : 256;
    constexpr int OSTR = OCOLS + 8;  // padded LDS row (elements)
    uint16_t* ot = smem;
    const int64_t wbase = GU ? w.wt * 128 : w.wt * 256;
    auto put = [&](int row, int col, float a0, float a1, float a2, float a3) {
        *(uint2*)(ot + row * OSTR + col) = make_uint2(pack_bf16x2(a0, a1), pack_bf16x2(a2, a3));
    };
    auto flush_rows = [&](int r0, int nrows) {
        // tile rows r0 .. r0+nrows-1 (held in LDS rows 0 ..) -> global,
        // 16 bytes per thread
        constexpr int CH = OCOLS / 8;
        uint16_t* C = (uint16_t*)w.C;
        for (int q = threadIdx.x; q < nrows * CH; q += G_THREADS) {
            const int rr = q / CH, ch = q % CH;
            const int64_t col = wbase + ch * 8;
            if (r0 + rr < mc && col < w.Nout)
                *(uint4*)(C + (w.m0 + r0 + rr) * w.Nout + col) = *(const uint4*)(ot + rr * OSTR + ch * 8);
        }
    };
    // 16x16 layout: lane l holds column (token) l%16 and rows 4*(l/16) + v of
    // its block.  gate/up: blocks 0, 1 are the W1 rows and 2, 3 the W3 rows of
    // the wave's h columns 32*wr + 16*i + 4*g + v.
    if (GU) {
        if constexpr (NB > 0) {
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int row = tg * 160 + j * 16 + l16;
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    float h[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v) h[v] = silu_f(acc[i][j][v]) * acc[i + 2][j][v];
                    put(row, wr * 32 + i * 16 + 4 * g, h[0], h[1], h[2], h[3]);
                    if (MODE == 2 && row < mc) {
                        // a and b (rounded to bf16) for the backward: row of E is [a | b]
                        uint16_t* e = (uint16_t*)w.E + (w.m0 + row) * 2 * w.Nout + wbase +
                                      wr * 32 + i * 16 + 4 * g;
                        *(uint2*)e = make_uint2(pack_bf16x2(acc[i][j][0], acc[i][j][1]),
                                                pack_bf16x2(acc[i][j][2], acc[i][j][3]));
                        *(uint2*)(e + w.Nout) =
                            make_uint2(pack_bf16x2(acc[i + 2][j][0], acc[i + 2][j][1]),
                                       pack_bf16x2(acc[i + 2][j][2], acc[i + 2][j][3]));
                    }
                }
            }
        }
        __syncthreads();
        flush_rows(0, (int)mc);
    } else if (MODE == 3) {
        // dh of token row m, columns n..n+3 -> da, db (direct 8-byte stores);
        // a, b are read back from E, the recompute's bf16 copy
        if constexpr (NB > 0) {
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int row = tg * 160 + j * 16 + l16;
                if (row >= mc) continue;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t n = wbase + wr * 64 + i * 16 + 4 * g;
                    if (n >= w.Nout) continue;
                    const uint16_t* e = (const uint16_t*)w.E + (w.m0 + row) * 2 * w.Nout + n;
                    const uint2 qa = *(const uint2*)e;
                    const uint2 qb = *(const uint2*)(e + w.Nout);
                    const float a[4] = {__uint_as_float(qa.x << 16), __uint_as_float(qa.x & 0xffff0000u),
                                        __uint_as_float(qa.y << 16), __uint_as_float(qa.y & 0xffff0000u)};
                    const float b[4] = {__uint_as_float(qb.x << 16), __uint_as_float(qb.x & 0xffff0000u),
                                        __uint_as_float(qb.y << 16), __uint_as_float(qb.y & 0xffff0000u)};
                    float da[4], db[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-a[v]));
                        const float dh = acc[i][j][v];
                        da[v] = dh * b[v] * sg * (1.0f + a[v] * (1.0f - sg));
                        db[v] = dh * a[v] * sg;
                    }
                    uint16_t* o = (uint16_t*)w.C + (w.m0 + row) * 2 * w.Nout + n;
                    *(uint2*)o = make_uint2(pack_bf16x2(da[0], da[1]), pack_bf16x2(da[2], da[3]));
                    *(uint2*)(o + w.Nout) = make_uint2(pack_bf16x2(db[0], db[1]),
                                                       pack_bf16x2(db[2], db[3]));
                }
            }
        }
    } else {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            if (half == 1) lds_barrier();  // the first half's rows are read out of LDS
            if constexpr (NB > 0) {
                if (tg == half) {
#pragma unroll
                    for (int j = 0; j < NB; ++j) {
                        const int row = j * 16 + l16;
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            put(row, wr * 64 + i * 16 + 4 * g, acc[i][j][0], acc[i][j][1],
                                acc[i][j][2], acc[i][j][3]);
                    }
                }
            }
            lds_barrier();
            const int nrows = (int)(mc - half * 160 < 160 ? mc - half * 160 : 160);
            if (nrows > 0) flush_rows(half * 160, nrows);
        }
    }
}

template <int MODE, int BK, int NS>
__global__ void __launch_bounds__(G_THREADS, 1) ffn_gemm_bf16_kernel(GemmParamsV2 p) {
    WorkV2 w;
    if (!decode_v2<2>(p, MODE, w)) return;
    constexpr int STAGES_EL = NS * (G_WR + G_TR) * BK;
    constexpr bool GU = MODE == 0 || MODE == 2;
    constexpr int EPI_EL = GU ? G_TR * (128 + 8) : 160 * (256 + 8);
    __shared__ __attribute__((aligned(1024))) uint16_t smem[STAGES_EL > EPI_EL ? STAGES_EL : EPI_EL];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave % G_WRG, tg = wave / G_WRG;
    const int64_t mc = w.M - w.m0 < G_TR ? w.M - w.m0 : G_TR;
    // token blocks of this wave that hold real rows; none if all its weight rows
    // are past the end of the matrix (last tile of the down projection)
    int64_t nb = (mc - tg * 160 + 15) / 16;
    nb = nb < 0 ? 0 : (nb > 10 ? 10 : nb);
    const int64_t wbase = GU ? w.wt * 128 : w.wt * 256;
    if (!GU && wbase + wr * 64 >= w.Nout) nb = 0;
    switch (nb) {
        case 10: gemm_bf16_body<MODE, BK, NS, 10>(w, smem); break;
        case 9: gemm_bf16_body<MODE, BK, NS, 9>(w, smem); break;
        case 8: gemm_bf16_body<MODE, BK, NS, 8>(w, smem); break;
        case 7: gemm_bf16_body<MODE, BK, NS, 7>(w, smem); break;
        case 6: gemm_bf16_body<MODE, BK, NS, 6>(w, smem); break;
        case 5: gemm_bf16_body<MODE, BK, NS, 5>(w, smem); break;
        case 4: gemm_bf16_body<MODE, BK, NS, 4>(w, smem); break;
        case 3: gemm_bf16_body<MODE, BK, NS, 3>(w, smem); break;
        case 2: gemm_bf16_body<MODE, BK, NS, 2>(w, smem); break;
        case 1: gemm_bf16_body<MODE, BK, NS, 1>(w, smem); break;
        default: gemm_bf16_body<MODE, BK, NS, 0>(w, smem); break;
    }
}

// ---------------------------------------------------------------- fp32 path
// VALU kernel for fp32 storage (small layers): 64 token rows x 64 output
// columns per 256-thread block; thread = (row tid%64, columns (tid/64)*16..+15),
// each output one fma chain over k ascending from +0.  The block's token rows
// and weight rows pass through LDS F32_KC contraction elements at a time
// (coalesced global loads), so the chains read their operands from LDS
// instead of waiting on a global load per step.
constexpr int F32_KC = 32;

template <int MODE>
__global__ void __launch_bounds__(256) ffn_gemm_f32_kernel(GemmParamsV2 p) {
    WorkV2 w;
    if (!decode_v2<4>(p, MODE, w)) return;
    constexpr int WR = MODE == 0 ? 128 : 64;  // staged weight rows: W1 then W3, or W2
    __shared__ float xs[64][F32_KC + 1];
    __shared__ float wsm[WR][F32_KC + 1];
    const int tid = threadIdx.x;
    const int rl = tid & 63, cg = tid >> 6;
    const int64_t K = w.K;
    const int64_t mrows = w.M - w.m0 < 64 ? w.M - w.m0 : 64;
    const float* X = (const float*)w.X;
    const float* B = (const float*)w.W;
    const int64_t cbase = w.wt * 64;
    float sa[16], sb[16];
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) sa[jj] = sb[jj] = 0.0f;
    for (int64_t k0 = 0; k0 < K; k0 += F32_KC) {
        const int kc = (int)(K - k0 < F32_KC ? K - k0 : F32_KC);
        __syncthreads();  // the previous chunk has been read
        for (int i = tid; i < 64 * F32_KC; i += 256) {
            const int rr = i / F32_KC, kk = i % F32_KC;
            xs[rr][kk] = rr < mrows && kk < kc ? X[(w.m0 + rr) * K + k0 + kk] : 0.0f;
        }
        for (int i = tid; i < WR * F32_KC; i += 256) {
            const int wr = i / F32_KC, kk = i % F32_KC;
            const int64_t c = cbase + (wr & 63);
            const int64_t row = MODE == 0 && wr >= 64 ? w.Nout + c : c;
            wsm[wr][kk] = c < w.Nout && kk < kc ? B[row * K + k0 + kk] : 0.0f;
        }
        __syncthreads();
        for (int kk = 0; kk < kc; ++kk) {
            const float a = xs[rl][kk];
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                sa[jj] = __builtin_fmaf(a, wsm[cg * 16 + jj][kk], sa[jj]);
                if (MODE == 0) sb[jj] = __builtin_fmaf(a, wsm[64 + cg * 16 + jj][kk], sb[jj]);
            }
        }
    }
    if (rl >= mrows) return;
    float* C = (float*)w.C;
    const int64_t r = w.m0 + rl;
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
        const int64_t c = cbase + cg * 16 + jj;
        if (c < w.Nout)
            C[r * w.Nout + c] = MODE == 0 ? sa[jj] / (1.0f + expf(-sa[jj])) * sb[jj] : sa[jj];
    }
}

// ---------------------------------------------------------------- launch

struct FfnWs {
    int2* tiles;
    int32_t* counts;  // [2]
    int32_t* order;   // routed tiles, largest first [max routed tiles]
    int32_t* keys;    // row count of each routed tile [max routed tiles]
    void* h_r;        // [TK, I]
    void* h_s;        // [T, Is]
    float* hs_r;      // FP8 scales [TK, I/128]
    float* hs_s;      // FP8 scales [T, Is/128]
};

static int ffn_bm(const moe_cfg& c) {
    if (c.gemm_dtype == MOE_FP8_E4M3) return FP8_BM;
    return c.act_dtype == MOE_F32 ? F32_BM : BF_BM;
}

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
    b += 2 * align256(ffn_max_routed_tiles(c) * 4);
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
    w.order = (int32_t*)p;
    p += align256(ffn_max_routed_tiles(c) * 4);
    w.keys = (int32_t*)p;
    p += align256(ffn_max_routed_tiles(c) * 4);
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

// ---------------------------------------------------------------- weight packing

struct PackShape {
    int mode;  // 0 gate/up, 1 plain rows, 2 transposed (source [K][Nout])
    int64_t n_mats, Nout, K, ntn;
};

// which: 0/2 W13 (routed/shared), 1/3 W2, and for the backward's dgrad
// GEMMs 4/6 W13 transposed (rows = d, K = 2I), 5/7 W2 transposed (rows = I, K = d)
static PackShape pack_shape(const moe_cfg& c, int which) {
    const bool routed = which == 0 || which == 1 || which == 4 || which == 5;
    const int64_t n = routed ? c.n_experts : 1;
    const int64_t I = routed ? c.inter : c.inter_shared;
    if (which == 0 || which == 2) return {0, n, I, c.hidden, cdiv(I, 128)};
    if (which == 1 || which == 3) return {1, n, c.hidden, I, cdiv(c.hidden, 256)};
    if (which == 4 || which == 6) return {2, n, c.hidden, 2 * I, cdiv(c.hidden, 256)};
    return {2, n, I, c.hidden, cdiv(I, 256)};
}

size_t packed_weight_bytes(const moe_cfg& c, int which) {
    const PackShape s = pack_shape(c, which);
    if (c.act_dtype == MOE_F32 && c.gemm_dtype == MOE_F32)
        return (size_t)(s.n_mats * (s.mode == 0 ? 2 * s.Nout : s.Nout) * s.K * 4);
    if (c.gemm_dtype == MOE_FP8_E4M3) return packed_weight_bytes_fp8(c, which);
    return (size_t)(s.n_mats * s.ntn * G_WR * s.K * 2);
}

hipError_t launch_pack_weights(const moe_cfg& c, int which, const void* w, void* out,
                               hipStream_t st) {
    const PackShape s = pack_shape(c, which);
    if (s.n_mats == 0 || s.Nout == 0) return hipSuccess;
    if (c.act_dtype == MOE_F32 && c.gemm_dtype == MOE_F32)
        return hipMemcpyAsync(out, w, packed_weight_bytes(c, which), hipMemcpyDeviceToDevice, st);
    if (c.gemm_dtype == MOE_FP8_E4M3) return launch_pack_weights_fp8(c, which, w, out, st);
    const int64_t n = s.n_mats * s.ntn * (s.K / G_SUB) * G_WR * G_CPR;
    const unsigned blocks = (unsigned)cdiv(n, 256);
    if (s.mode == 2)
        pack_weights_t_kernel<<<blocks, 256, 0, st>>>((const uint16_t*)w, (uint4*)out, s.n_mats,
                                                      s.Nout, s.K, s.ntn);
    else if (s.mode == 0)
        pack_weights_kernel<0><<<blocks, 256, 0, st>>>((const uint4*)w, (uint4*)out, s.n_mats,
                                                       s.Nout, s.K, s.ntn);
    else
        pack_weights_kernel<1><<<blocks, 256, 0, st>>>((const uint4*)w, (uint4*)out, s.n_mats,
                                                       s.Nout, s.K, s.ntn);
    return hipGetLastError();
}

void launch_tile_map(const int32_t* offsets, int N, int64_t T, bool has_shared, int BM,
                     int2* tiles, int32_t* counts, int32_t* order, int32_t* keys, hipStream_t st) {
    ffn_tile_map_kernel<<<1, 256, 0, st>>>(offsets, N, T, has_shared ? 1 : 0, BM, tiles, counts,
                                           order, keys);
}

hipError_t launch_expert_ffn_fp8(const moe_cfg& c, const FfnArgs& a, const int2* tiles,
                                 const int32_t* counts, const int32_t* order, void* h_r,
                                 void* h_s, float* hs_r, float* hs_s, int64_t max_r,
                                 int64_t max_s, hipStream_t st, const SavedActs* sv,
                                 float* hf_r, float* hf_s);

void ffn_h_offsets(const moe_cfg& c, size_t off[4]) {
    char* base = (char*)(uintptr_t)4096;  // any aligned base: only differences are used
    const FfnWs w = carve_ffn(c, base);
    off[0] = (size_t)((char*)w.h_r - base);
    off[1] = (size_t)((char*)w.h_s - base);
    const bool fp8 = c.gemm_dtype == MOE_FP8_E4M3;
    off[2] = fp8 ? (size_t)((char*)w.hs_r - base) : SIZE_MAX;
    off[3] = fp8 ? (size_t)((char*)w.hs_s - base) : SIZE_MAX;
}

hipError_t launch_expert_ffn(const moe_cfg& c, const FfnArgs& a, void* ws, hipStream_t st,
                             void* saved, float* hf_r, float* hf_s) {
    const int64_t T = c.tokens, TK = T * c.top_k;
    const bool has_shared = c.inter_shared > 0 && T > 0;
    if (TK == 0) return hipSuccess;
    FfnWs w = carve_ffn(c, ws);
    SavedActs sv{};
    const bool fp8 = c.gemm_dtype == MOE_FP8_E4M3;
    if (saved && fp8) {
        sv = carve_saved(c, saved);  // FP8: the h codes stay in the workspace
    } else if (saved) {
        // training forward: h lives in the saved activations (with a, b)
        sv = carve_saved(c, saved);
        w.h_r = sv.h_r;
        w.h_s = sv.h_s;
    }
    const int BM = ffn_bm(c);
    const int64_t max_r = ffn_max_routed_tiles(c);
    const int64_t max_s = has_shared ? ffn_max_shared_tiles(c) : 0;
    launch_tile_map(a.offsets, (int)c.n_experts, T, has_shared, BM, w.tiles, w.counts, w.order,
                    w.keys, st);
    if (fp8)
        return launch_expert_ffn_fp8(c, a, w.tiles, w.counts, w.order, w.h_r, w.h_s, w.hs_r, w.hs_s,
                                     max_r, max_s, st, saved ? &sv : nullptr, hf_r, hf_s);

    GemmParamsV2 p{};
    p.tiles = w.tiles;
    p.counts = w.counts;
    p.order = w.order;
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
    p.gather_r = a.gather;  // bf16 inference only (checked by the caller)
    const int cols0 = bf ? 128 : 64;
    p.ntn_r = (int)cdiv(c.inter, cols0);
    p.ntn_s = has_shared ? (int)cdiv(c.inter_shared, cols0) : 0;
    // a block for every (XCD, slot) the mapping can produce
    unsigned grid = (unsigned)ffn_grid_blocks(max_r, p.ntn_r, max_s, p.ntn_s);
    if (bf && saved) {
        p.E_r = sv.ab_r;  // mode 2: also a and b
        p.E_s = sv.ab_s;
        ffn_gemm_bf16_kernel<2, MOE_GEMM_BK, MOE_GEMM_NS><<<grid, G_THREADS, 0, st>>>(p);
        p.E_r = p.E_s = nullptr;
    } else if (bf) {
        ffn_gemm_bf16_kernel<0, MOE_GEMM_BK, MOE_GEMM_NS><<<grid, G_THREADS, 0, st>>>(p);
    } else if (saved) {
        const hipError_t e = launch_ffn_save_f32(c, a.x_perm, a.x_sh, a.offsets, a.w13, a.ws13,
                                                 saved, st);
        if (e != hipSuccess) return e;
    } else {
        ffn_gemm_f32_kernel<0><<<grid, 256, 0, st>>>(p);
    }

    // down: h x W2 -> y  (bf16: 256 output columns per weight tile)
    p.gather_r = nullptr;
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
    grid = (unsigned)ffn_grid_blocks(max_r, p.ntn_r, max_s, p.ntn_s);
    if (bf)
        ffn_gemm_bf16_kernel<1, MOE_GEMM_BK, MOE_GEMM_NS><<<grid, G_THREADS, 0, st>>>(p);
    else
        ffn_gemm_f32_kernel<1><<<grid, 256, 0, st>>>(p);
    return hipGetLastError();
}

}  // namespace moe

namespace moe {

// ---------------------------------------------------------------- backward GEMMs
// Recompute (unless a training forward saved a, b and h), down-projection dgrad
// and up-projection dgrad of the backward, on the forward's kernel (modes 2, 3
// and 1).  The tile list is built here with the forward's row tile.
size_t ffn_bwd_tile_ws_bytes(const moe_cfg& c) {
    return (size_t)(align256((ffn_max_routed_tiles(c) + ffn_max_shared_tiles(c)) * 8) + 256 +
                    2 * align256(ffn_max_routed_tiles(c) * 4));
}

hipError_t launch_ffn_bwd_dgrad_bf16(const moe_cfg& c, const FfnBwdArgs& a, void* tile_ws,
                                     void* ab_r, void* ab_s, void* h_r, void* h_s, void* dab_r,
                                     void* dab_s, bool recompute, hipStream_t st) {
    const int64_t T = c.tokens, d = c.hidden, I = c.inter, Is = c.inter_shared;
    const bool has_shared = Is > 0 && T > 0;
    char* q = (char*)tile_ws;
    int2* tiles = (int2*)q;
    q += align256((ffn_max_routed_tiles(c) + ffn_max_shared_tiles(c)) * 8);
    int32_t* counts = (int32_t*)q;
    q += 256;
    int32_t* order = (int32_t*)q;
    q += align256(ffn_max_routed_tiles(c) * 4);
    int32_t* keys = (int32_t*)q;
    const int64_t max_r = ffn_max_routed_tiles(c);
    const int64_t max_s = has_shared ? ffn_max_shared_tiles(c) : 0;
    launch_tile_map(a.offsets, (int)c.n_experts, T, has_shared, BF_BM, tiles, counts, order, keys,
                    st);
    GemmParamsV2 p{};
    p.tiles = tiles;
    p.counts = counts;
    p.order = order;
    p.offsets = a.offsets;
    p.N = (int)c.n_experts;
    p.T = has_shared ? T : 0;
    // recompute: a, b (E) and h (C) from x and the forward-packed W13
    p.K_r = p.K_s = d;
    p.Nout_r = I;
    p.Nout_s = Is;
    p.A_r = a.x_perm;
    p.A_s = a.x_sh;
    p.B_r = a.w13;
    p.B_s = a.ws13;
    p.C_r = h_r;
    p.C_s = h_s;
    p.E_r = ab_r;
    p.E_s = ab_s;
    p.ntn_r = (int)cdiv(I, 128);
    p.ntn_s = has_shared ? (int)cdiv(Is, 128) : 0;
    unsigned grid = (unsigned)ffn_grid_blocks(max_r, p.ntn_r, max_s, p.ntn_s);
    if (recompute) ffn_gemm_bf16_kernel<2, MOE_GEMM_BK, MOE_GEMM_NS><<<grid, G_THREADS, 0, st>>>(p);
    // down dgrad: dh = dY W2 (W2 transposed and packed), epilogue -> da, db
    p.A_r = a.dy_perm;
    p.A_s = a.dy_sh;
    p.B_r = a.w2t;
    p.B_s = a.ws2t;
    p.C_r = dab_r;
    p.C_s = dab_s;
    p.c_stride2 = 1;
    p.ntn_r = (int)cdiv(I, 256);
    p.ntn_s = has_shared ? (int)cdiv(Is, 256) : 0;
    grid = (unsigned)ffn_grid_blocks(max_r, p.ntn_r, max_s, p.ntn_s);
    ffn_gemm_bf16_kernel<3, MOE_GEMM_BK, MOE_GEMM_NS><<<grid, G_THREADS, 0, st>>>(p);
    // up dgrad: dX = [da db] W13 (W13 transposed and packed), K = 2I
    p.K_r = 2 * I;
    p.K_s = 2 * Is;
    p.Nout_r = p.Nout_s = d;
    p.A_r = dab_r;
    p.A_s = dab_s;
    p.B_r = a.w13t;
    p.B_s = a.ws13t;
    p.C_r = a.dx_perm;
    p.C_s = a.dx_sh;
    p.E_r = p.E_s = nullptr;
    p.c_stride2 = 0;
    p.ntn_r = (int)cdiv(d, 256);
    p.ntn_s = has_shared ? (int)cdiv(d, 256) : 0;
    grid = (unsigned)ffn_grid_blocks(max_r, p.ntn_r, max_s, p.ntn_s);
    ffn_gemm_bf16_kernel<1, MOE_GEMM_BK, MOE_GEMM_NS><<<grid, G_THREADS, 0, st>>>(p);
    return hipGetLastError();
}

}  // namespace moe
