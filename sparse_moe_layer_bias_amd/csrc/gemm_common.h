// gemm_common.h -- pieces shared by the bf16 and FP8 grouped expert GEMMs:
// work-unit decoding over the device tile list, LDS addressing helpers and
// the packed weight-tile row map.
#pragma once

#include "moe_internal.h"

namespace moe {

constexpr int G_WR_PACK = 256;  // rows per packed weight tile

// ---------------------------------------------------------------- work units

struct GemmParamsV2 {
    const int2* tiles;     // routed tiles [0, n_r), shared tiles [n_r, n_r + n_s)
    const int32_t* counts; // [0] = routed tiles, [1] = shared tiles
    const int32_t* order;  // routed tiles, largest first
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
    // backward launches only: [rows][2 Nout] side array of the epilogue -- the
    // stored a, b (written by the recompute, read by the down-projection dgrad)
    void* E_r;
    void* E_s;
    int c_stride2;         // output rows are 2 Nout wide (down-projection dgrad: da, db)
    // bf16 gate/up only, optional: routed row r of the token rows is row
    // gather_r[r] of A_r (the layer input x, src_token), not row r
    const int32_t* gather_r;
};

struct WorkV2 {
    int64_t m0, M, K, Nout, wt;
    int64_t rowbase;  // first row of the group in the token / output arrays
    int g;            // group: routed expert, or N for the shared expert
    const char* X;   // token rows of the group
    const char* W;   // weights of the group
    char* C;         // output rows of the group
    char* E;         // side array rows of the group (backward launches)
    const int32_t* gather;  // the group's source-row indices into X (nullptr: X rows in order)
};

// Units: routed (tile, wt) tile-major -- the weight tiles of one expert run
// next to each other and share its token rows in L2; shared (wt, tile)
// wt-major -- the token chunks of one weight panel run next to each other and
// share it.  Unit u runs on blockIdx (u % per) * 8 + u / per, per = ceil(units/8),
// so each XCD (blockIdx x, x+8, ...) gets a contiguous unit range.
// grid of a decode_v2 launch: 8 XCD slots x the most units one XCD can get
// (at most max_r routed and max_s shared tiles in all)
inline int64_t ffn_grid_blocks(int64_t max_r, int64_t ntn_r, int64_t max_s, int64_t ntn_s) {
    return 8 * cdiv(max_r + max_s, 8) * (ntn_r > ntn_s ? ntn_r : ntn_s);
}

template <int ESZ>
__device__ __forceinline__ bool decode_v2(const GemmParamsV2& p, int mode, WorkV2& w) {
    const int64_t nr = p.counts[0], ns = p.counts[1];
    // Tiles are dealt to the 8 XCDs (block L runs on XCD L % 8) in rounds of 8
    // along the sequence [shared tiles, routed tiles largest first], the
    // direction reversed every round: position q goes to XCD q % 8 or 7 - q % 8.
    // That evens out each XCD's work, and each XCD starts with its largest
    // tiles.  An XCD runs its tiles in order, the weight panels of one tile back
    // to back, so a tile's token rows are shared in that XCD's L2.
    const int64_t x = blockIdx.x % 8, i = blockIdx.x / 8;
    const int64_t rf = ns / 8, rem = ns % 8;
    const int64_t sx = rf + ((rf % 2 == 0) ? (x < rem) : (x >= 8 - rem));  // shared tiles here
    int64_t tile;
    if (i < sx * p.ntn_s) {
        const int64_t j = i / p.ntn_s;
        tile = nr + j * 8 + (j % 2 == 0 ? x : 7 - x);
        w.wt = i % p.ntn_s;
    } else {
        const int64_t i2 = i - sx * p.ntn_s;
        const int64_t j = sx + i2 / p.ntn_r;
        const int64_t k = j * 8 + (j % 2 == 0 ? x : 7 - x) - ns;
        if (k < 0 || k >= nr) return false;
        tile = p.order[k];
        w.wt = i2 % p.ntn_r;
    }
    const int2 t = p.tiles[tile];
    const int g = t.x;
    w.g = g;
    w.m0 = t.y;
    w.rowbase = 0;
    if (g < p.N) {
        const int64_t rowbase = p.offsets[g];
        w.rowbase = rowbase;
        w.M = p.offsets[g + 1] - rowbase;
        w.K = p.K_r;
        w.Nout = p.Nout_r;
        w.gather = p.gather_r ? p.gather_r + rowbase : nullptr;
        w.X = (const char*)p.A_r + (p.gather_r ? 0 : rowbase * w.K * ESZ);
        // weights of one expert: ntn_r packed tiles of G_WR_PACK rows (bf16,
        // FP8 codes) or the plain [rows][K] matrix (fp32)
        const int64_t wrows = ESZ != 4 ? (int64_t)p.ntn_r * G_WR_PACK
                                       : (mode == 0 ? 2 * w.Nout : w.Nout);
        w.W = (const char*)p.B_r + (int64_t)g * wrows * w.K * ESZ;
        w.C = (char*)p.C_r + rowbase * w.Nout * (p.c_stride2 ? 2 : 1) * ESZ;
        w.E = p.E_r ? (char*)p.E_r + rowbase * 2 * w.Nout * ESZ : nullptr;
    } else {
        w.M = p.T;
        w.K = p.K_s;
        w.Nout = p.Nout_s;
        w.gather = nullptr;
        w.X = (const char*)p.A_s;
        w.W = (const char*)p.B_s;
        w.C = (char*)p.C_s;
        w.E = (char*)p.E_s;
    }
    return true;
}

// silu(a) = a / (1 + e^-a), with the hardware reciprocal (1 ulp) instead of a
// division: it feeds bf16 / E4M3 outputs
__device__ __forceinline__ float silu_f(float a) { return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ lds_void* to_lds(const void* p) { return (lds_void*)p; }

// Workgroup barrier for LDS reuse: waits for this wave's LDS (and scalar)
// operations only.  __syncthreads also waits for the wave's global stores to
// complete (its fence covers global memory), which an epilogue that stores
// one part of a tile and then reuses the LDS for the next does not need.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Raw buffer descriptor over [base, base + bytes) (wave-uniform, in SGPRs):
// loads at offsets past the end return zero.  bytes must stay below 2^32.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t make_rsrc(const void* base, int64_t bytes) {
    const uint64_t a = (uint64_t)base;
    i32x4_t r;
    r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)) & 0xffff;  // stride 0
    r.z = __builtin_amdgcn_readfirstlane((int)(uint32_t)bytes);
    r.w = 0x00020000;  // raw 32-bit data format
    return r;
}

// Global -> LDS copy through a buffer descriptor: lane l copies SIZE (16 or 4)
// bytes from rsrc + voff + soff to LDS address lds + l*SIZE.  Written as
// inline asm on purpose: for the compiler's own LDS-DMA instructions its
// waitcnt pass makes every later LDS read wait for all copies in flight
// (vmcnt(0)), which would serialise the next stage's copies with the MFMAs of
// the current one.  The caller orders copies and reads itself (s_waitcnt
// vmcnt + barrier).  The compiler does not check hazards against the asm's
// operands, so the asm waits for them itself: s_nop 4 gives the 5 wait states
// a VMEM instruction needs after a VALU write of an SGPR it reads (the
// descriptor and offset SGPRs can come straight from v_readlane /
// v_readfirstlane), which also covers the 1 after an M0 write.
template <int SIZE>
__device__ __forceinline__ void dma_to_lds(i32x4_t rsrc, const void* lds, uint32_t voff,
                                           uint32_t soff) {
    const uint32_t m0 = (uint32_t)(uintptr_t)lds;
    if constexpr (SIZE == 16)
        asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc),
                     "s"(soff), "{m0}"(m0)
                     : "memory");
    else
        asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc),
                     "s"(soff), "{m0}"(m0)
                     : "memory");
}

// physical chunk of logical chunk c in row r of a 64-byte-row sub-tile (an
// involution).  A ds_read_b128 is served 16 lanes (256 bytes, the 64 banks)
// at a time; those lanes read one chunk of 16 consecutive rows, i.e. 4 rows
// for each of the 4 row positions within a 256-byte bank line, and the XOR
// with (r >> 2) & 3 gives those 4 rows 4 distinct chunk slots.
__device__ __forceinline__ int sub_chunk(int r, int c) { return c ^ ((r >> 2) & 3); }

// the same for 128-byte rows (8 chunks, two rows per 256-byte bank line):
// the 16 lanes reading one chunk of 16 consecutive rows get 16 distinct slots
__device__ __forceinline__ int sub_chunk8(int r, int c) { return c ^ ((r >> 1) & 7); }

template <int N>
__device__ __forceinline__ void vm_wait() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// s_waitcnt vmcnt(n) for a wave-uniform n in 0..23 (the counter field takes
// an immediate, hence the switch)
__device__ __forceinline__ void vm_wait_n(int n) {
    switch (n) {
#define MOE_VMW(i) \
    case i: vm_wait<i>(); break;
        MOE_VMW(0) MOE_VMW(1) MOE_VMW(2) MOE_VMW(3) MOE_VMW(4) MOE_VMW(5) MOE_VMW(6) MOE_VMW(7)
        MOE_VMW(8) MOE_VMW(9) MOE_VMW(10) MOE_VMW(11) MOE_VMW(12) MOE_VMW(13) MOE_VMW(14)
        MOE_VMW(15) MOE_VMW(16) MOE_VMW(17) MOE_VMW(18) MOE_VMW(19) MOE_VMW(20) MOE_VMW(21)
        MOE_VMW(22) MOE_VMW(23)
#undef MOE_VMW
        default: vm_wait<0>(); break;
    }
}

// weight row (of the [2*Nout or Nout][K] expert matrix) held in packed row r of
// weight tile wt; -1 for padding rows past the end (down projection only)
template <int MODE>
__device__ __forceinline__ int64_t packed_row_source(int64_t wt, int r, int64_t Nout) {
    if (MODE == 0) {
        const int g4 = r >> 6, half = (r >> 5) & 1, j = r & 31;
        return (half ? Nout : 0) + wt * 128 + g4 * 32 + j;
    }
    const int64_t wr = wt * 256 + r;
    return wr < Nout ? wr : -1;
}

}  // namespace moe
