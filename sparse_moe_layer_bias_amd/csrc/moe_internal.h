// moe_internal.h -- launchers shared between the kernel files and the C ABI.
#pragma once

#include "moe_device.h"

namespace moe {

// sets the thread's moe_last_error() text (cleared for MOE_OK); returns code
int set_error(int code, const char* msg);

// ---------------------------------------------------------------- route
hipError_t launch_route(const moe_cfg& c, const void* x, const float* centroids,
                        const float* bias, float* scores, int32_t* idx, float* gate,
                        int32_t* counts, hipStream_t st);

// ---------------------------------------------------------------- permute
// tokens per block of the stable rank; workspace layout in permute.hip
constexpr int PERM_TB = 64;
size_t permute_workspace_bytes(const moe_cfg& c);
hipError_t launch_permute(const moe_cfg& c, const void* x, const int32_t* idx,
                          int32_t* offsets, int32_t* src_token, int32_t* dst_row, void* x_perm,
                          float* x_perm_scale, uint8_t* x_q, float* x_s, void* ws,
                          hipStream_t st);
// moe_permute_noalloc: its device-resident scratch (a file-scope array in
// permute.hip) and the address of the current device's copy
constexpr size_t PERM_SCRATCH_BYTES = (size_t)8 << 20;
hipError_t permute_scratch(void** ptr);

// ---------------------------------------------------------------- expert FFN
struct FfnArgs {
    const void* x_perm;
    const float* x_perm_scale;
    const int32_t* offsets;
    const void* w13;
    const float* w13_scale;
    const void* w2;
    const float* w2_scale;
    void* y_perm;
    const void* x_sh;
    const float* x_sh_scale;
    const void* ws13;
    const float* ws13_scale;
    const void* ws2;
    const float* ws2_scale;
    void* y_shared;
    // optional (bf16 inference forward): routed row r is x_perm[gather[r]] --
    // x_perm is then the layer input x and gather the permutation's src_token
    const int32_t* gather = nullptr;
};
size_t ffn_workspace_bytes(const moe_cfg& c);
// FP8 expert GEMM: contraction blocks of 128 per tile whose weight scales it
// stages in LDS, i.e. hidden, inter and inter_shared <= 128 * FP8_MAX_KB
constexpr int FP8_MAX_KB = 512;
// which: 0 = routed W13, 1 = routed W2, 2 = shared W13, 3 = shared W2
size_t packed_weight_bytes(const moe_cfg& c, int which);
hipError_t launch_pack_weights(const moe_cfg& c, int which, const void* w, void* out,
                               hipStream_t st);
size_t packed_weight_bytes_fp8(const moe_cfg& c, int which);
hipError_t launch_pack_weights_fp8(const moe_cfg& c, int which, const void* w, void* out,
                                   hipStream_t st);
// Activations a training forward keeps for the backward (act_dtype):
// ab [T*k][2I] (a, then b, of each routed row), h [T*k][I], and the same for
// the shared expert's T rows.
struct SavedActs {
    void* ab_r;
    void* h_r;
    void* ab_s;
    void* h_s;
};
size_t ffn_saved_bytes(const moe_cfg& c);
SavedActs carve_saved(const moe_cfg& c, void* saved);
// saved == nullptr: inference forward; else also store a, b and h there.
// hf_r / hf_s (FP8 layers, optional): the gate/up epilogue's fp32 h values
// before quantisation, [T*k][I] and [T][Is]
hipError_t launch_expert_ffn(const moe_cfg& c, const FfnArgs& a, void* ws, hipStream_t st,
                             void* saved = nullptr, float* hf_r = nullptr,
                             float* hf_s = nullptr);
// byte offsets inside the FFN workspace of h as the down GEMM reads it:
// routed h, shared h, routed tile scales, shared tile scales (FP8 only; the
// last two are SIZE_MAX for other layers)
void ffn_h_offsets(const moe_cfg& c, size_t off[4]);
// device tile list of the grouped GEMMs: routed expert g gets ceil(M_g / BM)
// tiles (group, first row), then the shared expert's ceil(T / BM); counts[0],
// counts[1] = their numbers; order = routed tiles by row count, largest first
void launch_tile_map(const int32_t* offsets, int N, int64_t T, bool has_shared, int BM,
                     int2* tiles, int32_t* counts, int32_t* order, int32_t* keys, hipStream_t st);

// ---------------------------------------------------------------- backward
// weights as moe_pack_weights lays them out: w13 / ws13 forward-packed
// (which 0 / 2), w13t / ws13t and w2t / ws2t transposed (which 4 / 6, 5 / 7)
struct FfnBwdArgs {
    const void* x_perm;
    const int32_t* offsets;
    const void* w13;
    const void* w13t;
    const void* w2t;
    const void* dy_perm;
    const void* x_sh;
    const void* ws13;
    const void* ws13t;
    const void* ws2t;
    const void* dy_sh;
    void* dx_perm;
    void* dx_sh;
    void* dw13;
    void* dw2;
    void* dws13;
    void* dws2;
};
size_t ffn_backward_workspace_bytes(const moe_cfg& c);
// recompute and both dgrad GEMMs on the forward's bf16 kernel (gemm.hip)
size_t ffn_bwd_tile_ws_bytes(const moe_cfg& c);
hipError_t launch_ffn_bwd_dgrad_bf16(const moe_cfg& c, const FfnBwdArgs& a, void* tile_ws,
                                     void* ab_r, void* ab_s, void* h_r, void* h_s, void* dab_r,
                                     void* dab_s, bool recompute, hipStream_t st);
// saved == nullptr: recompute a, b, h; else read them from a training forward
hipError_t launch_expert_ffn_backward(const moe_cfg& c, const FfnBwdArgs& a, void* ws,
                                      hipStream_t st, const void* saved = nullptr);
// fp32 layers: a, b and h of every row into `saved` (the training forward)
hipError_t launch_ffn_save_f32(const moe_cfg& c, const void* x_perm, const void* x_sh,
                               const int32_t* offsets, const void* w13, const void* ws13,
                               void* saved, hipStream_t st);
// One grouped FP8 GEMM launch on the forward's kernel (gemm_fp8.hip) over a
// tile list from launch_tile_map (row tile FP8_BM): mode 2 = gate/up with a,
// b and h kept in bf16 (C = h [rows][Nout], E = [a | b] [rows][2 Nout]),
// mode 1 = plain rows with a bf16 output C [rows][Nout].  A: codes [rows][K]
// with 1x128 scales as [rows][K/128]; B: packed weight codes; bs: block
// scales, bs_t = 1 when indexed [mat][K/128][Nout/128].
struct Fp8Gemm {
    int mode;
    int64_t K_r, K_s, Nout_r, Nout_s;
    const void* A_r;
    const void* A_s;
    const float* as_r;
    const float* as_s;
    const void* B_r;
    const void* B_s;
    const float* bs_r;
    const float* bs_s;
    int bs_t;
    void* C_r;
    void* C_s;
    void* E_r;
    void* E_s;
};
hipError_t launch_fp8_gemm(const Fp8Gemm& op, const int2* tiles, const int32_t* counts,
                           const int32_t* order, const int32_t* offsets, int N, int64_t T_shared,
                           int64_t max_r, int64_t max_s, hipStream_t st);
constexpr int FP8_BM = 320;  // FP8 GEMM row tile

// FP8 backward of the experts (backward_fp8.hip)
struct FfnBwdFp8Args {
    const void* x;             // [T][d] bf16 layer input
    const int32_t* src_token;  // [T*k]
    const int32_t* offsets;    // [N+1]
    const void* x_perm_q;      // forward's routed activation tiles: codes, scales
    const float* x_perm_s;
    const void* x_q;           // forward's shared-expert activation tiles
    const float* x_s;
    const void* w13;           // packed which 0 / 4, scales [N][2I/128][d/128]
    const void* w13t;
    const float* w13_s;
    const void* w2t;           // packed which 5, scales [N][d/128][I/128]
    const float* w2_s;
    const void* ws13;          // shared: which 2 / 6 / 7
    const void* ws13t;
    const float* ws13_s;
    const void* ws2t;
    const float* ws2_s;
    const void* dy_perm;
    const void* dy_sh;
    void* dx_perm;
    void* dx_sh;
    void* dw13;
    void* dw2;
    void* dws13;
    void* dws2;
};
size_t ffn_backward_fp8_workspace_bytes(const moe_cfg& c);
// byte offsets of the FP8 backward's intermediates in its workspace, in the
// order of the MOE_BWD8_* indices of moe_inspect.h
void ffn_backward_fp8_offsets(const moe_cfg& c, size_t off[25]);
// saved: the a, b, h a training forward kept (carve_saved), else recomputed
hipError_t launch_expert_ffn_backward_fp8(const moe_cfg& c, const FfnBwdFp8Args& a, void* ws,
                                          hipStream_t st, const void* saved = nullptr);
hipError_t launch_combine_backward(const moe_cfg& c, const void* dout, const void* y_perm,
                                   const float* gate, const int32_t* dst_row, void* dy_perm,
                                   float* dgate, hipStream_t st);
hipError_t launch_route_backward(const moe_cfg& c, const void* x, const float* scores,
                                 const int32_t* idx, const float* dgate, const int32_t* offsets,
                                 const int32_t* src_token, const int32_t* dst_row, float* dz,
                                 float* dz_perm, float* dcentroids, hipStream_t st);
hipError_t launch_input_grad(const moe_cfg& c, const void* dout, const void* dx_shared,
                             const void* dx_perm, const int32_t* dst_row, const float* dz,
                             const int32_t* idx, const float* centroids, void* dx,
                             hipStream_t st);

// ---------------------------------------------------------------- combine / bias / prep
hipError_t launch_combine(const moe_cfg& c, const void* x, const void* y_shared,
                          const void* y_perm, const float* gate, const int32_t* dst_row,
                          void* out, hipStream_t st);
hipError_t launch_bias_update(int64_t N, int64_t TK, const int32_t* counts, float gamma,
                              float* bias, hipStream_t st);
size_t seq_balance_workspace_bytes(int64_t T, int64_t N, int64_t S);
hipError_t launch_seq_balance_loss(int64_t T, int64_t N, int64_t k, int64_t S, float alpha,
                                   const float* scores, const int32_t* idx, float* loss,
                                   void* ws, hipStream_t st);
hipError_t launch_quantize_weights(int64_t n_mats, int64_t rows, int64_t cols, const void* w,
                                   uint8_t* q, float* s, hipStream_t st);
hipError_t launch_e4m3_inspect(const float* v, int64_t n, float scale, uint8_t* c4, uint8_t* c1,
                               hipStream_t st);

}  // namespace moe
