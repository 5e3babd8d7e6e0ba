/*
 * moe_inspect.h -- intermediate values of the expert FFN, for checks of the
 * quantisation steps against an independent implementation.  They are not a
 * second way to run the layer: moe_expert_ffn_inspect computes exactly what
 * moe_expert_ffn computes (bitwise), and also writes one intermediate.
 *
 * Common rules as in moe.h: device pointers owned by the caller (cfg and
 * `off` are host pointers), asynchronous on `stream`, MOE_OK or an error code
 * with moe_last_error(); arguments are validated before anything is enqueued.
 */
#ifndef MOE_INSPECT_H
#define MOE_INSPECT_H

#include <stddef.h>
#include <stdint.h>

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Where moe_expert_ffn keeps the intermediate h = silu(W1 u) * (W3 u) inside
 * its workspace, as the down GEMM reads it (DeepSeek-V3 reading guide,
 * "Kernideen", FP8 bullet: h is an activation like any other, so FP8 layers
 * hold it as 1x128-tile E4M3 codes and fp32 tile scales).  Byte offsets from
 * the workspace start:
 *  off[0]  routed h   [T*k, I]     act_dtype, or E4M3 codes for FP8 layers
 *  off[1]  shared h   [T, Is]      same element type
 *  off[2]  routed tile scales [T*k, I/128]  fp32 (FP8 layers; else SIZE_MAX)
 *  off[3]  shared tile scales [T, Is/128]   fp32 (FP8 layers; else SIZE_MAX)
 * Valid after a moe_expert_ffn (or moe_expert_ffn_inspect) call on that
 * workspace, until the workspace is reused.  Returns MOE_OK or MOE_ERR_ARG. */
int moe_expert_ffn_h_offsets(const moe_cfg* cfg, size_t off[4]);

/* moe_expert_ffn of an FP8 layer (gemm_dtype == MOE_FP8_E4M3), same arguments
 * and the same results bit for bit, that also writes the fp32 values of
 * h = silu(a) * b that the gate/up GEMM's epilogue quantises per 1x128 tile
 * (before that quantisation):
 *  h_f32         [T*k, I]  fp32 out, routed rows in x_perm's row order
 *  h_f32_shared  [T, Is]   fp32 out; NULL when Is == 0
 * Other layers: MOE_ERR_UNSUPPORTED. */
int moe_expert_ffn_inspect(const moe_cfg* cfg, const void* x_perm, const float* x_perm_scale,
                           const int32_t* offsets, const void* w13, const float* w13_scale,
                           const void* w2, const float* w2_scale, void* y_perm, const void* x_sh,
                           const float* x_sh_scale, const void* ws13, const float* ws13_scale,
                           const void* ws2, const float* ws2_scale, void* y_shared,
                           float* h_f32, float* h_f32_shared, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Where moe_expert_ffn_backward_fp8 keeps its intermediates inside its
 * workspace (reading guide "Kernideen", FP8 bullet: every operand of every
 * backward GEMM is E4M3 in tiles along that GEMM's contraction), byte offsets
 * from the workspace start, for checks of each step against an independent
 * implementation.  Valid after a call on that workspace until it is reused.
 * R = T*k routed rows (x_perm order), S = T shared rows (0 without a shared
 * expert), Ir = I, Is = inter_shared, Im = max(I, Is):
 *  DY_Q  [R, d] u8,  DY_S  [R, d/128] fp32    dY (dy_perm) in 1x128 row tiles
 *  DH    [R, I] bf16                          dh = dY W2
 *  DAB   [R, 2I] bf16                         [da | db]
 *  DAB_Q [R, 2I] u8, DAB_S [R, 2I/128] fp32   [da db] in 1x128 row tiles
 *  the same four for the shared expert's S rows (_SH), with Is for I
 *  COL_*    [P/128][F][128] u8, COL_*_S [P/128][F] fp32: the 128x1 row-direction
 *           tiles of dY (F = d), h (F = Im), [da db] (F = 2 Im) and x gathered
 *           through src_token (F = d); 128-row block pb of group g (routed
 *           experts 0..N-1, then the shared expert) is POFF[g]/128 + its
 *           block index in the group, codes [pb][feature][row % 128]
 *  POFF  [N+2] int32: prefix of the groups' row counts, each rounded up to 128
 *  AB [R, 2I], H [R, I], AB_SH, H_SH bf16: a, b, h when the call recomputes
 *           them (with saved activations they are in the saved buffer at the
 *           offsets of moe_expert_ffn_saved_offsets)
 * Returns MOE_OK, or MOE_ERR_ARG / MOE_ERR_UNSUPPORTED for a bad cfg. */
#define MOE_BWD8_DY_Q 0
#define MOE_BWD8_DY_S 1
#define MOE_BWD8_DY_Q_SH 2
#define MOE_BWD8_DY_S_SH 3
#define MOE_BWD8_DH 4
#define MOE_BWD8_DH_SH 5
#define MOE_BWD8_DAB 6
#define MOE_BWD8_DAB_SH 7
#define MOE_BWD8_DAB_Q 8
#define MOE_BWD8_DAB_S 9
#define MOE_BWD8_DAB_Q_SH 10
#define MOE_BWD8_DAB_S_SH 11
#define MOE_BWD8_COL_DY 12
#define MOE_BWD8_COL_DY_S 13
#define MOE_BWD8_COL_H 14
#define MOE_BWD8_COL_H_S 15
#define MOE_BWD8_COL_DAB 16
#define MOE_BWD8_COL_DAB_S 17
#define MOE_BWD8_COL_X 18
#define MOE_BWD8_COL_X_S 19
#define MOE_BWD8_POFF 20
#define MOE_BWD8_AB 21
#define MOE_BWD8_H 22
#define MOE_BWD8_AB_SH 23
#define MOE_BWD8_H_SH 24
#define MOE_BWD8_N 25
int moe_expert_ffn_backward_fp8_offsets(const moe_cfg* cfg, size_t off[MOE_BWD8_N]);

/* Byte offsets inside the saved-activation buffer of a training forward
 * (moe_expert_ffn_train / moe_expert_ffn_train_fp8): off[0] routed [a | b]
 * [T*k, 2I], off[1] routed h [T*k, I], off[2] shared [a | b] [T, 2Is],
 * off[3] shared h [T, Is], all in act_dtype.  Returns MOE_OK or MOE_ERR_ARG. */
int moe_expert_ffn_saved_offsets(const moe_cfg* cfg, size_t off[4]);

/* The E4M3 quantisation step the kernels apply, on given fp32 values
 * (reading guide "Kernideen", FP8 bullet; the singularity-lens summary's
 * formula paragraph: code = E4M3(clip(v / S, -448, 448)), nearest, ties to
 * even; S = 0 gives code 0), both ways the kernels perform it:
 *  codes4 [n] u8 out: as the FP8 gate/up epilogue quantises h (IEEE fp32
 *                     quotient, clamp, four values per converter pair)
 *  codes1 [n] u8 out: as the activation and weight quantisers do (one value
 *                     per converter instruction)
 *  v      [n] fp32; scale: the tile scale S (>= 0, finite); n >= 0.
 * Returns MOE_OK, MOE_ERR_ARG, or MOE_ERR_HIP. */
int moe_inspect_e4m3(const float* v, int64_t n, float scale, uint8_t* codes4, uint8_t* codes1,
                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_INSPECT_H */
