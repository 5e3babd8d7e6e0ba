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
