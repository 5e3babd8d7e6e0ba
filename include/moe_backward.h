/*
 * moe_backward.h -- C ABI of libmoe, backward pass: the gradients of the layer
 * forward declared in moe.h, for bf16 and fp32 storage (gemm_dtype ==
 * act_dtype) and for FP8 expert GEMMs (moe_expert_ffn_backward_fp8 in place
 * of moe_expert_ffn_backward; the other three calls are the bf16 ones).
 *
 * The layer, from the DeepSeek-V3 report reading guide (xyznot.com/de),
 * "Methode", item 2:
 *   h'_t = u_t + FFN^(s)(u_t) + sum_j g_{t,j} FFN^(r)_{idx_j}(u_t)
 *   s_{i,t} = Sigmoid(u_t^T e_i),  g_{t,j} = s_{t,idx_j} / sum_j' s_{t,idx_j'}
 * with FFN read as SwiGLU without biases, W2 (silu(W1 u) * (W3 u)).  The
 * selection idx is piecewise constant and the balancing bias b_i only enters
 * the selection key, so neither has a gradient.  Given dout = dL/dh' the chain
 * rule splits into four calls, run in this order after a forward step whose
 * buffers (scores, idx, gate, offsets, src_token, dst_row, x_perm, y_perm)
 * are kept:
 * The forward's expert call may be moe_expert_ffn_train, which also keeps the
 * SwiGLU inputs a, b and its output h for the backward (else the backward
 * recomputes them).
 *   moe_combine_backward     dout -> routed-row gradients dy_perm and dgate
 *   moe_expert_ffn_backward  dy_perm, dout -> dx_perm, dx_shared and every
 *                            expert's weight gradients
 *   moe_route_backward       dgate -> logit gradients dz and the centroid
 *                            gradient
 *   moe_input_grad           dout + dx_shared + routed rows + dz e -> dx
 * The shared expert's output gradient and the residual's are dout itself.
 *
 * The common rules of moe.h hold: device pointers owned by the caller
 * (cfg on the host), dense row-major 16-byte-aligned tensors, asynchronous on
 * `stream`, no allocation, arguments validated before anything is enqueued,
 * MOE_OK or an error code with moe_last_error(), bitwise deterministic.
 * Accumulation is fp32; each output is rounded once to its dtype.
 */
#ifndef MOE_BACKWARD_H
#define MOE_BACKWARD_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Backward of moe_combine.  out[t] = x[t] + y_shared[t] + sum_j gate[t,j] y_perm[dst_row[t,j]]:
 *  dout    [T, d]    act_dtype  upstream gradient dL/dh'
 *  y_perm  [T*k, d]  act_dtype  the forward's routed expert outputs
 *  gate, dst_row [T, k]          the forward's gates and rows
 *  dy_perm [T*k, d]  act_dtype  out, dy_perm[dst_row[t,j]] = gate[t,j] * dout[t]
 *  dgate   [T, k]    fp32       out, dgate[t,j] = dout[t] . y_perm[dst_row[t,j]]
 * dy_perm must not alias dout or y_perm. */
int moe_combine_backward(const moe_cfg* cfg, const void* dout, const void* y_perm,
                         const float* gate, const int32_t* dst_row, void* dy_perm, float* dgate,
                         void* stream);

/* Bytes of the activations a training forward keeps: a, b and h of every
 * routed row and every shared-expert row, in act_dtype. */
size_t moe_expert_ffn_saved_size(const moe_cfg* cfg);

/* Training forward of the grouped SwiGLU experts: the same results as
 * moe_expert_ffn (bitwise), and it also stores into `saved`
 * (moe_expert_ffn_saved_size bytes, caller-owned, device) the activations
 * a = X W1^T and b = X W3^T (rounded to act_dtype) and h = silu(a) * b of
 * every row, for moe_expert_ffn_backward.  bf16 and fp32 layers only
 * (gemm_dtype == act_dtype); weights packed as for moe_expert_ffn; the other
 * arguments as there. */
int moe_expert_ffn_train(const moe_cfg* cfg, const void* x_perm, const int32_t* offsets,
                         const void* w13, const void* w2, void* y_perm, const void* x_sh,
                         const void* ws13, const void* ws2, void* y_shared, void* saved,
                         size_t saved_bytes, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Training forward of FP8 expert GEMMs: the same results as moe_expert_ffn
 * (bitwise; the arguments as there), and it also stores into `saved`
 * (moe_expert_ffn_saved_size bytes) a and b (the fp32 sums rounded to bf16)
 * and h = silu(a) * b in bf16 of every row, for moe_expert_ffn_backward_fp8.
 * gemm_dtype FP8_E4M3, act_dtype BF16. */
int moe_expert_ffn_train_fp8(const moe_cfg* cfg, const void* x_perm, const float* x_perm_scale,
                             const int32_t* offsets, const void* w13, const float* w13_scale,
                             const void* w2, const float* w2_scale, void* y_perm,
                             const void* x_sh, const float* x_sh_scale, const void* ws13,
                             const float* ws13_scale, const void* ws2, const float* ws2_scale,
                             void* y_shared, void* saved, size_t saved_bytes, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Bytes of workspace moe_expert_ffn_backward needs: the recomputed a, b, h and
 * the gradients da, db of every row (bf16 V3 shape: about 1.5 GB). */
size_t moe_expert_ffn_backward_workspace_size(const moe_cfg* cfg);

/* Backward of the grouped SwiGLU experts (routed experts over their rows of
 * x_perm, the shared expert over all T rows).  For one expert with rows X:
 *   a = X W1^T, b = X W3^T, h = silu(a) b   (read from `saved`, or recomputed)
 *   dh = dY W2;  da = dh b silu'(a), db = dh silu(a)   (stored in act_dtype)
 *   dX = da W1 + db W3;  dW2 = dY^T h;  dW1 = da^T X;  dW3 = db^T X
 * with silu'(a) = sig(a) (1 + a (1 - sig(a))).
 *  x_perm    [T*k, d]      the forward's routed rows
 *  offsets   [N+1]         the forward's expert row offsets
 *  w13       routed gate/up weights packed as for the forward (moe_pack_weights
 *            which = 0), used to recompute a, b, h; may be NULL with `saved`
 *  w13t      the same weights [N, 2I, d] packed transposed (which = 4), for dX
 *  w2t       routed down weights [N, d, I] packed transposed (which = 5), for dh
 *  dy_perm   [T*k, d]      from moe_combine_backward
 *  x_sh      [T, d]        shared-expert input x (NULL if inter_shared == 0)
 *  ws13, ws13t, ws2t       the shared expert's weights packed the same way
 *                          (which = 2, 6, 7)
 *  dy_shared [T, d]        gradient of the shared output: dout
 *  dx_perm   [T*k, d]      out, gradient of each routed row
 *  dx_shared [T, d]        out, gradient of x through the shared expert
 *  dw13 [N, 2I, d], dw2 [N, d, I], dws13 [2Is, d], dws2 [d, Is]
 *                          out, plain row-major like the weights; an expert
 *                          without rows gets zeros
 *  saved     the activations kept by moe_expert_ffn_train for this step
 *            (saved_bytes >= moe_expert_ffn_saved_size), or NULL: recompute
 * Activations and gradients in act_dtype.  fp32 layers: every packed form is
 * a plain copy.  bf16 needs hidden, inter, inter_shared % 128 == 0. */
int moe_expert_ffn_backward(const moe_cfg* cfg, const void* x_perm, const int32_t* offsets,
                            const void* w13, const void* w13t, const void* w2t,
                            const void* dy_perm, const void* x_sh, const void* ws13,
                            const void* ws13t, const void* ws2t, const void* dy_shared,
                            void* dx_perm, void* dx_shared, void* dw13, void* dw2, void* dws13,
                            void* dws2, const void* saved, size_t saved_bytes, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Bytes of workspace moe_expert_ffn_backward_fp8 needs (V3 shape: about 5 GB). */
size_t moe_expert_ffn_backward_fp8_workspace_size(const moe_cfg* cfg);

/* FP8 backward of the grouped SwiGLU experts (gemm_dtype FP8_E4M3, act_dtype
 * BF16).  Reading guide "Kernideen", FP8 bullet (E4M3 for all tensors, 1x128
 * activation tiles, 128x128 weight blocks, FP32 promotion every 128) applied
 * to every GEMM of the backward, each operand quantised along that GEMM's
 * contraction:
 *   a, b, h  as kept by moe_expert_ffn_train_fp8 (bf16), or recomputed on FP8
 *   dh = dY W2                    dY in 1x128 row tiles
 *   da, db as in moe_expert_ffn_backward (bf16), then [da db] in 1x128 tiles
 *   dX = [da db] [W1; W3]
 *   dW2 = dY^T h, dW13 = [da db]^T X   with dY, h, [da db] and X (the bf16
 *        layer input rows) quantised in 128x1 tiles down each expert's rows
 *        (blocks of 128 rows from the expert's first row, the last partial)
 *   every weight GEMM operand in the forward's 128x128 blocks (the same codes
 *   and scales; the gradient passes through the block quantisation)
 *  x [T, d] bf16 layer input; src_token [T*k], offsets [N+1]: the forward's
 *  x_perm, x_perm_scale   the forward's routed activation tiles (moe_permute)
 *  x_q, x_scale           the forward's shared-expert tiles (NULL if Is == 0)
 *  w13 / w13t             routed gate/up codes packed with which = 0 / 4 (the
 *                         forward's codes [N, 2I, d] in both cases)
 *  w13_scale              [N, 2I/128, d/128] the forward's block scales
 *  w2t, w2_scale          down codes packed with which = 5, [N, d/128, I/128]
 *  ws13, ws13t, ws13_scale, ws2t, ws2_scale   the shared expert's (2, 6, 7)
 *  dy_perm [T*k, d], dy_shared [T, d]  bf16 output gradients (dy_shared = dout)
 *  dx_perm, dx_shared     out, bf16, as moe_expert_ffn_backward
 *  dw13 [N, 2I, d], dw2 [N, d, I], dws13, dws2   out, bf16; zeros for an
 *                         expert without rows
 *  saved                  a, b, h kept by moe_expert_ffn_train_fp8 for this step
 *                         (saved_bytes >= moe_expert_ffn_saved_size), or NULL:
 *                         recomputed on FP8 (w13, ws13 are read only then)
 * Deterministic (no atomics); the common rules of moe.h hold. */
int moe_expert_ffn_backward_fp8(const moe_cfg* cfg, const void* x, const int32_t* src_token,
                                const int32_t* offsets, const uint8_t* x_perm,
                                const float* x_perm_scale, const uint8_t* x_q,
                                const float* x_scale, const void* w13, const void* w13t,
                                const float* w13_scale, const void* w2t, const float* w2_scale,
                                const void* ws13, const void* ws13t, const float* ws13_scale,
                                const void* ws2t, const float* ws2_scale, const void* dy_perm,
                                const void* dy_shared, void* dx_perm, void* dx_shared,
                                void* dw13, void* dw2, void* dws13, void* dws2, const void* saved,
                                size_t saved_bytes, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Bytes of workspace moe_route_backward needs (T*k fp32). */
size_t moe_route_backward_workspace_size(const moe_cfg* cfg);

/* Backward of the gates and the affinity.  With S the sum of the chosen s:
 *   dz[t,j] = (dgate[t,j] - sum_j' dgate[t,j'] s_j'/S) / S * s_j (1 - s_j),
 *   s_j = scores[t, idx[t,j]]  (S and the weighted sum in double, dz rounded to fp32)
 *   dcentroids[i] = sum over the rows r of expert i of dz[r] x[src_token[r]]
 *                   (fp32, rows in order; zero for experts nobody chose)
 *  x [T, d] act_dtype; scores [T, N] fp32 (the forward's, required here);
 *  idx, dgate, dst_row [T, k]; offsets [N+1]; src_token [T*k];
 *  dz [T, k] fp32 out; dcentroids [N, d] fp32 out. */
int moe_route_backward(const moe_cfg* cfg, const void* x, const float* scores,
                       const int32_t* idx, const float* dgate, const int32_t* offsets,
                       const int32_t* src_token, const int32_t* dst_row, float* dz,
                       float* dcentroids, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Gradient of the layer input:
 *   dx[t] = dout[t] + dx_shared[t] + sum_j (dx_perm[dst_row[t,j]] + dz[t,j] e_{idx[t,j]})
 * summed in fp32 in that order, rounded once to act_dtype.  dout may be NULL
 * (the forward had no residual), dx_shared NULL (no shared expert).
 * centroids [N, d] fp32; dx [T, d] out, must not alias an input. */
int moe_input_grad(const moe_cfg* cfg, const void* dout, const void* dx_shared,
                   const void* dx_perm, const int32_t* dst_row, const float* dz,
                   const int32_t* idx, const float* centroids, void* dx, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_BACKWARD_H */
