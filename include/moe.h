/*
 * moe.h -- C ABI of libmoe: the forward pass of one DeepSeekMoE feed-forward
 * layer with auxiliary-loss-free bias balancing, on one AMD Instinct MI355X
 * (gfx950).
 *
 * The layer, as the DeepSeek-V3 report reading guide (xyznot.com/de) states it
 * in "Methode", item 2 "DeepSeekMoE mit Auxiliary-Loss-Free Balancing":
 *
 *   h'_t = u_t + sum_{i<=N_s} FFN^(s)_i(u_t) + sum_{i<=N_r} g_{i,t} FFN^(r)_i(u_t)
 *   s_{i,t} = Sigmoid(u_t^T e_i)
 *   g'_{i,t} = s_{i,t} if s_{i,t} + b_i is among the K_r largest of {s_{j,t} + b_j}, else 0
 *   g_{i,t} = g'_{i,t} normalised over the chosen experts
 *   end of step: overloaded expert b_i -= gamma, underloaded b_i += gamma, gamma = 0.001
 *
 * One call per step of that statement:
 *   moe_route        affinity, biased (group-limited) top-k, gates, per-expert load
 *   moe_permute      stable sort of the (token, slot) pairs by expert; row gather
 *   moe_expert_ffn   grouped SwiGLU expert GEMMs, routed experts + the shared expert
 *   moe_combine      u_t + shared output + gate-weighted routed outputs
 *   moe_bias_update  the end-of-step bias rule
 *
 * Common rules for every call:
 *  - Every pointer argument is a DEVICE pointer owned by the caller, except
 *    `cfg`, which is a host pointer read during the call only.  The library
 *    allocates no memory and keeps no state between calls (it is thread-safe);
 *    the one exception is moe_permute_noalloc's built-in per-GPU scratch.
 *  - Tensors are dense, row-major, contiguous, 16-byte aligned.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue work; they never synchronise the host.  Counts and offsets stay
 *    on the device.
 *  - Return value: MOE_OK, or an error code; moe_last_error() then returns a
 *    message (per calling thread).  Arguments are validated before anything
 *    is enqueued; a rejected call enqueues nothing.  Faults inside kernels
 *    surface at the caller's next synchronisation.
 *  - Inputs must be finite.  Results are bitwise deterministic run to run.
 *
 * Precision readings (where the pages are silent):
 *  - logits are the fixed-order fp32 chain acc = fma(x[t,j], e[i,j], acc) over
 *    j ascending from +0; the sigmoid is evaluated in double and rounded once;
 *  - the Topk order is (s+b descending, expert index ascending); -0 == +0;
 *  - group limit (n_group > 1): contiguous groups of N/n_group experts; group
 *    score = fp32 sum of the group's two largest biased keys; keep the
 *    topk_group best groups (ties to the lower group index);
 *  - gates g_j = s_j / (sum of chosen s, in double), no further scaling;
 *  - FFN_i is SwiGLU without biases: W2 (silu(W1 u) * (W3 u)).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MOE_OK 0
#define MOE_ERR_ARG 1         /* null / misaligned pointer, or a bad shape     */
#define MOE_ERR_UNSUPPORTED 2 /* a dtype / shape combination not implemented */
#define MOE_ERR_WORKSPACE 3   /* workspace smaller than the *_workspace_size  */
#define MOE_ERR_HIP 4         /* a HIP launch failed                          */

/* element types */
#define MOE_F32 0
#define MOE_BF16 1
#define MOE_FP8_E4M3 2 /* OCP E4M3FN, largest finite 448 */

/* Shapes and types of one layer. */
typedef struct moe_cfg {
    int64_t tokens;       /* T: tokens in the batch                              */
    int64_t hidden;       /* d: model width                                      */
    int64_t n_experts;    /* N: routed experts, 1..1024                          */
    int64_t top_k;        /* k: experts per token, 1..min(N, 64)                 */
    int64_t n_group;      /* G: 1 = no group limit, else N % G == 0, N/G >= 2   */
    int64_t topk_group;   /* TG: groups kept per token (ignored when G == 1)     */
    int64_t inter;        /* I: routed expert intermediate width                 */
    int64_t inter_shared; /* Is: shared expert intermediate width, 0 = none      */
    int32_t act_dtype;    /* MOE_F32 or MOE_BF16: x, weights, expert outputs, out */
    int32_t gemm_dtype;   /* == act_dtype, or MOE_FP8_E4M3 (needs act_dtype BF16,
                             hidden % 128 == 0, inter % 128 == 0, Is % 128 == 0) */
} moe_cfg;

/* ------------------------------------------------------------------ route */

/* Bytes of workspace moe_route needs when `scores` is NULL (0 otherwise). */
size_t moe_route_workspace_size(const moe_cfg* cfg);

/* Affinity, biased selection and gates ("Methode" item 2: s_{i,t}, g'_{i,t},
 * g_{i,t}) plus the step's per-expert load.
 *  x          [T, d]   act_dtype   token hidden states u_t
 *  centroids  [N, d]   fp32        expert centroids e_i
 *  bias       [N]      fp32        routing bias b_i (read only)
 *  scores     [T, N]   fp32        out, s_{i,t}; may be NULL (then workspace used)
 *  idx        [T, k]   int32       out, chosen experts in selection order
 *  gate       [T, k]   fp32        out, g for each chosen expert
 *  counts     [N]      int32       out, number of (token, slot) pairs per expert
 */
int moe_route(const moe_cfg* cfg, const void* x, const float* centroids, const float* bias,
              float* scores, int32_t* idx, float* gate, int32_t* counts, void* workspace,
              size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- permute */

size_t moe_permute_workspace_size(const moe_cfg* cfg);

/* Stable counting sort of the T*k (token, slot) pairs by expert, the dispatch
 * that feeds each expert its tokens (the pages only show it as the cross-node
 * all-to-all).  Row numbering: expert-major, tokens ascending inside an expert.
 *  x            [T, d]        act_dtype  token hidden states
 *  idx          [T, k]        int32      from moe_route
 *  offsets      [N+1]         int32      out, first row of each expert; offsets[N] = T*k
 *  src_token    [T*k]         int32      out, token of each row
 *  dst_row      [T, k]        int32      out, row of each (token, slot)
 *  x_perm       [T*k, d]      out: act_dtype rows (gemm_dtype != FP8) or
 *                             E4M3 codes (gemm_dtype == FP8).  May be NULL
 *                             (FP8: with x_perm_scale): then the rows are not
 *                             copied, only offsets, src_token, dst_row (and
 *                             for FP8 x_q, x_s) are written, for
 *                             moe_expert_ffn_gather, which reads the rows
 *                             through src_token itself
 *  x_perm_scale [T*k, d/128]  fp32 out, FP8 tile scales (FP8 only, else NULL)
 *  x_q          [T, d]        u8   out, FP8 codes of x for the shared expert (FP8 only)
 *  x_s          [T, d/128]    fp32 out, their tile scales (FP8 only)
 * FP8 quantisation (reading guide "Kernideen", FP8 bullet; singularity-lens
 * formula paragraph): per 1x128 tile along d, scale = amax/448 (fp32 divide),
 * code = E4M3(clamp(v/scale, -448, 448)) rounded to nearest-even; an all-zero
 * tile gets scale 0 and codes 0.
 */
int moe_permute(const moe_cfg* cfg, const void* x, const int32_t* idx, int32_t* offsets,
                int32_t* src_token, int32_t* dst_row, void* x_perm, float* x_perm_scale,
                uint8_t* x_q, float* x_s, void* workspace, size_t workspace_bytes,
                void* stream);

/* moe_permute for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments without the workspace, the same results bit for bit.
 * Its scratch (the per-(token, slot) ranks and per-64-token-block histograms
 * moe_permute keeps in the workspace) is a device-resident array built into
 * the library, one per GPU, held until the process ends; the call allocates
 * nothing.  Limit: moe_permute_workspace_size(cfg) <= moe_permute_noalloc_max_bytes()
 * (8 MiB: at N = 256 about 170k tokens of top-8), else MOE_ERR_WORKSPACE
 * and nothing is enqueued.  Every call on one GPU uses that GPU's array:
 * calls that overlap on one GPU (concurrent streams, or threads) race; calls
 * on one stream are ordered and safe.  Errors as moe_permute, plus MOE_ERR_HIP
 * if the array's device address cannot be obtained. */
size_t moe_permute_noalloc_max_bytes(void);
int moe_permute_noalloc(const moe_cfg* cfg, const void* x, const int32_t* idx, int32_t* offsets,
                        int32_t* src_token, int32_t* dst_row, void* x_perm, float* x_perm_scale,
                        uint8_t* x_q, float* x_s, void* stream);

/* ------------------------------------------------------------- expert FFN */

size_t moe_expert_ffn_workspace_size(const moe_cfg* cfg);

/* Grouped SwiGLU expert FFNs for every routed expert over its rows of x_perm,
 * and the shared expert over all T rows of x, in the same launches
 * ("Methode" item 2: FFN^(r)_i and FFN^(s)).
 *  x_perm      [T*k, d]   routed rows (act_dtype, or E4M3 codes for FP8)
 *  x_perm_scale[T*k, d/128] FP8 tile scales (FP8 only, else NULL)
 *  offsets     [N+1]      from moe_permute (device)
 *  w13         routed gate/up weights, PACKED by moe_pack_weights(which = 0) from
 *              [N, 2I, d] (per expert rows 0..I-1 = W1 (gate), I..2I-1 = W3 (up))
 *  w13_scale   [N, 2I/128, d/128]  FP8 block scales (FP8 only)
 *  w2          routed down weights, PACKED (which = 1) from [N, d, I]
 *  w2_scale    [N, d/128, I/128]   FP8 block scales (FP8 only)
 *  y_perm      [T*k, d]   act_dtype out, expert output per row (unweighted)
 *  x_sh        [T, d]     shared-expert input: x (act_dtype) or x_q (FP8); NULL if Is == 0
 *  x_sh_scale  [T, d/128] FP8 only
 *  ws13        shared gate/up, PACKED (which = 2) from [2Is, d]; ws13_scale (FP8)
 *  ws2         shared down, PACKED (which = 3) from [d, Is]; ws2_scale (FP8)
 *  y_shared    [T, d]     act_dtype out (NULL if Is == 0)
 * Accumulation is fp32.  bf16: h = silu(a)*b is rounded to bf16 between the
 * two GEMMs.  FP8 ("Kernideen": promotion every N_c = 128): each 128-wide
 * K block's partial sum is scaled by act_scale*weight_scale and added to an
 * fp32 accumulator; h is re-quantised per 1x128 tile before the down GEMM.
 */
int moe_expert_ffn(const moe_cfg* cfg, const void* x_perm, const float* x_perm_scale,
                   const int32_t* offsets, const void* w13, const float* w13_scale,
                   const void* w2, const float* w2_scale, void* y_perm, const void* x_sh,
                   const float* x_sh_scale, const void* ws13, const float* ws13_scale,
                   const void* ws2, const float* ws2_scale, void* y_shared, void* workspace,
                   size_t workspace_bytes, void* stream);

/* moe_expert_ffn without the permuted copy of the tokens, for bf16 layers and
 * FP8 layers (act_dtype bf16): routed row r is row src_token[r] of x, read by
 * the gate/up GEMM's own copies ("Methode" item 2: each routed expert sees
 * the tokens that chose it; the dispatch is the same permutation, its rows
 * are not materialised).  The shared expert reads the same x.  Results are
 * those of moe_expert_ffn on the x_perm (x_perm_scale) that moe_permute would
 * have written, bit for bit.
 *  x          [T, d]     bf16 layer input, or for FP8 layers its E4M3 codes
 *                        x_q from moe_permute
 *  x_scale    [T, d/128] FP8: the tile scales x_s from moe_permute; else NULL
 *  src_token  [T*k]      int32 from moe_permute (which may skip x_perm for this)
 *  the weights, scales and outputs as moe_expert_ffn.
 * Requires x (T * d elements) below 2^32 bytes (32-bit row offsets), else
 * MOE_ERR_UNSUPPORTED; fp32 layers: MOE_ERR_UNSUPPORTED. */
int moe_expert_ffn_gather(const moe_cfg* cfg, const void* x, const float* x_scale,
                          const int32_t* src_token, const int32_t* offsets, const void* w13,
                          const float* w13_scale, const void* w2, const float* w2_scale,
                          void* y_perm, const void* ws13, const float* ws13_scale,
                          const void* ws2, const float* ws2_scale, void* y_shared,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Weight preparation, off the per-step path (weights are constant across
 * steps).  Rearranges one weight stack into the order the expert GEMM streams
 * it: tiles of 256 output rows, 32-wide contraction blocks, 16-byte chunks in
 * the kernel's shared-memory order, so each pipeline stage reads one
 * contiguous block.  Gate/up tiles interleave 32 W1 rows with the matching 32
 * W3 rows.  fp32 layers keep the plain layout (a copy).
 *  which: 0 = routed W13 [N, 2I, d], 1 = routed W2 [N, d, I],
 *         2 = shared W13 [2Is, d],   3 = shared W2 [d, Is];
 *         for the backward (moe_expert_ffn_backward, and for FP8 layers
 *         moe_expert_ffn_backward_fp8), the same stacks transposed:
 *         4 = routed W13, 5 = routed W2, 6 = shared W13, 7 = shared W2
 *         (tiles of 256 columns of the stored matrix)
 *  w: act_dtype, row-major (FP8 layers: the E4M3 codes from
 *     moe_quantize_weights_fp8, same shape; their scales are passed to
 *     moe_expert_ffn unchanged); w_packed: moe_packed_weights_size(cfg, which) bytes. */
size_t moe_packed_weights_size(const moe_cfg* cfg, int which);
int moe_pack_weights(const moe_cfg* cfg, int which, const void* w, void* w_packed, void* stream);

/* ---------------------------------------------------------------- combine */

/* h'_t = u_t + y_shared[t] + sum_j gate[t,j] * y_perm[dst_row[t,j]]
 * ("Methode" item 2), summed in fp32, rounded once to act_dtype.
 *  x_residual [T, d] act_dtype or NULL (no residual term)
 *  y_shared   [T, d] act_dtype or NULL (no shared expert)
 *  y_perm     [T*k, d], gate [T, k], dst_row [T, k]
 *  out        [T, d] act_dtype out (must not alias the inputs)
 */
int moe_combine(const moe_cfg* cfg, const void* x_residual, const void* y_shared,
                const void* y_perm, const float* gate, const int32_t* dst_row, void* out,
                void* stream);

/* ------------------------------------------------------------ bias update */

/* End-of-step rule ("Methode" item 2; the singularity-lens formula paragraph
 * writes it b_i += gamma * sign(mean_load - load_i)): with mean load
 * tokens_times_k / n_experts, expert i is overloaded when
 * counts[i] * n_experts > tokens_times_k (compared exactly in integers):
 * bias[i] -= gamma; underloaded (<): bias[i] += gamma; equal: unchanged.
 * fp32 arithmetic.  counts [N] int32, bias [N] fp32 in/out. */
int moe_bias_update(int64_t n_experts, int64_t tokens_times_k, const int32_t* counts,
                    float gamma, float* bias, void* stream);

/* -------------------------------------------------- sequence-wise balance loss */

/* The minimal sequence-wise balance loss (alpha = 0.0001) that the reading
 * guide's "Methode" item 2 names, in its last sentence, as a complement to
 * the bias rule, evaluated as a forward statistic.  The pages print no
 * formula; the reading taken: the batch is tokens / seq_len sequences of
 * seq_len consecutive tokens, and for sequence b
 *   loss[b] = alpha * sum_i f_i P_i,
 *   f_i = N / (top_k seq_len) * (number of the sequence's idx entries == i),
 *   P_i = (1 / seq_len) * sum_t scores[t][i] / sum_j scores[t][j].
 * scores [T, N] fp32: the affinities s_{i,t} (moe_route's scores output);
 * idx [T, top_k] int32 from moe_route (entries outside 0..N-1 are not
 * counted); loss [T / seq_len] fp32 out.  Sums in double in a fixed order,
 * one rounding to fp32, the same bits on every run.  Uses tokens, n_experts
 * and top_k of cfg.  Errors: MOE_ERR_ARG when seq_len < 1, tokens is not a
 * multiple of seq_len or alpha is NaN; MOE_ERR_WORKSPACE when workspace_bytes
 * is below moe_seq_balance_loss_workspace_size(cfg, seq_len). */
size_t moe_seq_balance_loss_workspace_size(const moe_cfg* cfg, int64_t seq_len);
int moe_seq_balance_loss(const moe_cfg* cfg, int64_t seq_len, float alpha, const float* scores,
                         const int32_t* idx, float* loss, void* workspace,
                         size_t workspace_bytes, void* stream);

/* ----------------------------------------------------------- preparation */

/* Off the per-step path: 128x128 block quantisation of n_mats bf16 matrices
 * of rows x cols (both % 128 == 0) to E4M3 codes (same layout) and scales
 * [n_mats, rows/128, cols/128] (reading guide "Kernideen", FP8 bullet;
 * scale = amax/448 per block, as for activations). */
int moe_quantize_weights_fp8(int64_t n_mats, int64_t rows, int64_t cols, const void* w_bf16,
                             uint8_t* w_q, float* w_scale, void* stream);

/* Message of the last failed call on this thread ("" if none). */
const char* moe_last_error(void);

/* ABI version, bumped on any signature change. */
int moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
