// capi.cpp -- the C ABI of libmoe (include/moe.h): argument validation, error
// reporting and dispatch to the kernel launchers.  Validation runs on the host
// before anything is enqueued, so a rejected call has no effect on the device.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "moe_backward.h"
#include "moe_inspect.h"
#include "moe_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = 0;
    return MOE_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define REQ_PTR(p)                                                                   \
    do {                                                                             \
        if (!(p)) return fail(MOE_ERR_ARG, "%s: %s is NULL", fn, #p);                \
        if (!aligned16(p)) return fail(MOE_ERR_ARG, "%s: %s is not 16-byte aligned", \
                                       fn, #p);                                      \
    } while (0)

#define OPT_PTR(p)                                                                   \
    do {                                                                             \
        if ((p) && !aligned16(p))                                                    \
            return fail(MOE_ERR_ARG, "%s: %s is not 16-byte aligned", fn, #p);       \
    } while (0)

int check_cfg(const char* fn, const moe_cfg* c) {
    if (!c) return fail(MOE_ERR_ARG, "%s: cfg is NULL", fn);
    if (c->tokens < 0 || c->tokens > (int64_t)1 << 26)
        return fail(MOE_ERR_ARG, "%s: tokens=%lld out of range", fn, (long long)c->tokens);
    if (c->hidden <= 0) return fail(MOE_ERR_ARG, "%s: hidden must be > 0", fn);
    if (c->n_experts < 1 || c->n_experts > 1024)
        return fail(MOE_ERR_ARG, "%s: n_experts=%lld must be in 1..1024", fn,
                    (long long)c->n_experts);
    if (c->top_k < 1 || c->top_k > c->n_experts || c->top_k > 64)
        return fail(MOE_ERR_ARG, "%s: top_k=%lld must be in 1..min(n_experts, 64)", fn,
                    (long long)c->top_k);
    if (c->n_group < 1) return fail(MOE_ERR_ARG, "%s: n_group must be >= 1", fn);
    if (c->n_group > 1) {
        if (c->n_group > 64 || c->n_experts % c->n_group)
            return fail(MOE_ERR_ARG, "%s: n_group must divide n_experts and be <= 64", fn);
        if (c->n_experts / c->n_group < 2)
            return fail(MOE_ERR_ARG, "%s: groups need at least 2 experts", fn);
        if (c->topk_group < 1 || c->topk_group > c->n_group)
            return fail(MOE_ERR_ARG, "%s: topk_group must be in 1..n_group", fn);
        if (c->top_k > c->topk_group * (c->n_experts / c->n_group))
            return fail(MOE_ERR_ARG, "%s: top_k exceeds the experts of the kept groups", fn);
    }
    if (c->act_dtype != MOE_F32 && c->act_dtype != MOE_BF16)
        return fail(MOE_ERR_UNSUPPORTED, "%s: act_dtype must be MOE_F32 or MOE_BF16", fn);
    if (c->gemm_dtype != c->act_dtype && c->gemm_dtype != MOE_FP8_E4M3)
        return fail(MOE_ERR_UNSUPPORTED, "%s: gemm_dtype must equal act_dtype or be FP8", fn);
    if (c->gemm_dtype == MOE_FP8_E4M3 && c->act_dtype != MOE_BF16)
        return fail(MOE_ERR_UNSUPPORTED, "%s: FP8 expert GEMMs need bf16 activations", fn);
    if (c->act_dtype == MOE_BF16 && c->hidden % 8)
        return fail(MOE_ERR_UNSUPPORTED, "%s: bf16 needs hidden %% 8 == 0", fn);
    if (c->act_dtype == MOE_F32 && c->hidden % 4)
        return fail(MOE_ERR_UNSUPPORTED, "%s: fp32 needs hidden %% 4 == 0", fn);
    if ((int64_t)c->tokens * c->top_k > INT32_MAX)
        return fail(MOE_ERR_ARG, "%s: tokens*top_k exceeds int32 row indices", fn);
    return MOE_OK;
}

int check_ffn_shape(const char* fn, const moe_cfg* c) {
    if (c->inter <= 0) return fail(MOE_ERR_ARG, "%s: inter must be > 0", fn);
    if (c->inter_shared < 0) return fail(MOE_ERR_ARG, "%s: inter_shared must be >= 0", fn);
    if (c->act_dtype == MOE_BF16 || c->gemm_dtype == MOE_FP8_E4M3) {
        if (c->hidden % 128 || c->inter % 128 || c->inter_shared % 128)
            return fail(MOE_ERR_UNSUPPORTED,
                        "%s: bf16/FP8 expert GEMMs need hidden, inter, inter_shared %% 128 == 0",
                        fn);
    }
    if (c->gemm_dtype == MOE_FP8_E4M3) {
        const int64_t kmax = 128 * (int64_t)moe::FP8_MAX_KB;
        if (c->hidden > kmax || c->inter > kmax || c->inter_shared > kmax)
            return fail(MOE_ERR_UNSUPPORTED,
                        "%s: FP8 expert GEMMs need hidden, inter, inter_shared <= %lld", fn,
                        (long long)kmax);
    }
    return MOE_OK;
}

int hip_status(const char* fn, hipError_t e) {
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
    return ok();
}

}  // namespace

namespace moe {
int set_error(int code, const char* msg) {
    if (code == MOE_OK)
        g_err[0] = 0;
    else
        snprintf(g_err, sizeof(g_err), "%s", msg);
    return code;
}
}  // namespace moe

extern "C" {

int moe_abi_version(void) { return 7; }

const char* moe_last_error(void) { return g_err; }

size_t moe_route_workspace_size(const moe_cfg* cfg) {
    if (!cfg) return 0;
    return (size_t)(cfg->tokens * cfg->n_experts * 4);
}

int moe_route(const moe_cfg* cfg, const void* x, const float* centroids, const float* bias,
              float* scores, int32_t* idx, float* gate, int32_t* counts, void* workspace,
              size_t workspace_bytes, void* stream) {
    const char* fn = "moe_route";
    if (int r = check_cfg(fn, cfg)) return r;
    REQ_PTR(centroids);
    REQ_PTR(bias);
    REQ_PTR(counts);
    if (cfg->tokens > 0) {
        REQ_PTR(x);
        REQ_PTR(idx);
        REQ_PTR(gate);
    }
    OPT_PTR(scores);
    if (!scores && cfg->tokens > 0) {
        REQ_PTR(workspace);
        if (workspace_bytes < moe_route_workspace_size(cfg))
            return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, workspace_bytes,
                        moe_route_workspace_size(cfg));
        scores = (float*)workspace;
    }
    return hip_status(fn, moe::launch_route(*cfg, x, centroids, bias, scores, idx, gate, counts,
                                            (hipStream_t)stream));
}

size_t moe_permute_workspace_size(const moe_cfg* cfg) {
    if (!cfg) return 0;
    return moe::permute_workspace_bytes(*cfg);
}

int moe_permute(const moe_cfg* cfg, const void* x, const int32_t* idx, int32_t* offsets,
                int32_t* src_token, int32_t* dst_row, void* x_perm, float* x_perm_scale,
                uint8_t* x_q, float* x_s, void* workspace, size_t workspace_bytes,
                void* stream) {
    const char* fn = "moe_permute";
    if (int r = check_cfg(fn, cfg)) return r;
    REQ_PTR(offsets);
    REQ_PTR(workspace);
    if (cfg->tokens > 0) {
        REQ_PTR(x);
        REQ_PTR(idx);
        REQ_PTR(src_token);
        REQ_PTR(dst_row);
        if (cfg->gemm_dtype == MOE_FP8_E4M3) {
            if (cfg->hidden % 128)
                return fail(MOE_ERR_UNSUPPORTED, "%s: FP8 needs hidden %% 128 == 0", fn);
            // x_perm, x_perm_scale: both or neither (without them the expert
            // GEMM gathers the rows from x_q, x_s through src_token)
            if ((x_perm == nullptr) != (x_perm_scale == nullptr))
                return fail(MOE_ERR_ARG, "%s: x_perm and x_perm_scale: both or neither", fn);
            if (x_perm) {
                REQ_PTR(x_perm);
                REQ_PTR(x_perm_scale);
            }
            REQ_PTR(x_q);
            REQ_PTR(x_s);
        }
    }
    if (workspace_bytes < moe_permute_workspace_size(cfg))
        return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, workspace_bytes,
                    moe_permute_workspace_size(cfg));
    return hip_status(fn, moe::launch_permute(*cfg, x, idx, offsets, src_token, dst_row, x_perm,
                                              x_perm_scale, x_q, x_s, workspace,
                                              (hipStream_t)stream));
}

size_t moe_permute_noalloc_max_bytes(void) { return moe::PERM_SCRATCH_BYTES; }

int moe_permute_noalloc(const moe_cfg* cfg, const void* x, const int32_t* idx, int32_t* offsets,
                        int32_t* src_token, int32_t* dst_row, void* x_perm, float* x_perm_scale,
                        uint8_t* x_q, float* x_s, void* stream) {
    const char* fn = "moe_permute_noalloc";
    if (int r = check_cfg(fn, cfg)) return r;
    REQ_PTR(offsets);
    if (cfg->tokens > 0) {
        REQ_PTR(x);
        REQ_PTR(idx);
        REQ_PTR(src_token);
        REQ_PTR(dst_row);
        if (cfg->gemm_dtype == MOE_FP8_E4M3) {
            if (cfg->hidden % 128)
                return fail(MOE_ERR_UNSUPPORTED, "%s: FP8 needs hidden %% 128 == 0", fn);
            // x_perm, x_perm_scale: both or neither (without them the expert
            // GEMM gathers the rows from x_q, x_s through src_token)
            if ((x_perm == nullptr) != (x_perm_scale == nullptr))
                return fail(MOE_ERR_ARG, "%s: x_perm and x_perm_scale: both or neither", fn);
            if (x_perm) {
                REQ_PTR(x_perm);
                REQ_PTR(x_perm_scale);
            }
            REQ_PTR(x_q);
            REQ_PTR(x_s);
        }
    }
    const size_t need = moe_permute_workspace_size(cfg);
    if (need > moe::PERM_SCRATCH_BYTES)
        return fail(MOE_ERR_WORKSPACE,
                    "%s: this shape needs %zu bytes of scratch, above the built-in %zu "
                    "(tokens * top_k * 4 + ceil(tokens / 64) * n_experts * 4 + n_experts * 4, "
                    "each rounded up to 256); use moe_permute with a workspace",
                    fn, need, moe::PERM_SCRATCH_BYTES);
    void* ws = nullptr;
    const hipError_t e = moe::permute_scratch(&ws);
    if (e != hipSuccess)
        return fail(MOE_ERR_HIP, "%s: scratch address: %s", fn, hipGetErrorString(e));
    return hip_status(fn, moe::launch_permute(*cfg, x, idx, offsets, src_token, dst_row, x_perm,
                                              x_perm_scale, x_q, x_s, ws, (hipStream_t)stream));
}

size_t moe_expert_ffn_workspace_size(const moe_cfg* cfg) {
    if (!cfg) return 0;
    return moe::ffn_workspace_bytes(*cfg);
}

}  // extern "C"

static int expert_ffn_impl(const char* fn, const moe_cfg* cfg, const void* x_perm,
                           const float* x_perm_scale, const int32_t* offsets, const void* w13,
                           const float* w13_scale, const void* w2, const float* w2_scale,
                           void* y_perm, const void* x_sh, const float* x_sh_scale,
                           const void* ws13, const float* ws13_scale, const void* ws2,
                           const float* ws2_scale, void* y_shared, void* saved,
                           void* workspace, size_t workspace_bytes, void* stream,
                           float* h_f32 = nullptr, float* h_f32_shared = nullptr,
                           const int32_t* gather = nullptr) {
    if (int r = check_cfg(fn, cfg)) return r;
    if (int r = check_ffn_shape(fn, cfg)) return r;
    const bool fp8 = cfg->gemm_dtype == MOE_FP8_E4M3;
    if (cfg->tokens > 0) {
        REQ_PTR(x_perm);
        REQ_PTR(offsets);
        REQ_PTR(w13);
        REQ_PTR(w2);
        REQ_PTR(y_perm);
        REQ_PTR(workspace);
        if (fp8) {
            REQ_PTR(x_perm_scale);
            REQ_PTR(w13_scale);
            REQ_PTR(w2_scale);
        }
        if (cfg->inter_shared > 0) {
            REQ_PTR(x_sh);
            REQ_PTR(ws13);
            REQ_PTR(ws2);
            REQ_PTR(y_shared);
            if (fp8) {
                REQ_PTR(x_sh_scale);
                REQ_PTR(ws13_scale);
                REQ_PTR(ws2_scale);
            }
        }
        if (workspace_bytes < moe_expert_ffn_workspace_size(cfg))
            return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, workspace_bytes,
                        moe_expert_ffn_workspace_size(cfg));
    }
    moe::FfnArgs a{x_perm, x_perm_scale, offsets, w13, w13_scale, w2, w2_scale, y_perm,
                   x_sh,   x_sh_scale,   ws13,    ws13_scale, ws2, ws2_scale, y_shared};
    a.gather = gather;
    return hip_status(fn, moe::launch_expert_ffn(*cfg, a, workspace, (hipStream_t)stream, saved,
                                                 h_f32, h_f32_shared));
}

int moe_expert_ffn_gather(const moe_cfg* cfg, const void* x, const float* x_scale,
                          const int32_t* src_token, const int32_t* offsets, const void* w13,
                          const float* w13_scale, const void* w2, const float* w2_scale,
                          void* y_perm, const void* ws13, const float* ws13_scale,
                          const void* ws2, const float* ws2_scale, void* y_shared,
                          void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "moe_expert_ffn_gather";
    if (int r = check_cfg(fn, cfg)) return r;
    const bool fp8 = cfg->gemm_dtype == MOE_FP8_E4M3;
    if (cfg->act_dtype != MOE_BF16)
        return fail(MOE_ERR_UNSUPPORTED, "%s: bf16 and FP8 layers only (use moe_expert_ffn)", fn);
    // the token copies address a row of x by a 32-bit byte offset
    if (cfg->tokens * cfg->hidden * (fp8 ? 1 : 2) >= ((int64_t)1 << 32))
        return fail(MOE_ERR_UNSUPPORTED, "%s: x must stay below 2^32 bytes", fn);
    if (cfg->tokens > 0) {
        REQ_PTR(src_token);
        if (fp8) REQ_PTR(x_scale);
    }
    // the shared expert reads the same rows (x, or its codes and scales)
    return expert_ffn_impl(fn, cfg, x, x_scale, offsets, w13, w13_scale, w2, w2_scale, y_perm,
                           cfg->inter_shared > 0 ? x : nullptr,
                           cfg->inter_shared > 0 ? x_scale : nullptr, ws13, ws13_scale, ws2,
                           ws2_scale, y_shared, nullptr, workspace, workspace_bytes, stream,
                           nullptr, nullptr, src_token);
}

extern "C" {

int moe_expert_ffn(const moe_cfg* cfg, const void* x_perm, const float* x_perm_scale,
                   const int32_t* offsets, const void* w13, const float* w13_scale,
                   const void* w2, const float* w2_scale, void* y_perm, const void* x_sh,
                   const float* x_sh_scale, const void* ws13, const float* ws13_scale,
                   const void* ws2, const float* ws2_scale, void* y_shared, void* workspace,
                   size_t workspace_bytes, void* stream) {
    return expert_ffn_impl("moe_expert_ffn", cfg, x_perm, x_perm_scale, offsets, w13, w13_scale,
                           w2, w2_scale, y_perm, x_sh, x_sh_scale, ws13, ws13_scale, ws2,
                           ws2_scale, y_shared, nullptr, workspace, workspace_bytes, stream);
}

int moe_expert_ffn_h_offsets(const moe_cfg* cfg, size_t off[4]) {
    const char* fn = "moe_expert_ffn_h_offsets";
    if (int r = check_cfg(fn, cfg)) return r;
    if (!off) return fail(MOE_ERR_ARG, "%s: off is NULL", fn);
    moe::ffn_h_offsets(*cfg, off);
    return ok();
}

int moe_expert_ffn_inspect(const moe_cfg* cfg, const void* x_perm, const float* x_perm_scale,
                           const int32_t* offsets, const void* w13, const float* w13_scale,
                           const void* w2, const float* w2_scale, void* y_perm, const void* x_sh,
                           const float* x_sh_scale, const void* ws13, const float* ws13_scale,
                           const void* ws2, const float* ws2_scale, void* y_shared,
                           float* h_f32, float* h_f32_shared, void* workspace,
                           size_t workspace_bytes, void* stream) {
    const char* fn = "moe_expert_ffn_inspect";
    if (int r = check_cfg(fn, cfg)) return r;
    if (cfg->gemm_dtype != MOE_FP8_E4M3)
        return fail(MOE_ERR_UNSUPPORTED, "%s: FP8 layers only", fn);
    if (cfg->tokens > 0) {
        REQ_PTR(h_f32);
        if (cfg->inter_shared > 0) REQ_PTR(h_f32_shared);
    }
    return expert_ffn_impl(fn, cfg, x_perm, x_perm_scale, offsets, w13, w13_scale, w2, w2_scale,
                           y_perm, x_sh, x_sh_scale, ws13, ws13_scale, ws2, ws2_scale, y_shared,
                           nullptr, workspace, workspace_bytes, stream, h_f32,
                           cfg->inter_shared > 0 ? h_f32_shared : nullptr);
}

int moe_expert_ffn_backward_fp8_offsets(const moe_cfg* cfg, size_t off[MOE_BWD8_N]) {
    const char* fn = "moe_expert_ffn_backward_fp8_offsets";
    if (int r = check_cfg(fn, cfg)) return r;
    if (int r = check_ffn_shape(fn, cfg)) return r;
    if (cfg->gemm_dtype != MOE_FP8_E4M3)
        return fail(MOE_ERR_UNSUPPORTED, "%s: FP8 layers only", fn);
    if (!off) return fail(MOE_ERR_ARG, "%s: off is NULL", fn);
    static_assert(MOE_BWD8_N == 25, "one offset per intermediate");
    moe::ffn_backward_fp8_offsets(*cfg, off);
    return ok();
}

int moe_expert_ffn_saved_offsets(const moe_cfg* cfg, size_t off[4]) {
    const char* fn = "moe_expert_ffn_saved_offsets";
    if (int r = check_cfg(fn, cfg)) return r;
    if (!off) return fail(MOE_ERR_ARG, "%s: off is NULL", fn);
    char* base = (char*)(uintptr_t)4096;
    const moe::SavedActs s = moe::carve_saved(*cfg, base);
    off[0] = (size_t)((char*)s.ab_r - base);
    off[1] = (size_t)((char*)s.h_r - base);
    off[2] = (size_t)((char*)s.ab_s - base);
    off[3] = (size_t)((char*)s.h_s - base);
    return ok();
}

int moe_inspect_e4m3(const float* v, int64_t n, float scale, uint8_t* codes4, uint8_t* codes1,
                     void* stream) {
    const char* fn = "moe_inspect_e4m3";
    if (n < 0 || n > ((int64_t)1 << 40)) return fail(MOE_ERR_ARG, "%s: bad n", fn);
    if (!(scale >= 0.0f) || scale > 3.4e38f)
        return fail(MOE_ERR_ARG, "%s: scale must be finite and >= 0", fn);
    if (n > 0) {
        REQ_PTR(v);
        if (!codes4 || !codes1) return fail(MOE_ERR_ARG, "%s: codes4 / codes1 is NULL", fn);
    }
    return hip_status(fn, moe::launch_e4m3_inspect(v, n, scale, codes4, codes1,
                                                   (hipStream_t)stream));
}

size_t moe_expert_ffn_saved_size(const moe_cfg* cfg) {
    if (!cfg) return 0;
    return moe::ffn_saved_bytes(*cfg);
}

int moe_expert_ffn_train(const moe_cfg* cfg, const void* x_perm, const int32_t* offsets,
                         const void* w13, const void* w2, void* y_perm, const void* x_sh,
                         const void* ws13, const void* ws2, void* y_shared, void* saved,
                         size_t saved_bytes, void* workspace, size_t workspace_bytes,
                         void* stream) {
    const char* fn = "moe_expert_ffn_train";
    if (int r = check_cfg(fn, cfg)) return r;
    if (cfg->gemm_dtype != cfg->act_dtype)
        return fail(MOE_ERR_UNSUPPORTED, "%s: the training forward covers bf16 and fp32 storage",
                    fn);
    if (cfg->tokens > 0) {
        REQ_PTR(saved);
        if (saved_bytes < moe_expert_ffn_saved_size(cfg))
            return fail(MOE_ERR_WORKSPACE, "%s: saved %zu < %zu bytes", fn, saved_bytes,
                        moe_expert_ffn_saved_size(cfg));
    }
    return expert_ffn_impl(fn, cfg, x_perm, nullptr, offsets, w13, nullptr, w2, nullptr, y_perm,
                           x_sh, nullptr, ws13, nullptr, ws2, nullptr, y_shared,
                           cfg->tokens > 0 ? saved : nullptr, workspace, workspace_bytes, stream);
}

int moe_expert_ffn_train_fp8(const moe_cfg* cfg, const void* x_perm, const float* x_perm_scale,
                             const int32_t* offsets, const void* w13, const float* w13_scale,
                             const void* w2, const float* w2_scale, void* y_perm,
                             const void* x_sh, const float* x_sh_scale, const void* ws13,
                             const float* ws13_scale, const void* ws2, const float* ws2_scale,
                             void* y_shared, void* saved, size_t saved_bytes, void* workspace,
                             size_t workspace_bytes, void* stream) {
    const char* fn = "moe_expert_ffn_train_fp8";
    if (int r = check_cfg(fn, cfg)) return r;
    if (cfg->gemm_dtype != MOE_FP8_E4M3 || cfg->act_dtype != MOE_BF16)
        return fail(MOE_ERR_UNSUPPORTED, "%s: needs gemm_dtype FP8_E4M3 and act_dtype BF16", fn);
    if (cfg->tokens > 0) {
        REQ_PTR(saved);
        if (saved_bytes < moe_expert_ffn_saved_size(cfg))
            return fail(MOE_ERR_WORKSPACE, "%s: saved %zu < %zu bytes", fn, saved_bytes,
                        moe_expert_ffn_saved_size(cfg));
    }
    return expert_ffn_impl(fn, cfg, x_perm, x_perm_scale, offsets, w13, w13_scale, w2, w2_scale,
                           y_perm, x_sh, x_sh_scale, ws13, ws13_scale, ws2, ws2_scale, y_shared,
                           cfg->tokens > 0 ? saved : nullptr, workspace, workspace_bytes, stream);
}

}  // extern "C"

extern "C" {

size_t moe_packed_weights_size(const moe_cfg* cfg, int which) {
    if (!cfg || which < 0 || which > 7) return 0;
    return moe::packed_weight_bytes(*cfg, which);
}

int moe_pack_weights(const moe_cfg* cfg, int which, const void* w, void* w_packed,
                     void* stream) {
    const char* fn = "moe_pack_weights";
    if (int r = check_cfg(fn, cfg)) return r;
    if (int r = check_ffn_shape(fn, cfg)) return r;
    if (which < 0 || which > 7) return fail(MOE_ERR_ARG, "%s: which must be 0..7", fn);
    if ((which == 2 || which == 3 || which == 6 || which == 7) && cfg->inter_shared == 0)
        return fail(MOE_ERR_ARG, "%s: no shared expert (inter_shared == 0)", fn);
    REQ_PTR(w);
    REQ_PTR(w_packed);
    if (w == w_packed) return fail(MOE_ERR_ARG, "%s: packing cannot run in place", fn);
    return hip_status(fn, moe::launch_pack_weights(*cfg, which, w, w_packed, (hipStream_t)stream));
}

int moe_combine(const moe_cfg* cfg, const void* x_residual, const void* y_shared,
                const void* y_perm, const float* gate, const int32_t* dst_row, void* out,
                void* stream) {
    const char* fn = "moe_combine";
    if (int r = check_cfg(fn, cfg)) return r;
    if (cfg->tokens > 0) {
        REQ_PTR(y_perm);
        REQ_PTR(gate);
        REQ_PTR(dst_row);
        REQ_PTR(out);
        OPT_PTR(x_residual);
        OPT_PTR(y_shared);
        if (out == x_residual || out == y_shared || out == y_perm)
            return fail(MOE_ERR_ARG, "%s: out must not alias an input", fn);
    }
    return hip_status(fn, moe::launch_combine(*cfg, x_residual, y_shared, y_perm, gate, dst_row,
                                              out, (hipStream_t)stream));
}

int moe_bias_update(int64_t n_experts, int64_t tokens_times_k, const int32_t* counts,
                    float gamma, float* bias, void* stream) {
    const char* fn = "moe_bias_update";
    if (n_experts < 1 || n_experts > (int64_t)1 << 20)
        return fail(MOE_ERR_ARG, "%s: n_experts out of range", fn);
    if (tokens_times_k < 0) return fail(MOE_ERR_ARG, "%s: tokens_times_k < 0", fn);
    if (!(gamma == gamma)) return fail(MOE_ERR_ARG, "%s: gamma is NaN", fn);
    REQ_PTR(counts);
    REQ_PTR(bias);
    return hip_status(fn, moe::launch_bias_update(n_experts, tokens_times_k, counts, gamma, bias,
                                                  (hipStream_t)stream));
}

size_t moe_seq_balance_loss_workspace_size(const moe_cfg* cfg, int64_t seq_len) {
    if (!cfg) return 0;
    return moe::seq_balance_workspace_bytes(cfg->tokens, cfg->n_experts, seq_len);
}

int moe_seq_balance_loss(const moe_cfg* cfg, int64_t seq_len, float alpha, const float* scores,
                         const int32_t* idx, float* loss, void* workspace,
                         size_t workspace_bytes, void* stream) {
    const char* fn = "moe_seq_balance_loss";
    if (int r = check_cfg(fn, cfg)) return r;
    if (seq_len < 1) return fail(MOE_ERR_ARG, "%s: seq_len must be >= 1", fn);
    if (cfg->tokens % seq_len)
        return fail(MOE_ERR_ARG, "%s: tokens=%lld is not a multiple of seq_len=%lld", fn,
                    (long long)cfg->tokens, (long long)seq_len);
    if (!(alpha == alpha)) return fail(MOE_ERR_ARG, "%s: alpha is NaN", fn);
    if (cfg->tokens == 0) return ok();
    REQ_PTR(scores);
    REQ_PTR(idx);
    REQ_PTR(loss);
    REQ_PTR(workspace);
    const size_t need = moe_seq_balance_loss_workspace_size(cfg, seq_len);
    if (workspace_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, workspace_bytes,
                    need);
    return hip_status(fn, moe::launch_seq_balance_loss(cfg->tokens, cfg->n_experts, cfg->top_k,
                                                       seq_len, alpha, scores, idx, loss,
                                                       workspace, (hipStream_t)stream));
}

int moe_quantize_weights_fp8(int64_t n_mats, int64_t rows, int64_t cols, const void* w_bf16,
                             uint8_t* w_q, float* w_scale, void* stream) {
    const char* fn = "moe_quantize_weights_fp8";
    if (n_mats < 0 || rows <= 0 || cols <= 0 || rows % 128 || cols % 128)
        return fail(MOE_ERR_ARG, "%s: rows and cols must be positive multiples of 128", fn);
    if (n_mats * (rows / 128) * (cols / 128) > INT32_MAX)
        return fail(MOE_ERR_ARG, "%s: too many blocks", fn);
    if (n_mats > 0) {
        REQ_PTR(w_bf16);
        REQ_PTR(w_q);
        REQ_PTR(w_scale);
    }
    return hip_status(fn, moe::launch_quantize_weights(n_mats, rows, cols, w_bf16, w_q, w_scale,
                                                       (hipStream_t)stream));
}

}  // extern "C"

// ------------------------------------------------------------------ backward

extern "C" {

int moe_combine_backward(const moe_cfg* cfg, const void* dout, const void* y_perm,
                         const float* gate, const int32_t* dst_row, void* dy_perm, float* dgate,
                         void* stream) {
    const char* fn = "moe_combine_backward";
    if (int r = check_cfg(fn, cfg)) return r;
    if (cfg->tokens > 0) {
        REQ_PTR(dout);
        REQ_PTR(y_perm);
        REQ_PTR(gate);
        REQ_PTR(dst_row);
        REQ_PTR(dy_perm);
        REQ_PTR(dgate);
        if (dy_perm == dout || dy_perm == y_perm)
            return fail(MOE_ERR_ARG, "%s: dy_perm must not alias an input", fn);
    }
    return hip_status(fn, moe::launch_combine_backward(*cfg, dout, y_perm, gate, dst_row, dy_perm,
                                                       dgate, (hipStream_t)stream));
}

size_t moe_expert_ffn_backward_workspace_size(const moe_cfg* cfg) {
    if (!cfg) return 0;
    return moe::ffn_backward_workspace_bytes(*cfg);
}

int moe_expert_ffn_backward(const moe_cfg* cfg, const void* x_perm, const int32_t* offsets,
                            const void* w13, const void* w13t, const void* w2t,
                            const void* dy_perm, const void* x_sh, const void* ws13,
                            const void* ws13t, const void* ws2t, const void* dy_shared,
                            void* dx_perm, void* dx_shared, void* dw13, void* dw2, void* dws13,
                            void* dws2, const void* saved, size_t saved_bytes, void* workspace,
                            size_t workspace_bytes, void* stream) {
    const char* fn = "moe_expert_ffn_backward";
    if (int r = check_cfg(fn, cfg)) return r;
    if (int r = check_ffn_shape(fn, cfg)) return r;
    if (cfg->gemm_dtype != cfg->act_dtype)
        return fail(MOE_ERR_UNSUPPORTED, "%s: the backward covers bf16 and fp32 storage only", fn);
    // every routed weight gradient is written, also with no tokens (zeros)
    REQ_PTR(dw13);
    REQ_PTR(dw2);
    REQ_PTR(offsets);
    REQ_PTR(workspace);
    if (cfg->tokens > 0) {
        REQ_PTR(x_perm);
        OPT_PTR(w13);
        REQ_PTR(w13t);
        REQ_PTR(w2t);
        REQ_PTR(dy_perm);
        REQ_PTR(dx_perm);
        if (cfg->inter_shared > 0) {
            REQ_PTR(x_sh);
            if (!saved) REQ_PTR(ws13);
            REQ_PTR(ws13t);
            REQ_PTR(ws2t);
            REQ_PTR(dy_shared);
            REQ_PTR(dx_shared);
            REQ_PTR(dws13);
            REQ_PTR(dws2);
        }
    }
    if (cfg->act_dtype == MOE_BF16) {
        // weight-gradient copies address an expert's rows with 32-bit byte offsets
        const int64_t w = cfg->hidden > 2 * cfg->inter ? cfg->hidden : 2 * cfg->inter;
        const int64_t ws = 2 * cfg->inter_shared > w ? 2 * cfg->inter_shared : w;
        if ((cfg->tokens + 32) * ws * 2 >= ((int64_t)1 << 32))
            return fail(MOE_ERR_UNSUPPORTED, "%s: tokens * width exceeds the 32-bit row offsets",
                        fn);
    }
    if (cfg->act_dtype == MOE_F32) {
        // one thread per output element
        const int64_t T = cfg->tokens, I = cfg->inter, Is = cfg->inter_shared, d = cfg->hidden;
        const int64_t big = (T * cfg->top_k + T) * (I > Is ? I : Is) + cfg->n_experts * 2 * I * d;
        if (big > (int64_t)1 << 38)
            return fail(MOE_ERR_UNSUPPORTED, "%s: fp32 layer too large for the VALU path", fn);
    }
    if (workspace_bytes < moe_expert_ffn_backward_workspace_size(cfg))
        return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, workspace_bytes,
                    moe_expert_ffn_backward_workspace_size(cfg));
    OPT_PTR(saved);
    if (saved && saved_bytes < moe_expert_ffn_saved_size(cfg))
        return fail(MOE_ERR_WORKSPACE, "%s: saved %zu < %zu bytes", fn, saved_bytes,
                    moe_expert_ffn_saved_size(cfg));
    if (!saved && cfg->tokens > 0 && !w13)
        return fail(MOE_ERR_ARG, "%s: w13 is needed to recompute without saved activations", fn);
    moe::FfnBwdArgs a{x_perm,  offsets, w13,     w13t,      w2t,  dy_perm, x_sh, ws13,  ws13t,
                      ws2t,    dy_shared, dx_perm, dx_shared, dw13, dw2,     dws13, dws2};
    return hip_status(fn, moe::launch_expert_ffn_backward(*cfg, a, workspace, (hipStream_t)stream,
                                                          saved));
}

size_t moe_expert_ffn_backward_fp8_workspace_size(const moe_cfg* cfg) {
    if (!cfg) return 0;
    return moe::ffn_backward_fp8_workspace_bytes(*cfg);
}

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
                                void* stream) {
    const char* fn = "moe_expert_ffn_backward_fp8";
    if (int r = check_cfg(fn, cfg)) return r;
    if (int r = check_ffn_shape(fn, cfg)) return r;
    if (cfg->gemm_dtype != MOE_FP8_E4M3 || cfg->act_dtype != MOE_BF16)
        return fail(MOE_ERR_UNSUPPORTED, "%s: needs gemm_dtype FP8_E4M3 and act_dtype BF16", fn);
    const int64_t T = cfg->tokens, R = T * cfg->top_k;
    {
        // row-direction tiles: the padded rows times the widest feature count
        // must stay within the 32-bit offsets of the weight-gradient copies
        const int64_t P = R + 128 * (cfg->n_experts + 2) + T;
        const int64_t Im = cfg->inter > cfg->inter_shared ? cfg->inter : cfg->inter_shared;
        const int64_t F = cfg->hidden > 2 * Im ? cfg->hidden : 2 * Im;
        if (P >= ((int64_t)1 << 31) || P * F >= ((int64_t)1 << 32))
            return fail(MOE_ERR_UNSUPPORTED, "%s: too many rows for the 32-bit tile offsets", fn);
    }
    REQ_PTR(dw13);
    REQ_PTR(dw2);
    REQ_PTR(offsets);
    REQ_PTR(workspace);
    if (T > 0) {
        REQ_PTR(x);
        REQ_PTR(src_token);
        REQ_PTR(x_perm);
        REQ_PTR(x_perm_scale);
        REQ_PTR(w13);
        REQ_PTR(w13t);
        REQ_PTR(w13_scale);
        REQ_PTR(w2t);
        REQ_PTR(w2_scale);
        REQ_PTR(dy_perm);
        REQ_PTR(dx_perm);
        if (cfg->inter_shared > 0) {
            REQ_PTR(x_q);
            REQ_PTR(x_scale);
            REQ_PTR(ws13);
            REQ_PTR(ws13t);
            REQ_PTR(ws13_scale);
            REQ_PTR(ws2t);
            REQ_PTR(ws2_scale);
            REQ_PTR(dy_shared);
            REQ_PTR(dx_shared);
            REQ_PTR(dws13);
            REQ_PTR(dws2);
        }
    }
    if (workspace_bytes < moe_expert_ffn_backward_fp8_workspace_size(cfg))
        return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, workspace_bytes,
                    moe_expert_ffn_backward_fp8_workspace_size(cfg));
    OPT_PTR(saved);
    if (saved && saved_bytes < moe_expert_ffn_saved_size(cfg))
        return fail(MOE_ERR_WORKSPACE, "%s: saved %zu < %zu bytes", fn, saved_bytes,
                    moe_expert_ffn_saved_size(cfg));
    moe::FfnBwdFp8Args a{};
    a.x = x;
    a.src_token = src_token;
    a.offsets = offsets;
    a.x_perm_q = x_perm;
    a.x_perm_s = x_perm_scale;
    a.x_q = x_q;
    a.x_s = x_scale;
    a.w13 = w13;
    a.w13t = w13t;
    a.w13_s = w13_scale;
    a.w2t = w2t;
    a.w2_s = w2_scale;
    a.ws13 = ws13;
    a.ws13t = ws13t;
    a.ws13_s = ws13_scale;
    a.ws2t = ws2t;
    a.ws2_s = ws2_scale;
    a.dy_perm = dy_perm;
    a.dy_sh = dy_shared;
    a.dx_perm = dx_perm;
    a.dx_sh = dx_shared;
    a.dw13 = dw13;
    a.dw2 = dw2;
    a.dws13 = dws13;
    a.dws2 = dws2;
    return hip_status(fn, moe::launch_expert_ffn_backward_fp8(*cfg, a, workspace,
                                                              (hipStream_t)stream, saved));
}

size_t moe_route_backward_workspace_size(const moe_cfg* cfg) {
    if (!cfg) return 0;
    return (size_t)(cfg->tokens * cfg->top_k * 4);
}

int moe_route_backward(const moe_cfg* cfg, const void* x, const float* scores,
                       const int32_t* idx, const float* dgate, const int32_t* offsets,
                       const int32_t* src_token, const int32_t* dst_row, float* dz,
                       float* dcentroids, void* workspace, size_t workspace_bytes,
                       void* stream) {
    const char* fn = "moe_route_backward";
    if (int r = check_cfg(fn, cfg)) return r;
    REQ_PTR(offsets);
    REQ_PTR(dcentroids);
    if (cfg->tokens > 0) {
        REQ_PTR(x);
        REQ_PTR(scores);
        REQ_PTR(idx);
        REQ_PTR(dgate);
        REQ_PTR(src_token);
        REQ_PTR(dst_row);
        REQ_PTR(dz);
        REQ_PTR(workspace);
        if (workspace_bytes < moe_route_backward_workspace_size(cfg))
            return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, workspace_bytes,
                        moe_route_backward_workspace_size(cfg));
    }
    return hip_status(fn, moe::launch_route_backward(*cfg, x, scores, idx, dgate, offsets,
                                                     src_token, dst_row, dz, (float*)workspace,
                                                     dcentroids, (hipStream_t)stream));
}

int moe_input_grad(const moe_cfg* cfg, const void* dout, const void* dx_shared,
                   const void* dx_perm, const int32_t* dst_row, const float* dz,
                   const int32_t* idx, const float* centroids, void* dx, void* stream) {
    const char* fn = "moe_input_grad";
    if (int r = check_cfg(fn, cfg)) return r;
    if (cfg->tokens > 0) {
        REQ_PTR(dx_perm);
        REQ_PTR(dst_row);
        REQ_PTR(dz);
        REQ_PTR(idx);
        REQ_PTR(centroids);
        REQ_PTR(dx);
        OPT_PTR(dout);
        OPT_PTR(dx_shared);
        if (dx == dout || dx == dx_shared || dx == dx_perm)
            return fail(MOE_ERR_ARG, "%s: dx must not alias an input", fn);
    }
    return hip_status(fn, moe::launch_input_grad(*cfg, dout, dx_shared, dx_perm, dst_row, dz, idx,
                                                 centroids, dx, (hipStream_t)stream));
}

}  // extern "C"
