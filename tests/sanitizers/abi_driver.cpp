// abi_driver.cpp -- calls every entry point of libmoe's C ABI (include/*.h)
// with arguments its host-side validation must reject, and the host-only size
// and offset queries, against a library whose host code is built with
// AddressSanitizer and UndefinedBehaviorSanitizer.  No call reaches the GPU:
// each returns from validation (checked by its status code), so the run needs
// no device.  Exit status 0 and "abi driver ok" mean every status matched and
// the sanitizers saw nothing.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "moe.h"
#include "moe_backward.h"
#include "moe_inspect.h"
#include "moe_probe.h"

static int failures = 0;

static void expect(const char* what, int got, int want) {
    if (got != want) {
        std::printf("FAIL %s: status %d, expected %d (%s)\n", what, got, want, moe_last_error());
        ++failures;
    } else if (want != MOE_OK && std::strlen(moe_last_error()) == 0) {
        std::printf("FAIL %s: no error message\n", what);
        ++failures;
    }
}

static moe_cfg cfg(int64_t T = 64, int64_t d = 128, int64_t N = 16, int64_t k = 2,
                   int64_t G = 1, int64_t TG = 1, int64_t I = 64, int64_t Is = 64,
                   int act = MOE_F32, int gemm = MOE_F32) {
    moe_cfg c;
    c.tokens = T; c.hidden = d; c.n_experts = N; c.top_k = k; c.n_group = G; c.topk_group = TG;
    c.inter = I; c.inter_shared = Is; c.act_dtype = act; c.gemm_dtype = gemm;
    return c;
}

int main() {
    // aligned, non-null addresses that validation must refuse before any use
    char* F = reinterpret_cast<char*>(uintptr_t(1) << 20);
    char* M = F + 4;  // misaligned
    moe_cfg c = cfg();
    expect("route: NULL cfg", moe_route(nullptr, F, (float*)F, (float*)F, (float*)F, (int32_t*)F,
                                        (float*)F, (int32_t*)F, nullptr, 0, nullptr), MOE_ERR_ARG);
    moe_cfg bad[] = {cfg(64, 128, 16, 17), cfg(64, 128, 16, 0), cfg(64, 128, 0, 1),
                     cfg(64, 128, 2048, 2), cfg(64, 128, 16, 2, 5, 2), cfg(64, 128, 16, 5, 8, 2),
                     cfg(64, 128, 16, 2, 4, 5), cfg(64, 128, 16, 2, 16, 2), cfg(-1)};
    for (auto& b : bad)
        expect("route: bad shape", moe_route(&b, F, (float*)F, (float*)F, (float*)F, (int32_t*)F,
                                             (float*)F, (int32_t*)F, nullptr, 0, nullptr),
               MOE_ERR_ARG);
    moe_cfg bd = cfg(64, 100, 16, 2, 1, 1, 64, 64, MOE_BF16, MOE_BF16);
    expect("route: bf16 d % 8", moe_route(&bd, F, (float*)F, (float*)F, (float*)F, (int32_t*)F,
                                          (float*)F, (int32_t*)F, nullptr, 0, nullptr),
           MOE_ERR_UNSUPPORTED);
    expect("route: NULL centroids", moe_route(&c, F, nullptr, (float*)F, (float*)F, (int32_t*)F,
                                              (float*)F, (int32_t*)F, nullptr, 0, nullptr),
           MOE_ERR_ARG);
    expect("route: misaligned idx", moe_route(&c, F, (float*)F, (float*)F, (float*)F, (int32_t*)M,
                                              (float*)F, (int32_t*)F, nullptr, 0, nullptr),
           MOE_ERR_ARG);
    expect("route: small workspace", moe_route(&c, F, (float*)F, (float*)F, nullptr, (int32_t*)F,
                                               (float*)F, (int32_t*)F, F, 16, nullptr),
           MOE_ERR_WORKSPACE);
    if (moe_route_workspace_size(&c) != 64 * 16 * 4) { std::printf("FAIL route ws size\n"); ++failures; }
    if (moe_route_workspace_size(nullptr) != 0) { std::printf("FAIL route ws NULL\n"); ++failures; }

    // permute, and the variant without a workspace
    moe_cfg cb = cfg(64, 256, 16, 2, 1, 1, 128, 128, MOE_BF16, MOE_BF16);
    size_t need = moe_permute_workspace_size(&cb);
    expect("permute: small workspace",
           moe_permute(&cb, F, (int32_t*)F, (int32_t*)F, (int32_t*)F, (int32_t*)F, F, nullptr,
                       nullptr, nullptr, F, need - 1, nullptr), MOE_ERR_WORKSPACE);
    moe_cfg c8 = cfg(64, 256, 16, 2, 1, 1, 128, 128, MOE_BF16, MOE_FP8_E4M3);
    expect("permute: FP8 without scales",
           moe_permute(&c8, F, (int32_t*)F, (int32_t*)F, (int32_t*)F, (int32_t*)F, F, nullptr,
                       nullptr, nullptr, F, 1 << 30, nullptr), MOE_ERR_ARG);
    moe_cfg huge = cfg(int64_t(1) << 22, 1024, 256, 8, 1, 1, 512, 512, MOE_BF16, MOE_BF16);
    expect("permute_noalloc: above the built-in scratch",
           moe_permute_noalloc(&huge, F, (int32_t*)F, (int32_t*)F, (int32_t*)F, (int32_t*)F, F,
                               nullptr, nullptr, nullptr, nullptr), MOE_ERR_WORKSPACE);
    expect("permute_noalloc: NULL offsets",
           moe_permute_noalloc(&cb, F, (int32_t*)F, nullptr, (int32_t*)F, (int32_t*)F, F,
                               nullptr, nullptr, nullptr, nullptr), MOE_ERR_ARG);
    if (moe_permute_noalloc_max_bytes() != (size_t(8) << 20)) { std::printf("FAIL noalloc max\n"); ++failures; }

    // expert FFN and its size queries
    const void* P15[15];
    for (auto& p : P15) p = F;
    moe_cfg c8f = cfg(64, 128, 16, 2, 1, 1, 64, 64, MOE_F32, MOE_FP8_E4M3);
    expect("ffn: FP8 with fp32 activations",
           moe_expert_ffn(&c8f, F, (float*)F, (int32_t*)F, F, (float*)F, F, (float*)F, (void*)F, F,
                          (float*)F, F, (float*)F, F, (float*)F, (void*)F, F, 1 << 30, nullptr),
           MOE_ERR_UNSUPPORTED);
    moe_cfg c8i = cfg(64, 128, 16, 2, 1, 1, 96, 64, MOE_BF16, MOE_FP8_E4M3);
    expect("ffn: FP8 inter % 128",
           moe_expert_ffn(&c8i, F, (float*)F, (int32_t*)F, F, (float*)F, F, (float*)F, (void*)F, F,
                          (float*)F, F, (float*)F, F, (float*)F, (void*)F, F, 1 << 30, nullptr),
           MOE_ERR_UNSUPPORTED);
    need = moe_expert_ffn_workspace_size(&cb);
    expect("ffn: small workspace",
           moe_expert_ffn(&cb, F, nullptr, (int32_t*)F, F, nullptr, F, nullptr, (void*)F, F,
                          nullptr, F, nullptr, F, nullptr, (void*)F, F, need - 1, nullptr),
           MOE_ERR_WORKSPACE);
    expect("ffn_inspect: not FP8",
           moe_expert_ffn_inspect(&cb, F, nullptr, (int32_t*)F, F, nullptr, F, nullptr, (void*)F,
                                  F, nullptr, F, nullptr, F, nullptr, (void*)F, (float*)F,
                                  (float*)F, F, 1 << 30, nullptr), MOE_ERR_UNSUPPORTED);
    expect("ffn_inspect: NULL h", moe_expert_ffn_inspect(
               &c8, F, (float*)F, (int32_t*)F, F, (float*)F, F, (float*)F, (void*)F, F, (float*)F,
               F, (float*)F, F, (float*)F, (void*)F, nullptr, (float*)F, F, 1 << 30, nullptr),
           MOE_ERR_ARG);
    size_t off[4];
    expect("h_offsets: FP8", moe_expert_ffn_h_offsets(&c8, off), MOE_OK);
    if (!(off[0] < off[1] && off[1] < off[2] && off[2] < off[3] &&
          off[3] < moe_expert_ffn_workspace_size(&c8))) { std::printf("FAIL h offsets\n"); ++failures; }
    expect("h_offsets: bf16", moe_expert_ffn_h_offsets(&cb, off), MOE_OK);
    if (off[2] != SIZE_MAX || off[3] != SIZE_MAX) { std::printf("FAIL h offsets bf16\n"); ++failures; }
    expect("h_offsets: NULL", moe_expert_ffn_h_offsets(&cb, nullptr), MOE_ERR_ARG);
    for (int w = -1; w <= 8; ++w) {
        size_t s = moe_packed_weights_size(&cb, w);
        if ((w < 0 || w > 7) != (s == 0)) { std::printf("FAIL packed size %d\n", w); ++failures; }
    }
    expect("pack: which 9", moe_pack_weights(&cb, 9, F, F + 4096, nullptr), MOE_ERR_ARG);
    expect("pack: in place", moe_pack_weights(&cb, 0, F, F, nullptr), MOE_ERR_ARG);
    moe_cfg cns = cfg(64, 256, 16, 2, 1, 1, 128, 0, MOE_BF16, MOE_BF16);
    expect("pack: shared without Is", moe_pack_weights(&cns, 2, F, F + 4096, nullptr), MOE_ERR_ARG);

    // combine, bias update, weight quantiser, encoder inspection, probes
    expect("combine: out aliases x", moe_combine(&c, F, F + 16, F + 32, (float*)(F + 48),
                                                 (int32_t*)(F + 64), F, nullptr), MOE_ERR_ARG);
    expect("bias: N = 0", moe_bias_update(0, 10, (int32_t*)F, 0.001f, (float*)F, nullptr),
           MOE_ERR_ARG);
    expect("bias: NaN gamma", moe_bias_update(8, 10, (int32_t*)F, std::nanf(""), (float*)F,
                                              nullptr), MOE_ERR_ARG);
    expect("quantize: rows % 128", moe_quantize_weights_fp8(1, 100, 128, F, (uint8_t*)F,
                                                            (float*)F, nullptr), MOE_ERR_ARG);
    expect("inspect_e4m3: negative scale", moe_inspect_e4m3((float*)F, 4, -1.0f, (uint8_t*)F,
                                                            (uint8_t*)F, nullptr), MOE_ERR_ARG);
    expect("inspect_e4m3: n < 0", moe_inspect_e4m3((float*)F, -4, 1.0f, (uint8_t*)F,
                                                   (uint8_t*)F, nullptr), MOE_ERR_ARG);
    expect("probe hbm: NULL buffer", moe_probe_hbm_read(nullptr, 1 << 20, 16, (uint32_t*)F,
                                                        nullptr), MOE_ERR_ARG);
    expect("probe mfma: bad dtype", moe_probe_mfma(0, 10, 1, (float*)F, nullptr), MOE_ERR_ARG);

    // backward calls
    expect("combine_backward: alias", moe_combine_backward(&c, F, F + 16, (float*)(F + 32),
                                                           (int32_t*)(F + 48), F, (float*)(F + 64),
                                                           nullptr), MOE_ERR_ARG);
    need = moe_expert_ffn_backward_workspace_size(&cb);
    expect("ffn_backward: small workspace", moe_expert_ffn_backward(
               &cb, F, (int32_t*)F, F, F, F, F, F, F, F, F, F, (void*)F, (void*)F, (void*)F,
               (void*)F, (void*)F, (void*)F, nullptr, 0, (void*)F, need - 1, nullptr),
           MOE_ERR_WORKSPACE);
    expect("ffn_backward: FP8 layer", moe_expert_ffn_backward(
               &c8, F, (int32_t*)F, F, F, F, F, F, F, F, F, F, (void*)F, (void*)F, (void*)F,
               (void*)F, (void*)F, (void*)F, nullptr, 0, (void*)F, 1 << 30, nullptr),
           MOE_ERR_UNSUPPORTED);
    need = moe_expert_ffn_backward_fp8_workspace_size(&c8);
    expect("ffn_backward_fp8: small workspace", moe_expert_ffn_backward_fp8(
               &c8, F, (int32_t*)F, (int32_t*)F, (uint8_t*)F, (float*)F, (uint8_t*)F, (float*)F,
               F, F, (float*)F, F, (float*)F, F, F, (float*)F, F, (float*)F, F, F, (void*)F,
               (void*)F, (void*)F, (void*)F, (void*)F, (void*)F, nullptr, 0, (void*)F, need - 1,
               nullptr), MOE_ERR_WORKSPACE);
    size_t sv = moe_expert_ffn_saved_size(&cb);
    expect("train: small saved", moe_expert_ffn_train(&cb, F, (int32_t*)F, F, F, (void*)F, F, F,
                                                      F, (void*)F, (void*)F, sv - 1, (void*)F,
                                                      1 << 30, nullptr), MOE_ERR_WORKSPACE);
    expect("train_fp8: not FP8", moe_expert_ffn_train_fp8(
               &cb, F, (float*)F, (int32_t*)F, F, (float*)F, F, (float*)F, (void*)F, F, (float*)F,
               F, (float*)F, F, (float*)F, (void*)F, (void*)F, sv, (void*)F, 1 << 30, nullptr),
           MOE_ERR_UNSUPPORTED);
    expect("route_backward: small workspace", moe_route_backward(
               &c, F, (float*)F, (int32_t*)F, (float*)F, (int32_t*)F, (int32_t*)F, (int32_t*)F,
               (float*)F, (float*)F, (void*)F, 64 * 2 * 4 - 1, nullptr), MOE_ERR_WORKSPACE);
    expect("input_grad: alias", moe_input_grad(&c, F, F + 16, F + 32, (int32_t*)(F + 48),
                                               (float*)(F + 64), (int32_t*)(F + 80),
                                               (float*)(F + 96), F + 32, nullptr), MOE_ERR_ARG);
    if (moe_abi_version() <= 0) { std::printf("FAIL abi version\n"); ++failures; }
    if (failures) return 1;
    std::printf("abi driver ok\n");
    return 0;
}
