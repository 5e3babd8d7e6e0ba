"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/moe.h declares, and rejects bad arguments with the
documented status codes before enqueuing anything (these calls return from
validation and never reach a HIP launch)."""
import ctypes
import os
import re

import pytest

import torch

import sparse_moe_layer_bias_amd as moe

# The argument-rejection tests pass fake device addresses that validation must
# refuse; they are host checks and are not run where a GPU is visible.
host_only = pytest.mark.skipif(torch.cuda.is_available(),
                               reason="host-only validation checks use fake device pointers")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            src = open(os.path.join(ROOT, "include", h)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(moe_\w+)\s*\(", src))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    names = _declared()
    assert {"moe_route", "moe_permute", "moe_expert_ffn", "moe_combine",
            "moe_bias_update"} <= set(names)
    assert {"moe_probe_hbm_read", "moe_probe_mfma"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert moe.moe_abi_version() == 2


@host_only
@pytest.mark.parametrize("call,code", [
    (lambda L: L.moe_probe_hbm_read(None, 1 << 20, 16, ctypes.c_void_p(FAKE), None), 1),
    (lambda L: L.moe_probe_hbm_read(ctypes.c_void_p(FAKE), 1000, 16, ctypes.c_void_p(FAKE), None), 1),
    (lambda L: L.moe_probe_hbm_read(ctypes.c_void_p(FAKE), 1 << 20, 0, ctypes.c_void_p(FAKE), None), 1),
    (lambda L: L.moe_probe_hbm_read(ctypes.c_void_p(FAKE + 8), 1 << 20, 16, ctypes.c_void_p(FAKE), None), 1),
    (lambda L: L.moe_probe_mfma(0, 10, 1, ctypes.c_void_p(FAKE), None), 1),
    (lambda L: L.moe_probe_mfma(1, 0, 1, ctypes.c_void_p(FAKE), None), 1),
    (lambda L: L.moe_probe_mfma(2, 10, 0, ctypes.c_void_p(FAKE), None), 1),
    (lambda L: L.moe_probe_mfma(1, 10, 1, None, None), 1),
])
def test_probes_reject_bad_arguments(call, code):
    from sparse_moe_layer_bias_amd import probe
    L = probe._lib()
    assert call(L) == code
    assert moe.lib().moe_last_error()


def _cfg(**kw):
    base = dict(T=64, d=128, N=16, k=2, G=1, TG=1, I=64, Is=64, dtype="f32", fp8=False)
    base.update(kw)
    return moe.make_cfg(**base)


FAKE = 1 << 20  # an aligned non-null address; validation fails before any use


def _route(cfg, **over):
    args = dict(x=FAKE, centroids=FAKE, bias=FAKE, scores=FAKE, idx=FAKE, gate=FAKE,
                counts=FAKE)
    args.update(over)
    L = moe.lib()
    P = ctypes.c_void_p
    return L.moe_route(ctypes.byref(cfg), *(P(args[k]) if args[k] else None for k in
                                            ("x", "centroids", "bias", "scores", "idx", "gate",
                                             "counts")), None, 0, None)


@host_only
@pytest.mark.parametrize("kw,code", [
    (dict(k=17), moe.MOE_ERR_ARG),             # k > N
    (dict(k=0), moe.MOE_ERR_ARG),
    (dict(N=0), moe.MOE_ERR_ARG),
    (dict(N=2048), moe.MOE_ERR_ARG),
    (dict(G=5, TG=2), moe.MOE_ERR_ARG),        # N % G != 0
    (dict(G=8, TG=2, k=5), moe.MOE_ERR_ARG),   # k > TG * N/G
    (dict(G=4, TG=5), moe.MOE_ERR_ARG),
    (dict(G=16, TG=2), moe.MOE_ERR_ARG),       # 1 expert per group
    (dict(T=-1), moe.MOE_ERR_ARG),
    (dict(dtype="bf16", d=100), moe.MOE_ERR_UNSUPPORTED),
])
def test_route_rejects_bad_shapes(kw, code):
    assert _route(_cfg(**kw)) == code
    assert moe.lib().moe_last_error().decode().startswith("moe_route")


@host_only
def test_route_rejects_null_and_misaligned():
    assert _route(_cfg(), centroids=0) == moe.MOE_ERR_ARG
    assert _route(_cfg(), idx=FAKE + 4) == moe.MOE_ERR_ARG
    # scores == NULL needs a workspace of T*N*4 bytes
    assert _route(_cfg(), scores=0) == moe.MOE_ERR_ARG
    L = moe.lib()
    P = ctypes.c_void_p
    c = _cfg()
    rc = L.moe_route(ctypes.byref(c), P(FAKE), P(FAKE), P(FAKE), None, P(FAKE), P(FAKE),
                     P(FAKE), P(FAKE), 16, None)
    assert rc == moe.MOE_ERR_WORKSPACE
    assert moe.moe_route_workspace_size(c) == 64 * 16 * 4


@host_only
def test_fp8_requires_bf16_and_multiples_of_128():
    L = moe.lib()
    P = ctypes.c_void_p
    c = _cfg(fp8=True)  # fp32 activations + FP8
    rc = L.moe_expert_ffn(ctypes.byref(c), *([P(FAKE)] * 15), P(FAKE), 1 << 30, None)
    assert rc == moe.MOE_ERR_UNSUPPORTED
    c = _cfg(dtype="bf16", fp8=True, I=96)
    rc = L.moe_expert_ffn(ctypes.byref(c), *([P(FAKE)] * 15), P(FAKE), 1 << 30, None)
    assert rc == moe.MOE_ERR_UNSUPPORTED


@host_only
def test_workspace_checks():
    L = moe.lib()
    P = ctypes.c_void_p
    c = _cfg(dtype="bf16", d=256, I=128, Is=128)
    need = moe.moe_permute_workspace_size(c)
    assert need > 0
    rc = L.moe_permute(ctypes.byref(c), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE),
                       None, None, None, P(FAKE), need - 1, None)
    assert rc == moe.MOE_ERR_WORKSPACE
    need = moe.moe_expert_ffn_workspace_size(c)
    rc = L.moe_expert_ffn(ctypes.byref(c), *([P(FAKE)] * 15), P(FAKE), need - 1, None)
    assert rc == moe.MOE_ERR_WORKSPACE


@host_only
def test_combine_rejects_aliasing():
    L = moe.lib()
    P = ctypes.c_void_p
    c = _cfg()
    rc = L.moe_combine(ctypes.byref(c), P(FAKE), P(FAKE * 2), P(FAKE * 3), P(FAKE * 4),
                       P(FAKE * 5), P(FAKE), None)
    assert rc == moe.MOE_ERR_ARG


@host_only
def test_bias_update_and_quantize_validation():
    L = moe.lib()
    P = ctypes.c_void_p
    assert L.moe_bias_update(0, 10, P(FAKE), ctypes.c_float(0.001), P(FAKE), None) == \
        moe.MOE_ERR_ARG
    assert L.moe_bias_update(8, 10, None, ctypes.c_float(0.001), P(FAKE), None) == \
        moe.MOE_ERR_ARG
    assert L.moe_bias_update(8, 10, P(FAKE), ctypes.c_float(float("nan")), P(FAKE), None) == \
        moe.MOE_ERR_ARG
    assert L.moe_quantize_weights_fp8(1, 100, 128, P(FAKE), P(FAKE), P(FAKE), None) == \
        moe.MOE_ERR_ARG
