"""moe_permute_noalloc (include/moe.h): the permutation with its scratch in
the library's device-resident array instead of a caller workspace.  Through
the C ABI, its outputs must equal moe_permute's bit for bit, on two calls in a
row with the second on a smaller batch (the array keeps the first call's
contents), for bf16 rows and for FP8 codes and scales."""
import ctypes

import numpy as np
import pytest
import torch

import moe_inputs
import sparse_moe_layer_bias_amd as moe
from parity_util import Guards, assert_bits, log

pytestmark = pytest.mark.gpu


def _buffers(c, T, d, fp8):
    k, N = c["k"], c["N"]
    i32 = dict(dtype=torch.int32, device="cuda")
    b = dict(offsets=torch.full((N + 1,), -1, **i32), src_token=torch.full((T * k,), -1, **i32),
             dst_row=torch.full((T, k), -1, **i32))
    if fp8:
        b.update(x_perm=torch.zeros((T * k, d), dtype=torch.uint8, device="cuda"),
                 x_perm_scale=torch.zeros((T * k, d // 128), dtype=torch.float32, device="cuda"),
                 x_q=torch.zeros((T, d), dtype=torch.uint8, device="cuda"),
                 x_s=torch.zeros((T, d // 128), dtype=torch.float32, device="cuda"))
    else:
        b.update(x_perm=torch.zeros((T * k, d), dtype=torch.bfloat16, device="cuda"),
                 x_perm_scale=None, x_q=None, x_s=None)
    return b


def _routed(c, T, seed):
    cfg = moe.cfg_from_dict(c, T)
    inp = moe_inputs.make_router_inputs(dict(c, T=T), seed, "cuda")
    k, N = c["k"], c["N"]
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, k), dtype=torch.float32, device="cuda")
    counts = torch.empty((N,), dtype=torch.int32, device="cuda")
    scores = torch.empty((T, N), dtype=torch.float32, device="cuda")
    moe.moe_route(cfg, inp["x"], inp["centroids"], inp["bias"], scores, idx, gate, counts)
    return cfg, inp["x"], idx


@pytest.mark.parametrize("fp8", [False, True])
def test_permute_noalloc_matches_permute(fp8):
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    c = dict(moe_inputs.CONFIGS["mid_bf16"], G=8, TG=3, fp8=fp8)
    d = c["d"]
    for T, seed in ((2048, 1), (300, 2)):  # the second call is smaller
        log("noalloc permute fp8=%s T=%d" % (fp8, T))
        cfg, x, idx = _routed(c, T, seed)
        ref = _buffers(c, T, d, fp8)
        ws = torch.empty((moe.moe_permute_workspace_size(cfg),), dtype=torch.uint8,
                         device="cuda")
        moe.moe_permute(cfg, x, idx, ref["offsets"], ref["src_token"], ref["dst_row"],
                        ref["x_perm"], ref["x_perm_scale"], ref["x_q"], ref["x_s"], ws)
        got = _buffers(c, T, d, fp8)
        g = Guards()
        got = {n: g.like(v, n, copy=True) for n, v in got.items()}
        moe.moe_permute_noalloc(cfg, x, idx, got["offsets"], got["src_token"], got["dst_row"],
                                got["x_perm"], got["x_perm_scale"], got["x_q"], got["x_s"])
        torch.cuda.synchronize()
        g.check()
        for n in ref:
            if ref[n] is None:
                continue
            a, b = moe_inputs.to_host(got[n]), moe_inputs.to_host(ref[n])
            if a.dtype == np.float32:
                a, b = a.view(np.uint32), b.view(np.uint32)
            assert_bits(a, b, "%s (T=%d)" % (n, T))
        assert int(moe_inputs.to_host(got["offsets"])[-1]) == T * c["k"]


def test_permute_noalloc_rejects_oversize_shape():
    """A shape whose scratch exceeds the built-in array is rejected before
    anything is enqueued (no GPU work: validation fails first)."""
    big = moe.make_cfg(1 << 22, 1024, 256, 8, 1, 1, 512, 512, "bf16")
    assert moe.moe_permute_workspace_size(big) > moe.moe_permute_noalloc_max_bytes()
    P = ctypes.c_void_p
    FAKE = 1 << 20
    rc = moe.lib().moe_permute_noalloc(ctypes.byref(big), *([P(FAKE)] * 6), None, None, None,
                                       None)
    assert rc == moe.MOE_ERR_WORKSPACE
    assert b"scratch" in moe.lib().moe_last_error()
