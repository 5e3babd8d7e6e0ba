"""GPU parity of moe_route alone (through the C ABI) against the oracle, on
shapes that reach every instance of the router's logits kernels, and on rows
whose keys are NaN.

The launcher picks the logits kernel by batch size (a serial fp32 chain per
(token, expert) pair, so the tile per thread trades chains against
workgroups): one chain per lane when cdiv(N,64)*cdiv(T,64) < 64, the
matrix-core kernel (one contraction-1 MFMA per k) from 384 64x64 tiles on
(128-token tiles while they still number 256 or more),
else 2 or 1 token(s) per thread (TY) on the VALU by the number of workgroups
each gives; FULL instances need d % 32 == 0 (tiled) or d % 256 == 0 (one
chain per lane), the others pad the last stage.  Scores, indices, gates and
counts must match bit for bit.
"""
import numpy as np
import pytest
import torch

import moe_inputs
import sparse_moe_layer_bias_amd as moe
from parity_util import Guards, assert_bits, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the parity tests need the HIP library on an MI355X")
    moe.lib()
    yield
    torch.cuda.synchronize()


def _route_inputs(T, d, N, dtype, seed):
    cfg = dict(T=T, d=d, N=N, dtype=dtype, bias_std=1e-3)
    return moe_inputs.make_router_inputs(cfg, seed, "cpu")


def _route_gpu(T, d, N, k, G, TG, dtype, inp):
    c = moe.make_cfg(T, d, N, k, G, TG, 0, 0, dtype)
    dev = {n: v.cuda() for n, v in inp.items()}
    g = Guards()
    scores = g.empty((T, N), torch.float32, "scores")
    idx = g.empty((T, k), torch.int32, "idx")
    gate = g.empty((T, k), torch.float32, "gate")
    counts = g.empty((N,), torch.int32, "counts")
    moe.moe_route(c, dev["x"], dev["centroids"], dev["bias"], scores, idx, gate, counts)
    torch.cuda.synchronize()
    g.check()
    return {n: moe_inputs.to_host(v) for n, v in
            dict(scores=scores, idx=idx, gate=gate, counts=counts).items()}


# (T, d, N, k, G, TG, dtype): the logits kernel each reaches
ROUTE_CASES = [
    (1024, 7168, 256, 8, 8, 4, "bf16"),   # tiled, 1 token per thread
    (2048, 7168, 256, 8, 8, 4, "bf16"),   # tiled, 2 tokens per thread
    (8192, 7176, 256, 8, 8, 4, "bf16"),   # matrix cores, 128-token tile, d % 32 != 0
    (6200, 512, 250, 8, 1, 1, "bf16"),    # matrix cores, 64-token tile, ragged tokens and experts
    (2048, 1000, 256, 8, 1, 1, "bf16"),   # tiled, 2 tokens per thread, d % 32 != 0
    (1024, 1000, 256, 6, 1, 1, "bf16"),   # tiled, 1 token per thread, d % 32 != 0
    (4096, 1000, 64, 8, 1, 1, "f32"),     # fp32 x: tiled, 1 token per thread, d % 32 != 0
    (8192, 512, 64, 8, 1, 1, "f32"),      # fp32 x: tiled, 2 tokens per thread
    (32768, 256, 64, 4, 1, 1, "f32"),     # fp32 x: matrix cores, 128-token tile
    (32768, 1000, 64, 4, 1, 1, "f32"),    # fp32 x: matrix cores, 128-token tile, d % 32 != 0
    (24576, 1000, 64, 8, 1, 1, "f32"),    # fp32 x: matrix cores, 64-token tile, d % 32 != 0
    (24576, 512, 64, 8, 1, 1, "f32"),     # fp32 x: matrix cores, 64-token tile
    (128, 1000, 256, 8, 1, 1, "bf16"),    # one chain per lane, d % 256 != 0
    (100, 7168, 256, 8, 8, 4, "bf16"),    # one chain per lane, ragged tokens
]


@pytest.mark.parametrize("T,d,N,k,G,TG,dtype", ROUTE_CASES)
def test_route_kernel_instances(orc, T, d, N, k, G, TG, dtype):
    log("route case T=%d d=%d N=%d k=%d G=%d TG=%d %s" % (T, d, N, k, G, TG, dtype))
    inp = _route_inputs(T, d, N, dtype, seed=T + d)
    got = _route_gpu(T, d, N, k, G, TG, dtype, inp)
    h = {n: moe_inputs.to_host(v) for n, v in inp.items()}
    r = orc.route(h["x"], h["centroids"], h["bias"], k, G, TG, want_scores=True)
    for n in ("scores", "idx", "gate", "counts"):
        assert_bits(got[n], r[n], n)


def _bits_nan_aware(got, ref, what):
    """equal bits where the oracle's value is a number; NaN where it is NaN
    (NaN payloads and signs are not part of the reading)"""
    g, r = np.asarray(got), np.asarray(ref)
    nan = np.isnan(r)
    assert np.array_equal(np.isnan(g), nan), what + ": NaN positions differ"
    assert_bits(g[~nan], r[~nan], what)


@pytest.mark.parametrize("T,d,N,G,TG", [(256, 1024, 64, 1, 1), (256, 1024, 64, 8, 3),
                                        (8192, 512, 256, 8, 3)])  # the last on the matrix cores
def test_nan_rows_route_to_valid_experts(orc, T, d, N, G, TG):
    """Rows of x holding NaN or inf give NaN (or extreme) scores; every token
    must still get k distinct experts in [0, N), counts must sum to T*k, and
    idx must equal the oracle's (a NaN key ranks as -inf, lower index first)."""
    k = 6
    inp = _route_inputs(T, d, N, "bf16", seed=41)
    x = inp["x"]
    x[5, :] = float("nan")
    x[9, 3] = float("nan")
    x[17, 100] = float("inf")
    x[18, 7] = float("-inf")
    x[20, 1] = float("inf")
    x[20, 2] = float("-inf")
    got = _route_gpu(T, d, N, k, G, TG, "bf16", inp)
    h = {n: moe_inputs.to_host(v) for n, v in inp.items()}
    r = orc.route(h["x"], h["centroids"], h["bias"], k, G, TG, want_scores=True)
    idx = got["idx"]
    assert idx.min() >= 0 and idx.max() < N
    assert all(len(set(row)) == k for row in idx)
    assert int(got["counts"].sum()) == T * k
    assert np.isnan(r["scores"][5]).all() and np.isnan(r["scores"][9]).all()
    assert_bits(idx, r["idx"], "idx")
    assert_bits(got["counts"], r["counts"], "counts")
    _bits_nan_aware(got["scores"], r["scores"], "scores")
    _bits_nan_aware(got["gate"], r["gate"], "gate")


# (N, G, TG, k): group sizes gs = N / G that the select kernel reduces as
# aligned lane blocks (powers of two up to 64) and ones it reduces group by
# group (gs = 25, 128); N up to 1024 reaches every keys-per-lane instance
GROUP_CASES = [
    (128, 64, 16, 8),    # gs 2
    (256, 64, 8, 8),     # gs 4
    (64, 8, 3, 6),       # gs 8
    (256, 16, 4, 8),     # gs 16
    (96, 3, 2, 8),       # gs 32
    (192, 3, 2, 6),      # gs 64
    (256, 2, 1, 8),      # gs 128: group by group
    (100, 4, 2, 8),      # gs 25: group by group
    (512, 8, 4, 8),      # gs 64, 8 keys per lane
    (1024, 64, 8, 8),    # gs 16, 16 keys per lane
]


@pytest.mark.parametrize("N,G,TG,k", GROUP_CASES)
def test_group_limited_select(orc, N, G, TG, k):
    T, d = 300, 256
    log("group select case N=%d G=%d TG=%d k=%d" % (N, G, TG, k))
    inp = _route_inputs(T, d, N, "bf16", seed=N + G)
    got = _route_gpu(T, d, N, k, G, TG, "bf16", inp)
    h = {n: moe_inputs.to_host(v) for n, v in inp.items()}
    r = orc.route(h["x"], h["centroids"], h["bias"], k, G, TG, want_scores=True)
    for n in ("scores", "idx", "gate", "counts"):
        assert_bits(got[n], r[n], n)


@pytest.mark.parametrize("G,TG", [(1, 1), (8, 3), (4, 2)])
def test_select_ties_go_to_lower_indices(orc, G, TG):
    """x = 0 gives every score Sigmoid(0) = 0.5 exactly; a bias with three
    distinct values makes keys and group scores tie in many places, so every
    choice is decided by the lower index (expert, then group)."""
    T, d, N, k = 128, 256, 64, 8
    inp = _route_inputs(T, d, N, "bf16", seed=5)
    inp["x"].zero_()
    inp["bias"].copy_(torch.tensor([(i % 3) * 0.25 for i in range(N)], dtype=torch.float32))
    got = _route_gpu(T, d, N, k, G, TG, "bf16", inp)
    h = {n: moe_inputs.to_host(v) for n, v in inp.items()}
    r = orc.route(h["x"], h["centroids"], h["bias"], k, G, TG, want_scores=True)
    assert np.all(got["scores"] == 0.5)
    for n in ("idx", "gate", "counts"):
        assert_bits(got[n], r[n], n)
