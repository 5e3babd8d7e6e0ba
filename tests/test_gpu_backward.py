"""GPU parity of the layer backward: libmoe's four backward calls (through the
C ABI) against the oracle's chain rule on the same seeded inputs and the same
seeded upstream gradient.  Each side runs its own forward first.

Tolerance: bf16 layers 2e-2 with the row rule of parity_util for every
gradient, including the fp32-typed ones (dgate, dz, dcentroids): those are
sums over bf16 intermediates (y_perm) that the two sides round independently.
fp32 layers 1e-5 against the RMS of the whole tensor (assert_close_tensor: the
gradients are cancelling sums whose fp32 error scales with their terms).
"""
import numpy as np
import pytest
import torch

import moe_inputs
import sparse_moe_layer_bias_amd as moe
from parity_util import (RTOL, assert_close, assert_close_tensor, guard_grads, guard_layer,
                         host_inputs, log, small_layer_inputs)
from sparse_moe_layer_bias_amd.layer import MoeLayer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the parity tests need the HIP library on an MI355X")
    moe.lib()
    yield
    torch.cuda.synchronize()


def _run(name, orc, seed=0, residual=True, save=True, **over):
    cfg = dict(moe_inputs.CONFIGS[name])
    T = over.pop("T", None)
    cfg.update(over)
    c, inp, dev = small_layer_inputs(cfg, seed, T)
    log("backward case", name, "T=%d" % c["T"], over, "seed", seed, "residual", residual,
        "saved activations" if save else "recompute")
    dout = moe_inputs.make_upstream_grad(c, seed, "cpu")
    layer = MoeLayer(c, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"], train=True,
                     save_activations=save)
    guards = guard_layer(layer)
    guard_grads(layer, dev["centroids"], guards)
    layer.forward(dev["x"], dev["centroids"], dev["bias"].clone(), residual=residual)
    g = layer.backward(dout.cuda(), dev["x"], dev["centroids"], residual=residual)
    torch.cuda.synchronize()
    guards.check()
    h = host_inputs(inp)
    fwd = orc.layer_forward(h, c, residual=residual)
    ref = orc.layer_backward(h, c, fwd, moe_inputs.to_host(dout), residual=residual)
    return c, layer, g, ref


def _cmp(g, ref, names, dtype):
    for n in names:
        if ref[n] is None:
            assert g[n] is None, n
            continue
        if dtype == "bf16":
            assert_close(moe_inputs.to_host(g[n]), ref[n], RTOL["bf16"], n)
        else:
            assert_close_tensor(moe_inputs.to_host(g[n]), ref[n], RTOL["f32"], n)


BWD_CASES = [
    ("tiny_fp32", {}),
    ("tiny_fp32", dict(T=1)),
    ("tiny_fp32", dict(T=200, I=72, Is=40)),             # ragged, I not a multiple of 8
    ("mid_bf16", dict(T=256)),
    ("mid_bf16", dict(T=77)),                            # ragged rows, experts without rows
    ("mid_bf16", dict(T=1)),
    ("mid_bf16", dict(T=300, G=8, TG=3)),                # group-limited
    ("mid_bf16", dict(T=64, d=256, I=128, Is=256)),      # Is != I
    ("mid_bf16", dict(T=64, d=256, I=256, Is=128)),
    ("mid_bf16", dict(T=700, d=384, N=2, k=1, I=256, Is=128)),  # several 128-row tiles per expert
    ("mid_bf16", dict(T=130, N=1, k=1)),                 # one expert: gate 1, dz = 0
    ("mid_bf16", dict(T=50, N=16, k=16)),                # k = N
    # one expert with exactly T rows: the weight gradients' 32-row stages and
    # the data gradients' 320-row tiles, at and just past an edge
    ("mid_bf16", dict(T=32, N=1, k=1, d=256, I=256, Is=128)),
    ("mid_bf16", dict(T=33, N=1, k=1, d=256, I=256, Is=128)),
    ("mid_bf16", dict(T=321, N=1, k=1, d=256, I=256, Is=128)),
]


@pytest.mark.parametrize("name,over", BWD_CASES)
def test_backward_parity_small(orc, name, over):
    c, layer, g, ref = _run(name, orc, **dict(over))
    _cmp(g, ref, ("dy_perm", "dgate", "dz", "dcentroids", "dx_perm", "dx_shared", "dw13", "dw2",
                  "dws13", "dws2", "dx"), c["dtype"])


RECOMPUTE_CASES = [
    ("tiny_fp32", {}),
    ("mid_bf16", dict(T=77)),
    ("mid_bf16", dict(T=700, d=384, N=2, k=1, I=256, Is=128)),
    ("mid_bf16", dict(T=64, d=256, I=256, Is=128)),
]


@pytest.mark.parametrize("name,over", RECOMPUTE_CASES)
def test_backward_parity_recompute(orc, name, over):
    """Without saved activations the backward recomputes a, b and h."""
    c, layer, g, ref = _run(name, orc, save=False, **dict(over))
    _cmp(g, ref, ("dx_perm", "dx_shared", "dw13", "dw2", "dws13", "dws2", "dx"), c["dtype"])


@pytest.mark.parametrize("name,T", [("tiny_fp32", 200), ("mid_bf16", 300)])
def test_training_forward_is_bitwise_the_inference_forward(name, T):
    cfg = dict(moe_inputs.CONFIGS[name])
    c, inp, dev = small_layer_inputs(cfg, 9, T)
    outs = []
    for train in (False, True):
        layer = MoeLayer(c, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"], train=train)
        o = layer.forward(dev["x"], dev["centroids"], dev["bias"].clone()).clone()
        torch.cuda.synchronize()
        outs.append((moe_inputs.to_host(o), moe_inputs.to_host(layer.y_perm),
                     moe_inputs.to_host(layer.y_shared)))
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_backward_without_residual(orc):
    c, layer, g, ref = _run("mid_bf16", orc, seed=2, residual=False, T=96)
    _cmp(g, ref, ("dx",), "bf16")
    c, layer, g, ref = _run("tiny_fp32", orc, seed=2, residual=False, T=50)
    _cmp(g, ref, ("dx",), "f32")


def test_backward_deterministic_bytes(orc):
    cfg = dict(moe_inputs.CONFIGS["mid_bf16"])
    c, inp, dev = small_layer_inputs(cfg, 4, 300)
    dout = moe_inputs.make_upstream_grad(c, 4, "cuda")
    runs = []
    for _ in range(2):
        layer = MoeLayer(c, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"], train=True)
        layer.forward(dev["x"], dev["centroids"], dev["bias"].clone())
        g = layer.backward(dout, dev["x"], dev["centroids"])
        torch.cuda.synchronize()
        runs.append({n: moe_inputs.to_host(g[n]).copy() for n in
                     ("dx", "dw13", "dw2", "dws13", "dws2", "dcentroids", "dz")})
    for n in runs[0]:
        assert np.array_equal(runs[0][n].view(np.uint8), runs[1][n].view(np.uint8)), n


def test_backward_zero_tokens_gives_zero_weight_gradients():
    cfg = dict(moe_inputs.CONFIGS["mid_bf16"])
    c, inp, dev = small_layer_inputs(cfg, 0, 1)
    c0 = dict(c, T=0)
    layer = MoeLayer(c0, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"], train=True)
    x = torch.empty((0, c["d"]), dtype=torch.bfloat16, device="cuda")
    layer.forward(x, dev["centroids"], dev["bias"].clone())
    g = layer.backward(torch.empty_like(x), x, dev["centroids"])
    torch.cuda.synchronize()
    assert not torch.any(g["dw13"]) and not torch.any(g["dw2"])
    assert not torch.any(g["dcentroids"])


# ------------------------------------------------------------------ V3 shape, sampled

def test_v3_backward_one_expert_and_sampled_tokens(orc):
    """DeepSeek-V3-shaped bf16 layer, the launches the benchmark times:
    one expert's full weight gradients and its rows' input gradients, and the
    shared expert's input gradient on sampled tokens, against the oracle."""
    cfg = dict(moe_inputs.CONFIGS["v3_bf16"])
    T, N, k, d = cfg["T"], cfg["N"], cfg["k"], cfg["d"]
    log("generating V3-shaped inputs on the GPU")
    dev = moe_inputs.make_layer_inputs(cfg, 0, "cuda")
    dout = moe_inputs.make_upstream_grad(cfg, 0, "cuda")
    layer = MoeLayer(cfg, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"], train=True)
    layer.forward(dev["x"], dev["centroids"], dev["bias"].clone())
    g = layer.backward(dout, dev["x"], dev["centroids"])
    torch.cuda.synchronize()
    log("V3 backward done; oracle routing of all tokens")
    xh = moe_inputs.to_host(dev["x"])
    r = orc.route(xh, moe_inputs.to_host(dev["centroids"]), moe_inputs.to_host(dev["bias"]),
                  k, cfg["G"], cfg["TG"])
    off, src, dst = orc.permute(r["idx"], N)
    counts = np.diff(off)
    e = int(np.argsort(counts)[N // 2])  # a median-loaded expert
    rows = np.arange(off[e], off[e + 1])
    toks = src[rows]
    slot = np.array([int(np.nonzero(r["idx"][t] == e)[0][0]) for t in toks])
    douth = moe_inputs.to_host(dout)
    # dy rows of expert e: gate * dout (combine backward on those rows alone)
    gsel = r["gate"][toks, slot][:, None]
    fake_dst = np.arange(len(toks), dtype=np.int32)[:, None]
    zeros = np.zeros((len(toks), d), np.uint16)
    dy_e, _ = orc.combine_backward(douth[toks], zeros, gsel.astype(np.float32), fake_dst)
    log("oracle backward of expert", e, "with", len(rows), "rows")
    dA, dw13, dw2 = orc.swiglu_ffn_backward(xh[toks], moe_inputs.to_host(dev["w13"][e]),
                                            moe_inputs.to_host(dev["w2"][e]), dy_e)
    rtol = RTOL["bf16"]
    assert_close(moe_inputs.to_host(g["dy_perm"][int(off[e]):int(off[e + 1])]), dy_e, rtol,
                 "dy_perm rows of expert %d" % e)
    assert_close(moe_inputs.to_host(g["dx_perm"][int(off[e]):int(off[e + 1])]), dA, rtol,
                 "dx_perm rows of expert %d" % e)
    assert_close(moe_inputs.to_host(g["dw13"][e]), dw13, rtol, "dw13 of expert %d" % e)
    assert_close(moe_inputs.to_host(g["dw2"][e]), dw2, rtol, "dw2 of expert %d" % e)
    # shared expert: input gradient of sampled tokens (one row at a time)
    tok = np.unique(np.concatenate([np.random.default_rng(5).choice(T, 6, replace=False),
                                    [0, T - 1]]))
    ws13 = moe_inputs.to_host(dev["ws13"])
    ws2 = moe_inputs.to_host(dev["ws2"])
    for t in tok:
        dxs, _, _ = orc.swiglu_ffn_backward(xh[t:t + 1], ws13, ws2, douth[t:t + 1])
        assert_close(moe_inputs.to_host(g["dx_shared"][int(t):int(t) + 1]), dxs, rtol,
                     "dx_shared token %d" % t)
