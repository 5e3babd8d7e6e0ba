"""GPU parity of the FP8 backward: libmoe's backward calls for an FP8 layer
(moe_expert_ffn_backward_fp8 for the experts, through the C ABI) against the
oracle's FP8 backward on the same seeded inputs and upstream gradient.

Tolerance: the FP8 criterion of parity_util.assert_close_fp8_bwd (rtol 6e-2),
with the elementwise bound at 3 rtol instead of 2.  Both sides re-quantise
intermediate tensors (h, [da db], the row-direction tiles) from values that
differ in their last bits (MFMA summation order against exact sums), so a code
at a rounding midpoint can legitimately differ.  One code step is 2^-3 of its
value; a weight gradient of an expert with M rows is a sum of M such terms, and
at the small sizes here (10-30 rows per expert) one term can be ~4x the typical
one, so a single differing code moves an element by up to ~0.125 * 4 / sqrt(M)
~ 0.15 of its row's RMS.  The whole tensors agree to ~0.3% (relative L2), and
both sides are ~5% from the exact gradient of the dequantised operands.  The
weight gradients take the larger of the row's and the expert matrix's RMS as
an element's scale (parity_util.assert_close_fp8_grad): with one token an
expert's dW13 row is da[n] times x, and da[n] can be a near-cancelling sum.
"""
import numpy as np
import pytest
import torch

import moe_inputs
import sparse_moe_layer_bias_amd as moe
from parity_util import (assert_close_fp8_bwd, assert_close_fp8_grad, guard_grads, guard_layer,
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


def _run(orc, seed=0, residual=True, save=True, **over):
    cfg = dict(moe_inputs.CONFIGS["mid_bf16"], fp8=True)
    T = over.pop("T", None)
    cfg.update(over)
    c, inp, dev = small_layer_inputs(cfg, seed, T)
    log("fp8 backward case T=%d" % c["T"], over, "seed", seed, "residual", residual,
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
    layer.test_dout, layer.test_x, layer.test_centroids = dout.cuda(), dev["x"], dev["centroids"]
    h = host_inputs(inp)
    fwd = orc.layer_forward(h, c, residual=residual)
    ref = orc.layer_backward(h, c, fwd, moe_inputs.to_host(dout), residual=residual)
    ref["idx"] = fwd["idx"]
    return c, layer, g, ref


FP8_CASES = [
    dict(T=128),
    dict(T=77),                                          # experts without rows
    dict(T=1),
    dict(T=700, d=384, N=2, k=1, I=256, Is=128),         # several 128-row blocks and row tiles
    dict(T=64, d=256, I=128, Is=256),                    # Is != I
    dict(T=300, G=8, TG=3),                              # group-limited routing
]


@pytest.mark.parametrize("over", FP8_CASES)
def test_fp8_backward_parity_small(orc, over):
    c, layer, g, ref = _run(orc, **dict(over))
    assert np.array_equal(moe_inputs.to_host(layer.idx), ref["idx"])
    for n in ("dy_perm", "dx_perm", "dx_shared", "dz", "dcentroids", "dx"):
        assert_close_fp8_bwd(moe_inputs.to_host(g[n]), ref[n], n, elem=3.0)
    for n in ("dw13", "dw2", "dws13", "dws2"):
        assert_close_fp8_grad(moe_inputs.to_host(g[n]), ref[n], n)


@pytest.mark.parametrize("over", [dict(T=77), dict(T=700, d=384, N=2, k=1, I=256, Is=128)])
def test_fp8_backward_parity_recompute(orc, over):
    """Without kept activations the backward recomputes a, b, h on FP8."""
    c, layer, g, ref = _run(orc, save=False, **dict(over))
    for n in ("dx_perm", "dx_shared", "dx"):
        assert_close_fp8_bwd(moe_inputs.to_host(g[n]), ref[n], n, elem=3.0)
    for n in ("dw13", "dw2", "dws13", "dws2"):
        assert_close_fp8_grad(moe_inputs.to_host(g[n]), ref[n], n)


@pytest.mark.parametrize("T", [1, 300])
def test_fp8_training_forward_is_bitwise_the_inference_forward(T):
    cfg = dict(moe_inputs.CONFIGS["mid_bf16"], fp8=True)
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


def test_fp8_backward_without_residual_and_deterministic(orc):
    c, layer, g, ref = _run(orc, seed=3, residual=False, T=96)
    assert_close_fp8_bwd(moe_inputs.to_host(g["dx"]), ref["dx"], "dx", elem=3.0)
    first = {n: moe_inputs.to_host(g[n]).copy() for n in ("dx", "dw13", "dw2", "dws13", "dws2")}
    layer.backward(layer.test_dout, layer.test_x, layer.test_centroids, residual=False)
    torch.cuda.synchronize()
    for n, v in first.items():
        assert np.array_equal(moe_inputs.to_host(g[n]).view(np.uint8), v.view(np.uint8)), n


def test_fp8_transposed_packs_are_the_transposed_codes():
    """moe_pack_weights which = 5 of the codes equals which = 1 of the
    transposed codes (the same packing of the same matrix, built two ways)."""
    from sparse_moe_layer_bias_amd.layer import pack_weights, quantize_weights_fp8
    cfg = dict(moe_inputs.CONFIGS["mid_bf16"], T=64, fp8=True, d=256, I=384, N=4, k=2)
    c, inp, dev = small_layer_inputs(cfg, 5)
    layer = MoeLayer(c, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"], train=True)
    q2, _ = quantize_weights_fp8(dev["w2"])                  # [N, d, I]
    c_t = moe.cfg_from_dict(dict(c, d=c["I"], I=c["d"]))     # roles of d and I swapped
    direct = pack_weights(c_t, 1, q2.transpose(1, 2).contiguous())
    torch.cuda.synchronize()
    assert torch.equal(layer.w2t, direct)


def test_v3_fp8_backward_one_expert_and_sampled_tokens(orc):
    """DeepSeek-V3-shaped FP8 layer, the launches the benchmark times: the
    full weight gradients and row gradients of the least-loaded expert, and the
    shared expert's input gradient of sampled tokens, against the oracle."""
    cfg = dict(moe_inputs.CONFIGS["v3_fp8"])
    T, N, k, d = cfg["T"], cfg["N"], cfg["k"], cfg["d"]
    log("generating V3-shaped FP8 inputs on the GPU")
    dev = moe_inputs.make_layer_inputs(cfg, 0, "cuda")
    dout = moe_inputs.make_upstream_grad(cfg, 0, "cuda")
    layer = MoeLayer(cfg, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"], train=True)
    layer.forward(dev["x"], dev["centroids"], dev["bias"].clone())
    g = layer.backward(dout, dev["x"], dev["centroids"])
    torch.cuda.synchronize()
    log("V3 FP8 backward done")
    off = moe_inputs.to_host(layer.offsets).astype(np.int64)
    counts = np.diff(off)
    e = int(np.argmin(np.where(counts > 0, counts, 1 << 30)))
    a, b = int(off[e]), int(off[e + 1])
    src = moe_inputs.to_host(layer.src_token)[a:b]
    xh = moe_inputs.to_host(dev["x"])
    xq = moe_inputs.to_host(layer.x_perm[a:b])
    xs = moe_inputs.to_host(layer.x_perm_s[a:b])
    assert np.array_equal(xq, orc.quant_act_fp8(xh[src])[0])   # the forward's tiles
    dy = moe_inputs.to_host(g["dy_perm"][a:b])
    q13, s13 = orc.quant_weight_fp8(moe_inputs.to_host(dev["w13"][e]))
    q2, s2 = orc.quant_weight_fp8(moe_inputs.to_host(dev["w2"][e]))
    log("oracle FP8 backward of expert", e, "with", b - a, "rows")
    dA, dw13, dw2 = orc.swiglu_ffn_backward_fp8(xq, xs, xh[src], q13, s13, q2, s2, dy)
    assert_close_fp8_bwd(moe_inputs.to_host(g["dx_perm"][a:b]), dA, "dx_perm rows of expert %d" % e,
                     elem=3.0)
    assert_close_fp8_grad(moe_inputs.to_host(g["dw13"][e]), dw13, "dw13 of expert %d" % e)
    assert_close_fp8_grad(moe_inputs.to_host(g["dw2"][e]), dw2, "dw2 of expert %d" % e)
    # an expert without rows gets zeros
    if np.any(counts == 0):
        z = int(np.nonzero(counts == 0)[0][0])
        assert not torch.any(g["dw13"][z]) and not torch.any(g["dw2"][z])
