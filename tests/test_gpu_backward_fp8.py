"""GPU parity of the FP8 backward: libmoe's backward calls for an FP8 layer
(moe_expert_ffn_backward_fp8 for the experts, through the C ABI) against the
oracle's FP8 backward, step by step.

Each step of the expert FFN backward is compared with the oracle's step fed
the GPU's own inputs (read from the backward's workspace through
moe_expert_ffn_backward_fp8_offsets): every E4M3 code and tile scale bit for
bit (dY in 1x128 row tiles, [da db] in 1x128 row tiles, and the 128x1
row-direction tiles of dY, h, [da db] and the gathered x), the recomputed a, b
and h at the bf16 rule, dh, dX, dW2 and dW13 at the plain FP8 rule (6e-2 of the
row's RMS, elementwise within 2 of it), [da db] at the bf16 rule.  The
combine, gate, logit, centroid and input gradients are checked the same way
against the oracle's bf16 steps.

Beside that contract, each gradient is compared with the fully independent
oracle (its own quantisation of its own intermediates) norm-wise within 6e-2:
both sides re-quantise intermediates (h, [da db], the row-direction tiles)
from values that differ in their last bits (MFMA summation order against exact
sums), so single codes at rounding midpoints can differ, and elementwise bounds
on the end results would then measure that, not the kernels.
"""
import numpy as np
import pytest
import torch

import moe_inputs
import sparse_moe_layer_bias_amd as moe
from parity_util import (RTOL, ExpertCodes, RowsOf, assert_bits, check_fp8_backward_split,
                         assert_close, guard_grads, guard_layer, host_inputs, log, row_rel_l2,
                         small_layer_inputs, to_f64)
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
    layer.test_fwd, layer.test_host, layer.test_dout_host = fwd, h, moe_inputs.to_host(dout)
    return c, layer, g, ref


def _check_steps(orc, layer, g, ref, residual=True):
    """Every backward step against the oracle's step fed the GPU's own inputs
    (expert FFN: check_fp8_backward_split; combine, gate/logit, centroid and
    input gradients: the oracle's bf16 steps), at the plain rules; then, beside
    the contract, each gradient against the fully independent oracle,
    norm-wise within 6e-2 (both sides quantise intermediates that differ in
    their last bits, so single codes at rounding midpoints can differ)."""
    fwd, h, dout = layer.test_fwd, layer.test_host, layer.test_dout_host
    T = layer.c["T"]
    check_fp8_backward_split(orc, layer, fwd, h["x"], dout)
    H = moe_inputs.to_host
    gate, idx, dst = H(layer.gate), H(layer.idx), H(layer.dst_row)
    assert_bits(gate, fwd["gate"], "gate")
    assert_bits(dst, fwd["dst_row"], "dst_row")
    dyp, dg = orc.combine_backward(dout, H(layer.y_perm), gate, dst)
    assert_close(H(g["dy_perm"]), dyp, RTOL["bf16"], "dy_perm")
    assert_close(H(g["dgate"]), dg, RTOL["bf16"], "dgate")
    dz = orc.route_backward(H(layer.scores), idx, H(g["dgate"]))
    assert_close(H(g["dz"]), dz, RTOL["bf16"], "dz")
    dE = orc.centroid_grad(h["x"], idx, H(g["dz"]), layer.c["N"])
    assert_close(H(g["dcentroids"]), dE, RTOL["bf16"], "dcentroids")
    dx = orc.input_grad(dout if residual else None, H(g["dx_shared"]), H(g["dx_perm"]), dst,
                        H(g["dz"]), idx, h["centroids"])
    assert_close(H(g["dx"]), dx, RTOL["bf16"], "dx")
    for n in ("dx_perm", "dx_shared", "dx"):
        l2 = row_rel_l2(H(g[n]), ref[n])
        assert np.all(l2 <= RTOL["fp8"]), "%s vs independent oracle: row L2 %.3g" % (n, l2.max())
    for n in ("dw13", "dw2", "dws13", "dws2"):
        a, b = to_f64(H(g[n])), to_f64(ref[n])
        a3, b3 = a.reshape((-1,) + a.shape[-2:]), b.reshape((-1,) + b.shape[-2:])
        for i in range(a3.shape[0]):
            nr, ne = np.linalg.norm(b3[i]), np.linalg.norm(a3[i] - b3[i])
            assert ne <= RTOL["fp8"] * nr or (nr == 0 and ne == 0), "%s[%d] L2 %.3g" % (
                n, i, ne / max(nr, 1e-300))


FP8_CASES = [
    dict(T=128),
    dict(T=77),                                          # experts without rows
    dict(T=1),
    dict(T=700, d=384, N=2, k=1, I=256, Is=128),         # several 128-row blocks and row tiles
    dict(T=64, d=256, I=128, Is=256),                    # Is != I
    dict(T=300, G=8, TG=3),                              # group-limited routing
    # one expert with exactly T rows: a full 128-row block, one more row, and
    # a second 320-row forward tile of one row
    dict(T=128, N=1, k=1, d=256, I=256, Is=128),
    dict(T=129, N=1, k=1, d=256, I=256, Is=128),
    dict(T=321, N=1, k=1, d=256, I=256, Is=128),
]


@pytest.mark.parametrize("over", FP8_CASES)
def test_fp8_backward_parity_small(orc, over):
    c, layer, g, ref = _run(orc, **dict(over))
    assert np.array_equal(moe_inputs.to_host(layer.idx), ref["idx"])
    _check_steps(orc, layer, g, ref)


@pytest.mark.parametrize("over", [dict(T=77), dict(T=700, d=384, N=2, k=1, I=256, Is=128)])
def test_fp8_backward_parity_recompute(orc, over):
    """Without kept activations the backward recomputes a, b, h on FP8."""
    c, layer, g, ref = _run(orc, save=False, **dict(over))
    _check_steps(orc, layer, g, ref)


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
    _check_steps(orc, layer, g, ref, residual=False)
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


@pytest.mark.timeout(900)
def test_v3_fp8_backward_one_expert(orc):
    """DeepSeek-V3-shaped FP8 layer, the launches the benchmark times: every
    backward step of the least-loaded expert against the oracle's steps fed
    the GPU's own inputs (bytes bit for bit, values at the plain rules), and
    its gradients against the fully independent oracle norm-wise; an expert
    without rows gets zero weight gradients."""
    cfg = dict(moe_inputs.CONFIGS["v3_fp8"])
    T, N, k, d = cfg["T"], cfg["N"], cfg["k"], cfg["d"]
    log("generating V3-shaped FP8 inputs on the GPU")
    dev = moe_inputs.make_layer_inputs(cfg, 0, "cuda")
    dout = moe_inputs.make_upstream_grad(cfg, 0, "cuda")
    layer = MoeLayer(cfg, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"], train=True)
    bias0 = dev["bias"].clone()
    layer.forward(dev["x"], dev["centroids"], dev["bias"].clone())
    g = layer.backward(dout, dev["x"], dev["centroids"])
    torch.cuda.synchronize()
    log("V3 FP8 backward done")
    xh = moe_inputs.to_host(dev["x"])
    r = orc.route(xh, moe_inputs.to_host(dev["centroids"]), moe_inputs.to_host(bias0), k,
                  cfg["G"], cfg["TG"])
    off, src, dst = orc.permute(r["idx"], N)
    assert_bits(moe_inputs.to_host(layer.offsets), off, "offsets")
    xq, xs = orc.quant_act_fp8(xh)
    fwd = dict(offsets=off, src_token=src, x_q_perm=RowsOf(xq, src), x_s_perm=RowsOf(xs, src),
               x_q=xq, x_s=xs, w13_q=ExpertCodes(orc, dev["w13"], 0),
               w13_s=ExpertCodes(orc, dev["w13"], 1), w2_q=ExpertCodes(orc, dev["w2"], 0),
               w2_s=ExpertCodes(orc, dev["w2"], 1))
    counts = np.diff(off.astype(np.int64))
    e = int(np.argmin(np.where(counts > 0, counts, 1 << 30)))
    log("step checks of expert", e, "with", int(counts[e]), "rows")
    check_fp8_backward_split(orc, layer, fwd, xh, None, what="V3 FP8: ", groups=[e])
    a, b = int(off[e]), int(off[e + 1])
    dy = moe_inputs.to_host(g["dy_perm"][a:b])
    q13, s13 = orc.quant_weight_fp8(moe_inputs.to_host(dev["w13"][e]))
    q2, s2 = orc.quant_weight_fp8(moe_inputs.to_host(dev["w2"][e]))
    dA, dw13, dw2 = orc.swiglu_ffn_backward_fp8(xq[src[a:b]], xs[src[a:b]], xh[src[a:b]], q13,
                                                s13, q2, s2, dy)
    l2 = row_rel_l2(moe_inputs.to_host(g["dx_perm"][a:b]), dA)
    assert np.all(l2 <= RTOL["fp8"]), "dx_perm vs independent oracle: row L2 %.3g" % l2.max()
    for n, ref in (("dw13", dw13), ("dw2", dw2)):
        got = to_f64(moe_inputs.to_host(g[n][e]))
        ne, nr = np.linalg.norm(got - to_f64(ref)), np.linalg.norm(to_f64(ref))
        assert ne <= RTOL["fp8"] * nr, "%s of expert %d: L2 %.3g" % (n, e, ne / nr)
    # an expert without rows gets zeros
    if np.any(counts == 0):
        z = int(np.nonzero(counts == 0)[0][0])
        assert not torch.any(g["dw13"][z]) and not torch.any(g["dw2"][z])
