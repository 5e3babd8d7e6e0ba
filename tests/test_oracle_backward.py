"""Pins for the oracle's backward pass of the layer.

The layer (DeepSeek-V3 report reading guide, xyznot.com/de, "Methode" item 2):
h'_t = u_t + FFN^(s)(u_t) + sum_i g_{i,t} FFN^(r)_i(u_t), s_{i,t} = sigmoid(u_t^T e_i),
g = the chosen s normalised over the chosen experts; the bias b_i only
changes which experts are chosen.  The oracle's backward is the chain rule of
that statement written out by hand (oracle/moe_oracle.c).  It is pinned here
to things it does not contain:
  - reverse-mode automatic differentiation (torch.autograd, float64) of a
    plain dense forward of the same statement, with the selection fixed;
  - central finite differences of the oracle's own (separately pinned)
    forward, along random directions, in every parameter group;
  - closed forms of the gate normalisation's derivative.
"""
import math

import numpy as np
import pytest
import torch

import moe_inputs

F32_CFG = dict(T=24, d=40, N=8, k=3, G=2, TG=1, I=24, Is=16, dtype="f32", fp8=False,
               bias_std=1e-2, w_std="fan_in")


def _inputs(cfg, seed=0):
    inp = moe_inputs.make_layer_inputs(cfg, seed)
    return {k: moe_inputs.to_host(v) for k, v in inp.items()}


def _f64(a):
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _autograd(inp, fwd, dout, residual=True):
    """float64 autograd of a dense forward with the oracle's selection fixed."""
    T = inp["x"].shape[0]
    idx = torch.from_numpy(fwd["idx"].astype(np.int64))
    k = idx.shape[1]
    leaves = {n: torch.tensor(_f64(inp[n]), requires_grad=True)
              for n in ("x", "centroids", "w13", "w2", "ws13", "ws2")}
    x, E = leaves["x"], leaves["centroids"]

    def ffn(A, w13, w2):
        I = w13.shape[0] // 2
        a = A @ w13[:I].T
        b = A @ w13[I:].T
        return (torch.nn.functional.silu(a) * b) @ w2.T

    s = torch.sigmoid(x @ E.T)
    sel = torch.gather(s, 1, idx)
    g = sel / sel.sum(dim=1, keepdim=True)
    out = ffn(x, leaves["ws13"], leaves["ws2"])
    if residual:
        out = out + x
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            y = ffn(x[t:t + 1], leaves["w13"][e], leaves["w2"][e])[0]
            out = out.index_add(0, torch.tensor([t]), (g[t, j] * y)[None])
    loss = (out * torch.tensor(_f64(dout))).sum()
    loss.backward()
    return {n: v.grad.numpy() for n, v in leaves.items()}


def _close(got, ref, rtol):
    got = _f64(np.asarray(got))
    scale = np.abs(ref).max()
    err = np.abs(got - ref).max()
    assert err <= rtol * scale, (err, scale)


def test_layer_backward_matches_autograd_f32(orc):
    cfg = F32_CFG
    inp = _inputs(cfg, 3)
    fwd = orc.layer_forward(inp, cfg)
    rng = np.random.default_rng(7)
    dout = rng.standard_normal(inp["x"].shape).astype(np.float32)
    got = orc.layer_backward(inp, cfg, fwd, dout)
    ref = _autograd(inp, fwd, dout)
    _close(got["dx"], ref["x"], 2e-5)
    _close(got["dcentroids"], ref["centroids"], 2e-5)
    _close(got["dw13"], ref["w13"], 2e-5)
    _close(got["dw2"], ref["w2"], 2e-5)
    _close(got["dws13"], ref["ws13"], 2e-5)
    _close(got["dws2"], ref["ws2"], 2e-5)
    # every expert that received rows has a non-zero gradient, the others none
    used = np.bincount(fwd["idx"].ravel(), minlength=cfg["N"]) > 0
    for e in range(cfg["N"]):
        assert np.any(got["dw2"][e] != 0) == used[e]
        assert np.any(got["dcentroids"][e] != 0) == used[e]


def test_layer_backward_without_residual_matches_autograd(orc):
    cfg = dict(F32_CFG, T=9, G=1, TG=1, k=2)
    inp = _inputs(cfg, 5)
    fwd = orc.layer_forward(inp, cfg, residual=False)
    dout = np.random.default_rng(8).standard_normal(inp["x"].shape).astype(np.float32)
    got = orc.layer_backward(inp, cfg, fwd, dout, residual=False)
    ref = _autograd(inp, fwd, dout, residual=False)
    _close(got["dx"], ref["x"], 2e-5)


def test_layer_backward_bf16_storage_close_to_autograd(orc):
    """bf16 storage: h, da, db and every output rounded to bf16; the result
    stays within the bf16 tolerance of the exact gradient of the same
    (bf16-valued) inputs."""
    cfg = dict(F32_CFG, dtype="bf16")
    inp = _inputs(cfg, 4)
    fwd = orc.layer_forward(inp, cfg)
    dout = orc.round_to_dtype(np.random.default_rng(9).standard_normal(inp["x"].shape),
                              "bf16")
    got = orc.layer_backward(inp, cfg, fwd, dout)
    ref = _autograd(inp, fwd, dout)
    for name, key in (("dx", "x"), ("dw13", "w13"), ("dw2", "w2"), ("dws13", "ws13"),
                      ("dws2", "ws2"), ("dcentroids", "centroids")):
        _close(got[name], ref[key], 2e-2)


def _loss(orc, inp, cfg, dout):
    fwd = orc.layer_forward(inp, cfg)
    return float((fwd["out"].astype(np.float64) * dout.astype(np.float64)).sum()), fwd["idx"]


@pytest.mark.parametrize("name,grad", [("x", "dx"), ("centroids", "dcentroids"),
                                       ("w13", "dw13"), ("w2", "dw2"), ("ws13", "dws13"),
                                       ("ws2", "dws2")])
def test_backward_matches_finite_differences_of_forward_oracle(orc, name, grad):
    """Directional derivative of L = sum(dout * out) from the oracle's forward
    (fp32 storage), central differences, against <V, grad L>."""
    cfg = F32_CFG
    inp = _inputs(cfg, 11)
    rng = np.random.default_rng(12)
    dout = rng.standard_normal(inp["x"].shape).astype(np.float32)
    fwd = orc.layer_forward(inp, cfg)
    g = orc.layer_backward(inp, cfg, fwd, dout)[grad].astype(np.float64)
    V = rng.standard_normal(inp[name].shape)
    eps = 1e-3 * np.abs(inp[name]).max()
    lp, ip = _loss(orc, dict(inp, **{name: (inp[name] + eps * V).astype(np.float32)}), cfg, dout)
    lm, im = _loss(orc, dict(inp, **{name: (inp[name] - eps * V).astype(np.float32)}), cfg, dout)
    # the selection must not move inside the difference
    assert np.array_equal(ip, fwd["idx"]) and np.array_equal(im, fwd["idx"])
    fd = (lp - lm) / (2 * eps)
    an = float((g * V).sum())
    assert abs(fd - an) <= 2e-3 * max(abs(an), 1e-3 * np.abs(g).sum()), (fd, an)


def test_bias_has_no_gradient_through_the_gates(orc):
    """A bias change that keeps the selection leaves the output unchanged."""
    cfg = F32_CFG
    inp = _inputs(cfg, 13)
    base = orc.layer_forward(inp, cfg)
    moved = orc.layer_forward(dict(inp, bias=inp["bias"] + np.float32(1e-6)), cfg)
    assert np.array_equal(base["idx"], moved["idx"])
    assert np.array_equal(base["out"], moved["out"])


# ------------------------------------------------------------------ gate normalisation

def test_uniform_gate_gradient_gives_zero_logit_gradient(orc):
    """The gates sum to 1, so adding the same value to every dgate changes nothing."""
    rng = np.random.default_rng(20)
    T, N, k = 50, 16, 4
    s = (1.0 / (1.0 + np.exp(-rng.standard_normal((T, N))))).astype(np.float32)
    idx = np.stack([rng.choice(N, k, replace=False) for _ in range(T)]).astype(np.int32)
    dg = rng.standard_normal((T, k)).astype(np.float32)
    dz = orc.route_backward(s, idx, dg).astype(np.float64)
    dz_shift = orc.route_backward(s, idx, dg + np.float32(0.5)).astype(np.float64)
    assert np.allclose(dz, dz_shift, rtol=1e-5, atol=1e-7)
    assert np.abs(orc.route_backward(s, idx, np.ones((T, k), np.float32))).max() < 1e-7
    # k = 1: the single gate is identically 1
    assert not np.any(orc.route_backward(s, idx[:, :1], dg[:, :1]))


def test_route_backward_two_experts_closed_form(orc):
    """k = 2: g1 = s1/(s1+s2), so dL/dz1 = (dg1 - dg2) s2/(s1+s2)^2 * s1 (1-s1)."""
    s = np.array([[0.2, 0.7, 0.4]], np.float32)
    idx = np.array([[1, 2]], np.int32)
    dg = np.array([[1.5, -0.25]], np.float32)
    dz = orc.route_backward(s, idx, dg)
    s1, s2 = 0.7, 0.4
    S = s1 + s2
    want1 = (1.5 + 0.25) * s2 / S**2 * s1 * (1 - s1)
    want2 = (-0.25 - 1.5) * s1 / S**2 * s2 * (1 - s2)
    assert dz[0, 0] == pytest.approx(want1, rel=1e-6)
    assert dz[0, 1] == pytest.approx(want2, rel=1e-6)


def test_expert_without_rows_has_zero_weight_gradient(orc):
    d, I = 16, 8
    rng = np.random.default_rng(21)
    w13 = rng.standard_normal((2 * I, d)).astype(np.float32)
    w2 = rng.standard_normal((d, I)).astype(np.float32)
    empty = np.zeros((0, d), np.float32)
    dA, dw13, dw2 = orc.swiglu_ffn_backward(empty, w13, w2, empty)
    assert dA.shape == (0, d) and not np.any(dw13) and not np.any(dw2)


def test_combine_backward_scatter_and_dot(orc):
    """dy_perm rows are gate-scaled copies of dout; dgate is the dot product."""
    rng = np.random.default_rng(22)
    T, k, N, d = 10, 3, 6, 12
    idx = np.stack([rng.choice(N, k, replace=False) for _ in range(T)]).astype(np.int32)
    _, _, dst = orc.permute(idx, N)
    dout = rng.standard_normal((T, d)).astype(np.float32)
    yp = rng.standard_normal((T * k, d)).astype(np.float32)
    gate = rng.random((T, k)).astype(np.float32)
    dy, dg = orc.combine_backward(dout, yp, gate, dst)
    for t in range(T):
        for j in range(k):
            r = dst[t, j]
            assert np.allclose(dy[r], gate[t, j] * dout[t], rtol=1e-7)
            assert dg[t, j] == pytest.approx(float(dout[t].astype(np.float64) @ yp[r]),
                                             rel=1e-6)
