"""Pins for the oracle's FP8 backward of one SwiGLU expert.

The method (DeepSeek-V3 report reading guide, xyznot.com/de, "Kernideen",
FP8 bullet) runs every tensor of the expert GEMMs in E4M3 with 1x128
activation tiles and 128x128 weight blocks.  The oracle reads that for the
backward as: each GEMM operand is quantised along that GEMM's contraction, so
the weight-gradient GEMMs (which contract over an expert's rows) use 128x1
tiles running down the rows (oracle/moe_oracle.c, orc_quant_cols_fp8 and
orc_swiglu_ffn_backward_fp8).  Pinned here against things the oracle does not
contain:
  - closed forms of the row-direction tiles: the scale of each tile is its
    column's amax over the tile's rows / 448, the rows of one tile never
    reach another, and a value equal to the amax decodes exactly to 448;
  - float64 reverse-mode differentiation (torch.autograd) of a dense SwiGLU
    expert on the dequantised forward operands: the FP8 backward must agree
    within the quantisation error (relative Frobenius error), with block- and
    row-dependent magnitudes so that a scale taken from the wrong block, a
    transposed operand or a dropped term is an O(1) error;
  - exact odd symmetry in the output gradient (the quantisers round
    symmetrically), and zero output gradient / zero rows giving zeros.
"""
import numpy as np
import pytest
import torch


def _bf16(a):
    """float64 -> bf16 bits (round to nearest even, through torch)"""
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _f64(a):
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _decode(orc, q):
    return orc.e4m3_decode(q).astype(np.float64)


def test_row_direction_tiles_closed_form(orc):
    rng = np.random.default_rng(1)
    M, C = 130, 3
    x = rng.uniform(-1.0, 1.0, (M, C))
    x[5, 0] = 3.0           # amax of tile (0, 0)
    x[127, 1] = -40.0       # amax of tile (0, 1), last row of the first tile
    x[128, 1] = 0.25        # the second tile holds rows 128 and 129 only
    x[129, 1] = -0.125
    x[:, 2] = 0.0           # an all-zero column
    xb = _bf16(x)
    xv = _f64(xb)
    q, s = orc.quant_cols_fp8(xb)
    assert q.shape == (M, C) and s.shape == (2, C)
    for u, (r0, r1) in enumerate(((0, 128), (128, 130))):
        for c in range(C):
            amax = np.float32(np.abs(xv[r0:r1, c]).max())
            assert s[u, c] == amax / np.float32(448.0), (u, c)
    assert s[1, 1] == np.float32(0.25) / np.float32(448.0)   # row 127 does not reach tile 1
    assert np.all(q[:, 2] == 0) and np.all(s[:, 2] == 0)
    dec = _decode(orc, q)
    assert dec[5, 0] == 448.0 and dec[127, 1] == -448.0 and dec[128, 1] == 448.0
    # every code is the E4M3 value nearest x / scale (3 mantissa bits)
    for u, (r0, r1) in enumerate(((0, 128), (128, 130))):
        for c in range(2):
            t = xv[r0:r1, c] / np.float64(s[u, c])
            assert np.all(np.abs(dec[r0:r1, c] - t) <= np.abs(t) * 2.0 ** -4 + 2.0 ** -10)


def _expert_case(orc, M, d, I, seed):
    """bf16 rows, weights and output gradient with magnitudes that change per
    128-block (weights), per 128-column tile (rows) and per row"""
    rng = np.random.default_rng(seed)
    blk = lambda r, c: np.kron(2.0 ** rng.integers(-2, 3, (r // 128, c // 128)), np.ones((128, 128)))
    A = rng.standard_normal((M, d)) * (2.0 ** rng.integers(-1, 2, (M, 1)))
    A *= np.repeat(2.0 ** rng.integers(-1, 2, (1, d // 128)), 128, axis=1)
    w13 = rng.standard_normal((2 * I, d)) / np.sqrt(d) * blk(2 * I, d)
    w2 = rng.standard_normal((d, I)) / np.sqrt(I) * blk(d, I)
    dY = rng.standard_normal((M, d)) * (2.0 ** rng.integers(-2, 2, (M, 1)))
    A, w13, w2, dY = _bf16(A), _bf16(w13), _bf16(w2), _bf16(dY)
    Aq, As = orc.quant_act_fp8(A)
    w13q, w13s = orc.quant_weight_fp8(w13)
    w2q, w2s = orc.quant_weight_fp8(w2)
    return A, dY, Aq, As, w13q, w13s, w2q, w2s


def _dequant_rows(orc, q, s):
    return _decode(orc, q) * np.repeat(s.astype(np.float64), 128, axis=1)


def _dequant_blocks(orc, q, s):
    return _decode(orc, q) * np.kron(s.astype(np.float64), np.ones((128, 128)))


@pytest.mark.parametrize("M,d,I,seed", [(200, 256, 256, 0), (77, 384, 128, 1), (300, 128, 256, 2)])
def test_fp8_backward_against_float64_autograd(orc, M, d, I, seed):
    A, dY, Aq, As, w13q, w13s, w2q, w2s = _expert_case(orc, M, d, I, seed)
    dA, dw13, dw2 = orc.swiglu_ffn_backward_fp8(Aq, As, A, w13q, w13s, w2q, w2s, dY)
    Ad = torch.tensor(_dequant_rows(orc, Aq, As), requires_grad=True)
    W13 = torch.tensor(_dequant_blocks(orc, w13q, w13s), requires_grad=True)
    W2 = torch.tensor(_dequant_blocks(orc, w2q, w2s), requires_grad=True)
    a = Ad @ W13[:I].T
    b = Ad @ W13[I:].T
    y = (torch.nn.functional.silu(a) * b) @ W2.T
    (y * torch.from_numpy(_f64(dY))).sum().backward()
    for name, got, ref in (("dA", dA, Ad.grad), ("dw13", dw13, W13.grad), ("dw2", dw2, W2.grad)):
        g, r = _f64(got), ref.numpy()
        rel = np.linalg.norm(g - r) / np.linalg.norm(r)
        assert rel < 0.08, (name, rel)
        # no element far off: within 1.5 times the tensor's RMS
        assert np.max(np.abs(g - r)) < 1.5 * np.sqrt(np.mean(r ** 2)), name


def test_fp8_backward_is_odd_in_the_output_gradient(orc):
    A, dY, Aq, As, w13q, w13s, w2q, w2s = _expert_case(orc, 150, 256, 128, 3)
    pos = orc.swiglu_ffn_backward_fp8(Aq, As, A, w13q, w13s, w2q, w2s, dY)
    neg = orc.swiglu_ffn_backward_fp8(Aq, As, A, w13q, w13s, w2q, w2s, dY ^ np.uint16(0x8000))
    for p, n in zip(pos, neg):
        assert np.array_equal(_f64(p), -_f64(n))


def test_fp8_backward_zero_gradient_and_zero_rows(orc):
    A, dY, Aq, As, w13q, w13s, w2q, w2s = _expert_case(orc, 64, 128, 128, 4)
    z = orc.swiglu_ffn_backward_fp8(Aq, As, A, w13q, w13s, w2q, w2s, np.zeros_like(dY))
    for t in z:
        assert not np.any(_f64(t))
    dA, dw13, dw2 = orc.swiglu_ffn_backward_fp8(Aq[:0], As[:0], A[:0], w13q, w13s, w2q, w2s,
                                                dY[:0])
    assert dA.shape == (0, 128) and not np.any(_f64(dw13)) and not np.any(_f64(dw2))


# ------------------------------------------------------------------ the steps

def _tab():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    t = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    t[np.isnan(t)] = 0.0
    return t


def _bf(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _f(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _to_bf16(v):
    return torch.from_numpy(np.asarray(v, np.float64)).to(torch.bfloat16).to(torch.float64).numpy()


def test_fp8_dgrad_step_equals_dequantised_fp64(orc):
    """bf16(g W) from row-tiled codes and a block-scaled weight: the fp64 GEMM
    of the dequantised operands rounded once to bf16 (one bf16 step at most
    where fp64 rounding meets a midpoint); scales differ per block, so a
    transposed scale index fails."""
    rng = np.random.default_rng(41)
    M, K, N = 9, 384, 256
    g = rng.standard_normal((M, K)).astype(np.float32)
    g[:, 128:256] *= 30
    w = (rng.standard_normal((K, N)) / 20).astype(np.float32)
    w[128:256, :128] *= 0.01
    gq, gs = orc.quant_act_fp8(g)
    wq, ws = orc.quant_weight_fp8(w)
    out = orc.fp8_dgrad(gq, gs, wq, ws)
    t = _tab()
    ref = (t[gq] * np.repeat(gs.astype(np.float64), 128, 1)) @ (
        t[wq] * np.kron(ws.astype(np.float64), np.ones((128, 128))))
    got = _f(out)
    assert np.mean(got == _to_bf16(ref)) > 0.99
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-300)


def test_fp8_wgrad_step_equals_dequantised_fp64(orc):
    """bf16(A^T B) over 300 rows in 128x1 tiles (a partial last tile): the
    fp64 product of the dequantised row-direction tiles."""
    rng = np.random.default_rng(42)
    M, FA, FB = 300, 64, 48
    A = rng.standard_normal((M, FA)).astype(np.float32) * np.exp(rng.standard_normal((M, 1)))
    B = rng.standard_normal((M, FB)).astype(np.float32)
    Aq, As = orc.quant_cols_fp8(A.astype(np.float32))
    Bq, Bs = orc.quant_cols_fp8(B)
    out = orc.fp8_wgrad(Aq, As, Bq, Bs)
    t = _tab()
    rep = lambda s: np.repeat(s.astype(np.float64), 128, 0)[:M]
    ref = (t[Aq] * rep(As)).T @ (t[Bq] * rep(Bs))
    got = _f(out)
    assert np.mean(got == _to_bf16(ref)) > 0.99
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-300)


def test_swiglu_bwd_step_matches_autograd(orc):
    """[da db] from stored bf16 dh, a, b: float64 autograd of silu(a) b, rounded
    once to bf16 (at most one bf16 step apart where evaluation order meets a
    midpoint), with a spanning the region where silu' changes sign."""
    rng = np.random.default_rng(43)
    M, I = 5, 256
    a = rng.uniform(-6, 6, (M, I)).astype(np.float32)
    b = rng.standard_normal((M, I)).astype(np.float32)
    dh = rng.standard_normal((M, I)).astype(np.float32)
    ab = np.concatenate([_bf(a), _bf(b)], axis=1)
    dab = orc.swiglu_bwd_bf16(_bf(dh), ab)
    at = torch.tensor(_f(ab[:, :I]), requires_grad=True)
    bt = torch.tensor(_f(ab[:, I:]), requires_grad=True)
    h = at * torch.sigmoid(at) * bt
    h.backward(torch.tensor(_f(_bf(dh))))
    for got, ref in ((dab[:, :I], at.grad.numpy()), (dab[:, I:], bt.grad.numpy())):
        assert np.all(np.abs(_f(got) - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)


def test_fp8_recompute_step_matches_forward_half(orc):
    """a, b kept in bf16 are the forward's fp32 sums rounded to bf16 (checked
    against the fp64 GEMM of the dequantised operands), and h is within one
    bf16 step of the forward half's fp32 h."""
    rng = np.random.default_rng(44)
    M, d, I = 7, 256, 128
    x = rng.standard_normal((M, d)).astype(np.float32)
    w13 = (rng.standard_normal((2 * I, d)) / 16).astype(np.float32)
    xq, xs = orc.quant_act_fp8(x)
    wq, ws = orc.quant_weight_fp8(w13)
    ab, h = orc.fp8_recompute_ab(xq, xs, wq, ws)
    t = _tab()
    ref = (t[xq] * np.repeat(xs.astype(np.float64), 128, 1)) @ (
        t[wq] * np.kron(ws.astype(np.float64), np.ones((128, 128)))).T
    assert np.all(np.abs(_f(ab) - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)
    hf = orc.swiglu_gateup_fp8(xq, xs, wq, ws).astype(np.float64)
    assert np.all(np.abs(_f(h) - hf) <= 2.0 ** -8 * np.abs(hf) + 1e-30)


def test_fp8_backward_is_its_steps(orc):
    """The composite FP8 backward equals its steps chained in order, bit for
    bit (the GPU checks feed the GPU's own intermediates to the steps)."""
    rng = np.random.default_rng(45)
    M, d, I = 130, 256, 128
    A = _bf(rng.standard_normal((M, d)))
    dY = _bf(rng.standard_normal((M, d)))
    w13 = (rng.standard_normal((2 * I, d)) / 16).astype(np.float32)
    w2 = (rng.standard_normal((d, I)) / 16).astype(np.float32)
    Aq, As = orc.quant_act_fp8(A)
    q13, s13 = orc.quant_weight_fp8(w13)
    q2, s2 = orc.quant_weight_fp8(w2)
    dA, dw13, dw2 = orc.swiglu_ffn_backward_fp8(Aq, As, A, q13, s13, q2, s2, dY)
    ab, h = orc.fp8_recompute_ab(Aq, As, q13, s13)
    gq, gs = orc.quant_act_fp8(dY)
    dh = orc.fp8_dgrad(gq, gs, q2, s2)
    dab = orc.swiglu_bwd_bf16(dh, ab)
    tq, ts = orc.quant_act_fp8(dab)
    assert np.array_equal(dA, orc.fp8_dgrad(tq, ts, q13, s13))
    cols = [orc.quant_cols_fp8(v) for v in (dY, h, dab, A)]
    assert np.array_equal(dw2, orc.fp8_wgrad(*cols[0], *cols[1]))
    assert np.array_equal(dw13, orc.fp8_wgrad(*cols[2], *cols[3]))
