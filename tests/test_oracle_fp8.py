"""Pins for the oracle's FP8 E4M3 path.

Sources: DeepSeek-V3 report reading guide (xyznot.com/de), "Kernideen", FP8
bullet: E4M3 for all tensors, 1x128 activation tiles, 128x128 weight blocks,
FP32 promotion every N_c = 128 accumulation steps; the singularity-lens
summary's formula paragraph: S = max|X| / 448, X_fp8 = clip(round(X / S), -448, 448).

The independent references here are PyTorch's own float8_e4m3fn dtype (its
decode table and its float32 cast, which rounds to nearest-even), a
nearest-code search over that table, and numpy fp64 matmuls of dequantised
operands.
"""
import math

import numpy as np
import pytest
import torch


def _torch_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()


def _torch_encode(v):
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_table_matches_torch(orc):
    ref = _torch_decode_all()
    got = orc.e4m3_decode(np.arange(256, dtype=np.uint8))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2   # 0x7F, 0xFF
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def _nearest_code(v, table):
    """nearest finite code by exhaustive search, ties to the even code"""
    finite = [(c, float(table[c])) for c in range(256) if not math.isnan(table[c])]
    best = None
    for c, val in finite:
        if val == 0.0 and c != (0x80 if math.copysign(1, v) < 0 else 0):
            continue  # keep the sign of zero
        dist = abs(val - v)
        if best is None or dist < best[1] or (dist == best[1] and (c & 1) == 0 and best[0] & 1):
            best = (c, dist)
    return best[0]


def test_encode_all_midpoints_and_neighbours(orc):
    table = _torch_decode_all()
    pos = sorted(float(table[c]) for c in range(0x00, 0x7F))
    vals = []
    for a, b in zip(pos[:-1], pos[1:]):
        m = np.float32((a + b) / 2)           # every midpoint is exact in fp32
        vals += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(1e9)), a, b]
    vals = np.array(vals, np.float32)
    vals = np.concatenate([vals, -vals, np.array([0.0, -0.0], np.float32)])
    got = orc.e4m3_encode(vals)
    assert np.array_equal(got, _torch_encode(vals))
    # and against an exhaustive nearest-code search on a subsample
    for v, c in zip(vals[::7], got[::7]):
        assert c == _nearest_code(float(v), table)


def test_encode_random_values(orc):
    rng = np.random.default_rng(20)
    v = np.concatenate([rng.uniform(-448, 448, 200000),
                        rng.standard_normal(200000) * 2.0 ** rng.integers(-12, 8, 200000)])
    v = np.clip(v, -448, 448).astype(np.float32)
    assert np.array_equal(orc.e4m3_encode(v), _torch_encode(v))


def test_quant_act_tiles(orc):
    rng = np.random.default_rng(21)
    rows, cols = 6, 512
    x = (rng.standard_normal((rows, cols)) * np.exp(rng.standard_normal((rows, 1)))).astype(
        np.float32)
    x[2, 128:256] = 0.0            # an all-zero tile
    x[3, 0:128] = -x[3, 0:128]
    q, s = orc.quant_act_fp8(x)
    assert s.shape == (rows, cols // 128)
    assert s[2, 1] == 0 and np.all(q[2, 128:256] == 0)
    dec = orc.e4m3_decode(q).astype(np.float64)
    for r in range(rows):
        for c in range(cols // 128):
            tile = x[r, c * 128:(c + 1) * 128]
            amax = np.abs(tile).max()
            if amax == 0:
                continue
            assert s[r, c] == np.float32(amax) / np.float32(448.0)
            j = int(np.argmax(np.abs(tile)))
            assert q[r, c * 128 + j] in (0x7E, 0xFE)          # the amax maps to +-448
            # dequantisation error at most half a code spacing (spacing <= 32 * 2^-... )
            deq = dec[r, c * 128:(c + 1) * 128] * float(s[r, c])
            err = np.abs(deq - tile)
            spacing = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(np.abs(tile) / s[r, c],
                                                                       2.0 ** -6))) - 3),
                                 2.0 ** -9) * float(s[r, c])
            assert np.all(err <= 0.5 * spacing * (1 + 1e-6) + 1e-30)
            # the codes are the float32 quotient rounded by an independent converter
            t = np.clip(tile / np.float32(s[r, c]), -448, 448).astype(np.float32)
            assert np.array_equal(q[r, c * 128:(c + 1) * 128], _torch_encode(t))


def test_quant_weight_blocks(orc):
    rng = np.random.default_rng(22)
    w = (rng.standard_normal((2, 256, 384)) / 30).astype(np.float32)
    w[1, 128:, 256:] *= 100.0
    q, s = orc.quant_weight_fp8(w)
    assert s.shape == (2, 2, 3)
    for m in range(2):
        for rb in range(2):
            for cb in range(3):
                blk = w[m, rb * 128:(rb + 1) * 128, cb * 128:(cb + 1) * 128]
                assert s[m, rb, cb] == np.float32(np.abs(blk).max()) / np.float32(448)
                t = np.clip(blk / s[m, rb, cb], -448, 448).astype(np.float32)
                assert np.array_equal(q[m, rb * 128:(rb + 1) * 128, cb * 128:(cb + 1) * 128],
                                      _torch_encode(t))


def test_quant_bf16_input(orc):
    rng = np.random.default_rng(23)
    xf = rng.standard_normal((3, 256)).astype(np.float32)
    bits = (xf.view(np.uint32) >> 16).astype(np.uint16)
    wid = (bits.astype(np.uint32) << 16).view(np.float32)
    q1, s1 = orc.quant_act_fp8(bits)
    q2, s2 = orc.quant_act_fp8(wid)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


def test_fp8_ffn_equals_dequantised_fp64(orc):
    """The per-128-block scaled sums equal one fp64 GEMM of the dequantised
    operands (the same mathematical value): promotion every 128 K-elements."""
    rng = np.random.default_rng(24)
    M, d, I = 10, 256, 256
    A = rng.standard_normal((M, d)).astype(np.float32)
    w13 = (rng.standard_normal((2 * I, d)) / 16).astype(np.float32)
    w2 = (rng.standard_normal((d, I)) / 16).astype(np.float32)
    w13[:, :128] *= 3.0
    Aq, As = orc.quant_act_fp8(A)
    w13q, w13s = orc.quant_weight_fp8(w13)
    w2q, w2s = orc.quant_weight_fp8(w2)
    y = orc.swiglu_ffn_fp8(Aq, As, w13q, w13s, w2q, w2s)
    tab = _torch_decode_all().astype(np.float64)
    Ad = tab[Aq] * np.repeat(As.astype(np.float64), 128, axis=1)
    Wd = tab[w13q] * np.kron(w13s.astype(np.float64), np.ones((128, 128)))
    W2d = tab[w2q] * np.kron(w2s.astype(np.float64), np.ones((128, 128)))
    a = (Ad @ Wd[:I].T).astype(np.float32).astype(np.float64)
    b = (Ad @ Wd[I:].T).astype(np.float32).astype(np.float64)
    h = (a / (1 + np.exp(-a)) * b).astype(np.float32)
    hq, hs = orc.quant_act_fp8(h)
    Hd = tab[hq] * np.repeat(hs.astype(np.float64), 128, axis=1)
    ref = Hd @ W2d.T
    got = (y.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rel = np.abs(got - ref) / (np.abs(ref) + 1e-30)
    assert np.mean(rel <= 2.0 ** -8) > 0.99
    assert np.all(np.abs(got - ref) <= 2.0 ** -7 * (np.abs(ref) + np.sqrt(np.mean(ref ** 2))))
    # and FP8 stays close to the unquantised bf16-free computation
    full = ((lambda a_, b_: a_ / (1 + np.exp(-a_)) * b_)(A.astype(np.float64) @ w13[:I].T,
                                                         A.astype(np.float64) @ w13[I:].T)
            @ w2.astype(np.float64).T)
    # (3 mantissa bits: a few percent norm-wise after two quantised GEMMs)
    assert np.linalg.norm(got - full) <= 0.1 * np.linalg.norm(full)


def test_fp8_promotion_block_boundaries(orc):
    """Two K-blocks with very different scales: a kernel that applied one scale
    to the whole row would be off by orders of magnitude."""
    M, d, I = 1, 256, 128
    A = np.zeros((M, d), np.float32)
    A[0, :128] = 1000.0
    A[0, 128:] = 0.001
    w13 = np.ones((2 * I, d), np.float32) / 64
    w2 = np.eye(d, I, dtype=np.float32)
    Aq, As = orc.quant_act_fp8(A)
    assert As[0, 0] == np.float32(1000.0) / np.float32(448) and As[0, 1] == np.float32(
        0.001) / np.float32(448)
    w13q, w13s = orc.quant_weight_fp8(w13)
    w2q, w2s = orc.quant_weight_fp8(w2)
    y = orc.swiglu_ffn_fp8(Aq, As, w13q, w13s, w2q, w2s)
    a = 128 * 1000.0 / 64 + 128 * 0.001 / 64
    h = a / (1 + math.exp(-a)) * a
    got = float((y[0, 0].astype(np.uint32) << 16).view(np.float32))
    assert abs(got - h) <= h * 2.0 ** -6


def _dequant_rows(tab, q, s):
    return tab[q] * np.repeat(s.astype(np.float64), 128, axis=1)


def _dequant_blocks(tab, q, s):
    return tab[q] * np.kron(s.astype(np.float64), np.ones((128, 128)))


def test_fp8_gateup_half_equals_dequantised_fp64(orc):
    """The gate/up half alone: a, b are the fp64 GEMM of the dequantised
    operands (the block-scaled exact sums are the same value) rounded to fp32,
    h = silu(a) * b rounded to fp32.  Block scales differ per 128-row block
    and per K block, so a transposed scale index changes the result."""
    rng = np.random.default_rng(31)
    M, d, I = 9, 384, 256
    A = rng.standard_normal((M, d)).astype(np.float32)
    A[:, 128:256] *= 40.0
    w13 = (rng.standard_normal((2 * I, d)) / 16).astype(np.float32)
    w13[128:256] *= 0.01
    w13[:, 256:] *= 7.0
    Aq, As = orc.quant_act_fp8(A)
    wq, ws = orc.quant_weight_fp8(w13)
    assert len(set(ws.ravel().tolist())) == ws.size
    h = orc.swiglu_gateup_fp8(Aq, As, wq, ws)
    tab = _torch_decode_all().astype(np.float64)
    Ad, Wd = _dequant_rows(tab, Aq, As), _dequant_blocks(tab, wq, ws)
    a = (Ad @ Wd[:I].T).astype(np.float32).astype(np.float64)
    b = (Ad @ Wd[I:].T).astype(np.float32).astype(np.float64)
    ref = (a / (1 + np.exp(-a)) * b).astype(np.float32)
    # fp64 matmul rounding can move a or b across an fp32 rounding boundary
    # (then by one fp32 ulp); everything else is identical
    err = np.abs(h.astype(np.float64) - ref) / (np.abs(ref.astype(np.float64)) + 1e-30)
    assert np.mean(h == ref) > 0.99
    assert np.all(err <= 2.0 ** -21)


def test_fp8_down_half_equals_dequantised_fp64(orc):
    """The down half alone, from given h codes and 1x128 tile scales: the fp64
    GEMM of the dequantised operands rounded once to bf16 (at most one bf16
    step apart where fp64 rounding meets a bf16 midpoint)."""
    rng = np.random.default_rng(32)
    M, I, d = 7, 384, 256
    h = (rng.standard_normal((M, I)) * np.exp(rng.standard_normal((M, 1)))).astype(np.float32)
    h[:, 256:] *= 1e-3
    w2 = (rng.standard_normal((d, I)) / 20).astype(np.float32)
    w2[128:, :128] *= 50.0
    hq, hs = orc.quant_act_fp8(h)
    wq, ws = orc.quant_weight_fp8(w2)
    y = orc.ffn_down_fp8(hq, hs, wq, ws)
    tab = _torch_decode_all().astype(np.float64)
    ref = _dequant_rows(tab, hq, hs) @ _dequant_blocks(tab, wq, ws).T
    got = (y.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref_bf = torch.from_numpy(ref).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.mean(got == ref_bf) > 0.99
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-300)


def test_fp8_expert_is_its_two_halves(orc):
    """The whole FP8 expert = gate/up half -> 1x128 re-quantisation of h ->
    down half, bit for bit (the GPU tests feed the GPU's own h to the down
    half, so the split must not change the composite)."""
    rng = np.random.default_rng(33)
    M, d, I = 6, 256, 384
    A = rng.standard_normal((M, d)).astype(np.float32)
    w13 = (rng.standard_normal((2 * I, d)) / 16).astype(np.float32)
    w2 = (rng.standard_normal((d, I)) / 16).astype(np.float32)
    Aq, As = orc.quant_act_fp8(A)
    q13, s13 = orc.quant_weight_fp8(w13)
    q2, s2 = orc.quant_weight_fp8(w2)
    y = orc.swiglu_ffn_fp8(Aq, As, q13, s13, q2, s2)
    hq, hs = orc.quant_act_fp8(orc.swiglu_gateup_fp8(Aq, As, q13, s13))
    assert np.array_equal(y, orc.ffn_down_fp8(hq, hs, q2, s2))


def test_encode_nan_is_the_format_nan(orc):
    """A NaN (outside the layer's finite-input contract, but it must not be
    undefined behaviour) encodes as E4M3FN's NaN S.1111.111, as PyTorch's cast
    does; a tile holding a NaN keeps the scale of its finite values."""
    v = np.array([np.nan, -np.nan], np.float32)
    assert np.array_equal(orc.e4m3_encode(v), _torch_encode(v))
    x = np.linspace(-3, 3, 128).astype(np.float32)[None, :].copy()
    x[0, 5] = np.nan
    q, s = orc.quant_act_fp8(x)
    assert s[0, 0] == np.float32(3.0) / np.float32(448) and q[0, 5] in (0x7F, 0xFF)
