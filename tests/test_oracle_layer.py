"""Pins for the oracle's permutation, SwiGLU expert FFN, combine and bias update.

Sources: DeepSeek-V3 report reading guide (xyznot.com/de), "Methode" item 2:
h'_t = u_t + sum_i FFN^(s)_i(u_t) + sum_i g_{i,t} FFN^(r)_i(u_t), and the
end-of-step rule b_i <- b_i - gamma (overloaded) / + gamma (underloaded),
gamma = 0.001; the singularity-lens summary's formula paragraph writes the same
rule as b <- b + gamma * sign(mean_load - load_i).
"""
import math

import numpy as np
import pytest

import moe_inputs


def _bf16_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ------------------------------------------------------------------ permutation

@pytest.mark.parametrize("T,k,N", [(1, 1, 1), (7, 3, 5), (64, 2, 16), (333, 8, 64)])
def test_permutation_bijection_stable(orc, T, k, N):
    rng = np.random.default_rng(T + k + N)
    idx = np.stack([rng.choice(N, k, replace=False) for _ in range(T)]).astype(np.int32)
    off, src, dst = orc.permute(idx, N)
    counts = np.bincount(idx.ravel(), minlength=N)
    assert off[0] == 0 and np.array_equal(np.diff(off), counts) and off[-1] == T * k
    # bijection: every row is used once, and src/dst invert each other
    assert np.array_equal(np.sort(dst.ravel()), np.arange(T * k))
    for t in range(T):
        for j in range(k):
            assert src[dst[t, j]] == t
            e = idx[t, j]
            assert off[e] <= dst[t, j] < off[e + 1]
    # stable: ascending token order inside each expert's rows
    for e in range(N):
        seg = src[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)


def test_gather_round_trip_bitwise(orc):
    rng = np.random.default_rng(12)
    T, k, N, d = 50, 4, 8, 24
    idx = np.stack([rng.choice(N, k, replace=False) for _ in range(T)]).astype(np.int32)
    x = rng.integers(0, 65535, (T, d), dtype=np.uint16)
    off, src, dst = orc.permute(idx, N)
    xp = orc.gather_rows(x, src)
    for t in range(T):
        for j in range(k):
            assert np.array_equal(xp[dst[t, j]], x[t])


# ------------------------------------------------------------------ SwiGLU FFN

def _dense_swiglu_f32(A, w13, w2):
    """numpy fp64 matmuls with the oracle's stated rounding points (a, b, h, y -> fp32)"""
    I = w13.shape[0] // 2
    A64 = A.astype(np.float64)
    a = (A64 @ w13[:I].astype(np.float64).T).astype(np.float32).astype(np.float64)
    b = (A64 @ w13[I:].astype(np.float64).T).astype(np.float32).astype(np.float64)
    h = (a / (1.0 + np.exp(-a)) * b).astype(np.float32).astype(np.float64)
    return (h @ w2.astype(np.float64).T).astype(np.float32)


def test_swiglu_matches_dense_library_matmul(orc):
    rng = np.random.default_rng(13)
    M, d, I = 37, 96, 40   # d != I so a transposed W2 cannot pass
    A = rng.standard_normal((M, d)).astype(np.float32)
    w13 = (rng.standard_normal((2 * I, d)) / math.sqrt(d)).astype(np.float32)
    w2 = (rng.standard_normal((d, I)) / math.sqrt(I)).astype(np.float32)
    y = orc.swiglu_ffn(A, w13, w2)
    ref = _dense_swiglu_f32(A, w13, w2)
    assert np.allclose(y, ref, rtol=1e-6, atol=1e-7)
    # gate/up roles are not symmetric: swapping W1 and W3 must change the result
    swapped = np.concatenate([w13[I:], w13[:I]])
    assert not np.allclose(orc.swiglu_ffn(A, swapped, w2), y, rtol=1e-3)


def test_swiglu_bf16_storage(orc):
    rng = np.random.default_rng(14)
    M, d, I = 9, 64, 32
    f = lambda a: ((a.astype(np.float32).view(np.uint32) + 0x7FFF +
                    ((a.astype(np.float32).view(np.uint32) >> 16) & 1)) >> 16).astype(np.uint16)
    A = f(rng.standard_normal((M, d)))
    w13 = f(rng.standard_normal((2 * I, d)) / 8)
    w2 = f(rng.standard_normal((d, I)) / 6)
    y = orc.swiglu_ffn(A, w13, w2)
    ref = _dense_swiglu_f32(_bf16_to_f64(A).astype(np.float32),
                            _bf16_to_f64(w13).astype(np.float32),
                            _bf16_to_f64(w2).astype(np.float32)).astype(np.float64)
    got = _bf16_to_f64(y)
    # h is rounded to bf16 before the down projection: one bf16 rounding of h
    # and one of y -> relative error a few 2^-9 at most
    assert np.all(np.abs(got - ref) <= 2.0 ** -6 * (np.abs(ref) + np.sqrt(np.mean(ref ** 2))))


def test_round_to_bf16_single_rounding(orc):
    # 1 + 2^-8 + 2^-30 : a double that fp32-then-bf16 double rounding sends to 1,
    # but the single rounding sends up to 1 + 2^-7
    v = np.array([1.0 + 2.0 ** -8 + 2.0 ** -30, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8,
                  -(1.0 + 2.0 ** -8 + 2.0 ** -30), 3.4e38, 1e-40, 3.0e38], np.float64)
    out = orc.round_to_dtype(v, "bf16")
    assert out[0] == 0x3F81
    assert out[1] == 0x3F80          # tie -> even
    assert out[2] == 0x3F82          # tie -> even (upward)
    assert out[3] == 0xBF81
    assert out[4] == 0x7F80          # past the largest finite bf16 -> +inf
    assert abs(_bf16_to_f64(out[6:7])[0] - 3.0e38) <= 3.0e38 * 2.0 ** -9
    assert abs(_bf16_to_f64(out[5:6])[0] - 1e-40) <= 2.0 ** -134


# ------------------------------------------------------------------ combine

def test_combine_closed_forms(orc):
    rng = np.random.default_rng(15)
    T, k, N, d = 20, 3, 6, 16
    x = rng.standard_normal((T, d)).astype(np.float32)
    idx = np.stack([rng.choice(N, k, replace=False) for _ in range(T)]).astype(np.int32)
    _, src, dst = orc.permute(idx, N)
    gate = rng.uniform(0.1, 1.0, (T, k)).astype(np.float32)
    zeros_p = np.zeros((T * k, d), np.float32)
    # residual only
    assert np.array_equal(orc.combine(x, None, zeros_p, gate, dst, "f32"), x)
    yp = rng.standard_normal((T * k, d)).astype(np.float32)
    ys = rng.standard_normal((T, d)).astype(np.float32)
    out = orc.combine(x, ys, yp, gate, dst, "f32")
    ref = x.astype(np.float64) + ys
    for j in range(k):
        ref = ref + gate[:, j:j + 1].astype(np.float64) * yp[dst[:, j]].astype(np.float64)
    assert np.allclose(out, ref.astype(np.float32), rtol=2 ** -23, atol=1e-7)
    # without the residual
    out2 = orc.combine(None, ys, yp, gate, dst, "f32")
    assert np.allclose(out2, (ref - x).astype(np.float32), rtol=2 ** -22, atol=1e-6)


def test_layer_identical_experts_reduces_to_dense(orc):
    """All routed experts equal and gates summing to 1: the layer is
    u + FFN_s(u) + FFN(u), checked against numpy fp64 matmuls."""
    cfg = dict(moe_inputs.CONFIGS["tiny_fp32"])
    rng = np.random.default_rng(16)
    T, d, N, k, I = cfg["T"], cfg["d"], cfg["N"], cfg["k"], cfg["I"]
    x = rng.standard_normal((T, d)).astype(np.float32)
    E = (rng.standard_normal((N, d)) / math.sqrt(d)).astype(np.float32)
    w13 = (rng.standard_normal((2 * I, d)) / math.sqrt(d)).astype(np.float32)
    w2 = (rng.standard_normal((d, I)) / math.sqrt(I)).astype(np.float32)
    ws13 = (rng.standard_normal((2 * I, d)) / math.sqrt(d)).astype(np.float32)
    ws2 = (rng.standard_normal((d, I)) / math.sqrt(I)).astype(np.float32)
    inp = dict(x=x, centroids=E, bias=np.zeros(N, np.float32),
               w13=np.broadcast_to(w13, (N, 2 * I, d)).copy(),
               w2=np.broadcast_to(w2, (N, d, I)).copy(), ws13=ws13, ws2=ws2)
    res = orc.layer_forward(inp, cfg)
    ref = (x.astype(np.float64) + _dense_swiglu_f32(x, ws13, ws2) +
           _dense_swiglu_f32(x, w13, w2))
    rms = np.sqrt(np.mean(ref ** 2, axis=1, keepdims=True))
    assert np.all(np.abs(res["out"] - ref) <= 1e-5 * (np.abs(ref) + rms))


# ------------------------------------------------------------------ bias update

def test_gamma_is_nearest_fp32_to_one_thousandth(orc):
    assert np.float32(orc.GAMMA).view(np.uint32) == 0x3A83126F
    assert abs(float(orc.GAMMA) - 0.001) < 2.0 ** -34


def test_bias_update_closed_form(orc):
    N, TK = 8, 32  # mean load 4
    counts = np.array([0, 3, 4, 5, 12, 4, 2, 2], np.int32)
    b0 = np.array([0.0, 0.5, -0.25, 1.0, 0.0, 0.0, -1e-3, 1e-3], np.float32)
    b1 = orc.bias_update(counts, TK, b0)
    g = np.float32(0.001)
    exp = np.array([b0[0] + g, b0[1] + g, b0[2], b0[3] - g, b0[4] - g, b0[5],
                    b0[6] + g, b0[7] + g], np.float32)
    assert np.array_equal(b1.view(np.uint32), exp.view(np.uint32))
    assert np.array_equal(b0, np.array([0.0, 0.5, -0.25, 1.0, 0.0, 0.0, -1e-3, 1e-3],
                                       np.float32))


def test_bias_update_uniform_load_is_fixed_point(orc):
    N, T, k = 16, 64, 2
    counts = np.full(N, T * k // N, np.int32)
    b = np.linspace(-1, 1, N).astype(np.float32)
    assert np.array_equal(orc.bias_update(counts, T * k, b), b)


def test_bias_update_non_integer_mean(orc):
    # mean load 10/3: counts 3 is under, 4 is over; the comparison is exact
    counts = np.array([3, 4, 3], np.int32)
    b = orc.bias_update(counts, 10, np.zeros(3, np.float32))
    assert b[0] > 0 and b[1] < 0 and b[2] > 0


def test_balancing_reduces_skew(orc):
    """Repeated route + update on a skewed router lowers the max/mean load
    (the pages' qualitative claim; the rate is not stated)."""
    rng = np.random.default_rng(17)
    T, d, N, k = 256, 32, 16, 2
    E = (rng.standard_normal((N, d)) / math.sqrt(d)).astype(np.float32)
    E[:, 0] = -0.5 * np.log(np.arange(1, N + 1))  # skewed popularity
    b = np.zeros(N, np.float32)
    first = last = None
    for step in range(300):
        x = rng.standard_normal((T, d)).astype(np.float32)
        x[:, 0] = 1.0
        r = orc.route(x, E, b, k)
        imb = r["counts"].max() / (T * k / N)
        if step == 0:
            first = imb
        last = imb
        b = orc.bias_update(r["counts"], T * k, b)
    assert last < first
