"""Pins for the oracle's routing: logits, sigmoid affinity, biased (group-limited)
top-k, gate normalisation and load counts.

Source of the method: DeepSeek-V3 report reading guide (xyznot.com/de),
"Methode" item 2 -- s_{i,t} = Sigmoid(u_t^T e_i); g'_{i,t} = s_{i,t} when
s_{i,t} + b_i is in the Topk of {s_{j,t} + b_j}, else 0; g = normalised g'.
Each test checks the oracle against something other than itself: a worked
closed form, an arbitrary-precision evaluation, brute-force enumeration, or an
invariant the passage implies.
"""
import itertools
import math
from decimal import Decimal, getcontext

import numpy as np
import pytest

pytestmark = []


def _f32(v):
    return np.float32(v)


# ------------------------------------------------------------------ logits

def test_logits_chain_order_worked_example(orc):
    # u.e with e = 1: 2^24 + 1 + 1 - 2^24.  Exact value 2.  The index-ascending
    # fp32 chain gives 0 (each +1 is lost to round-to-even at 2^24); the reverse
    # order would give 2; a pairwise tree would give 2.
    x = np.array([[2.0 ** 24, 1.0, 1.0, -(2.0 ** 24)]], np.float32)
    e = np.ones((1, 4), np.float32)
    assert orc.logits(x, e)[0, 0] == 0.0
    # reversed operand order must give the exact 2 under the same rule
    assert orc.logits(x[:, ::-1].copy(), e)[0, 0] == 2.0


def test_logits_uses_fused_multiply_add(orc):
    # acc after the first term: fl((1+2^-12)^2) = 1 + 2^-11 (the 2^-24 tail is a
    # tie, rounded to even).  The second product -(1+2^-12)^2 added with one
    # rounding leaves exactly -2^-24; separately rounded it would cancel to 0.
    a = 1.0 + 2.0 ** -12
    x = np.array([[a, a]], np.float32)
    e = np.array([[a, -a]], np.float32)
    assert orc.logits(x, e)[0, 0] == np.float32(-(2.0 ** -24))


def test_logits_within_standard_dot_bound(orc):
    rng = np.random.default_rng(1)
    T, d, N = 16, 512, 32
    x = rng.standard_normal((T, d)).astype(np.float32)
    E = (rng.standard_normal((N, d)) / math.sqrt(d)).astype(np.float32)
    z = orc.logits(x, E).astype(np.float64)
    exact = x.astype(np.float64) @ E.astype(np.float64).T
    u = 2.0 ** -24
    gamma = d * u / (1 - d * u)
    bound = gamma * (np.abs(x.astype(np.float64)) @ np.abs(E.astype(np.float64)).T)
    assert np.all(np.abs(z - exact) <= bound)


def test_logits_bf16_input_is_exact_widening(orc):
    rng = np.random.default_rng(2)
    xf = rng.standard_normal((4, 64)).astype(np.float32)
    bits = (xf.view(np.uint32) >> 16).astype(np.uint16)  # truncated bf16 values
    widened = (bits.astype(np.uint32) << 16).view(np.float32)
    E = rng.standard_normal((8, 64)).astype(np.float32)
    assert np.array_equal(orc.logits(bits, E), orc.logits(widened, E))


# ------------------------------------------------------------------ sigmoid

def _sigmoid_correctly_rounded(z):
    getcontext().prec = 60
    v = Decimal(1) / (Decimal(1) + (-Decimal(float(z))).exp())
    # round the 60-digit value to the nearest float32
    f64 = float(v)  # nearest double
    f32 = np.float32(f64)
    # resolve a possible double rounding against the exact decimal value
    lo = np.nextafter(f32, np.float32(-np.inf))
    hi = np.nextafter(f32, np.float32(np.inf))
    best = min((f32, lo, hi), key=lambda c: abs(Decimal(float(c)) - v))
    return best


def test_sigmoid_correctly_rounded(orc):
    rng = np.random.default_rng(3)
    z = np.concatenate([rng.standard_normal(3000).astype(np.float32) * 4,
                        np.array([0.0, -0.0, 1e-30, -1e-30, 20.0, -20.0, 80.0, -80.0],
                                 np.float32)])
    s = orc.sigmoid(z)
    ref = np.array([_sigmoid_correctly_rounded(v) for v in z], np.float32)
    mism = np.count_nonzero(s.view(np.uint32) != ref.view(np.uint32))
    assert mism == 0
    assert orc.sigmoid(np.zeros(1, np.float32))[0] == 0.5


# ------------------------------------------------------------------ selection

def _order_key(r, i):
    return (-float(r), i)


def _brute_topk(s, b, k):
    """rank counting: i is chosen iff fewer than k experts beat it."""
    r = (s + b).astype(np.float32)
    r[r == 0] = 0.0
    N = r.size
    chosen = []
    for i in range(N):
        beaten_by = sum(1 for j in range(N) if (r[j] > r[i] or (r[j] == r[i] and j < i)))
        if beaten_by < k:
            chosen.append(i)
    return sorted(chosen, key=lambda i: _order_key(r[i], i))


def _brute_subset(s, b, k, allowed=None):
    """the chosen set maximises the sum of biased keys (distinct keys)"""
    r = (s + b).astype(np.float64)
    cand = range(r.size) if allowed is None else allowed
    best = max(itertools.combinations(cand, k), key=lambda c: (sum(r[list(c)]),
                                                               [-i for i in c]))
    return set(best)


@pytest.mark.parametrize("N,k", [(8, 1), (8, 3), (16, 2), (16, 4), (12, 5)])
def test_select_brute_force(orc, N, k):
    rng = np.random.default_rng(N * 10 + k)
    T = 64
    s = rng.uniform(0.01, 0.99, (T, N)).astype(np.float32)
    b = (rng.standard_normal(N) * 0.05).astype(np.float32)
    idx, gate = orc.select(s, b, k)
    for t in range(T):
        ref = _brute_topk(s[t], b, k)
        assert list(idx[t]) == ref
        assert set(idx[t]) == _brute_subset(s[t], b, k)


def _brute_group(s, b, k, G, TG):
    r = (s + b).astype(np.float32)
    N = r.size
    gs = N // G
    scores = []
    for g in range(G):
        vals = sorted(r[g * gs:(g + 1) * gs].tolist(), reverse=True)
        scores.append(np.float32(np.float32(vals[0]) + np.float32(vals[1])))
    # enumerate group subsets of size TG: the kept subset maximises the sum of
    # group scores, ties to the lexicographically smaller group list
    kept = max(itertools.combinations(range(G), TG),
               key=lambda c: (sum(float(scores[g]) for g in c), [-g for g in c]))
    allowed = [i for i in range(N) if i // gs in kept]
    return _brute_subset(s, b, k, allowed), kept


@pytest.mark.parametrize("N,G,TG,k", [(16, 4, 2, 3), (16, 4, 2, 4), (32, 8, 4, 8),
                                      (16, 8, 3, 2)])
def test_select_group_limited_brute_force(orc, N, G, TG, k):
    rng = np.random.default_rng(N + G * 7 + TG * 3 + k)
    T = 48
    s = rng.uniform(0.01, 0.99, (T, N)).astype(np.float32)
    b = (rng.standard_normal(N) * 0.05).astype(np.float32)
    idx, _ = orc.select(s, b, k, G, TG)
    gs = N // G
    for t in range(T):
        ref, kept = _brute_group(s[t], b, k, G, TG)
        assert set(idx[t]) == ref
        assert all(i // gs in kept for i in idx[t])
        r = (s[t] + b).astype(np.float32)
        order = sorted(idx[t], key=lambda i: _order_key(r[i], i))
        assert list(idx[t]) == order


def test_group_limit_changes_selection(orc):
    # a group holding the 2nd..4th best single experts can lose to a group whose
    # top-2 sum is larger: the group rule must exclude an otherwise-chosen expert
    N, G, TG, k = 8, 4, 1, 2
    s = np.array([[0.10, 0.95, 0.90, 0.20, 0.99, 0.05, 0.30, 0.31]], np.float32)
    b = np.zeros(N, np.float32)
    idx, _ = orc.select(s, b, k, G, TG)
    # groups: {0,1}=1.05, {2,3}=1.10, {4,5}=1.04, {6,7}=0.61 -> keep group 1
    assert list(idx[0]) == [2, 3]
    idx_free, _ = orc.select(s, b, k)
    assert list(idx_free[0]) == [4, 1]


def test_ties_go_to_lower_index(orc):
    rng = np.random.default_rng(5)
    d, N, k = 32, 8, 3
    E = rng.standard_normal((N, d)).astype(np.float32)
    E[5] = E[2]   # experts 2 and 5 identical -> identical logits and scores
    E[6] = E[2]
    x = rng.standard_normal((200, d)).astype(np.float32)
    r = orc.route(x, E, np.zeros(N, np.float32), k, want_scores=True)
    hits = 0
    for t in range(x.shape[0]):
        chosen = set(r["idx"][t])
        if 5 in chosen:
            assert 2 in chosen
        if 6 in chosen:
            assert 2 in chosen and 5 in chosen
        hits += 2 in chosen
    assert hits > 0


def test_negative_zero_equals_positive_zero(orc):
    # keys 0.0 and -0.0 tie; lower index must win
    s = np.array([[0.25, 0.25, 0.5]], np.float32)
    b = np.array([-0.25, np.float32(-0.25), -0.5], np.float32)  # keys +0, +0, 0
    s2 = np.array([[0.0, 0.0, 0.0]], np.float32)
    b2 = np.array([-0.0, 0.0, -0.0], np.float32)
    for ss, bb in ((s, b), (s2, b2)):
        idx, _ = orc.select(ss, bb, 1)
        assert idx[0, 0] == 0


def test_bias_forces_selection(orc):
    rng = np.random.default_rng(6)
    T, N, k = 100, 16, 2
    s = rng.uniform(0.01, 0.99, (T, N)).astype(np.float32)
    b = np.zeros(N, np.float32)
    b[11] = 1.0
    idx, _ = orc.select(s, b, k)
    assert np.all(idx[:, 0] == 11)


# ------------------------------------------------------------------ gates

def test_gates_sum_to_one_and_ignore_bias(orc):
    rng = np.random.default_rng(7)
    T, N, k = 500, 64, 8
    s = rng.uniform(0.01, 0.99, (T, N)).astype(np.float32)
    b1 = (rng.standard_normal(N) * 0.01).astype(np.float32)
    b2 = (rng.standard_normal(N) * 0.01).astype(np.float32)
    i1, g1 = orc.select(s, b1, k)
    i2, g2 = orc.select(s, b2, k)
    sums = g1.astype(np.float64).sum(1)
    assert np.all(np.abs(sums - 1.0) <= k * 2.0 ** -24)
    same = 0
    for t in range(T):
        if set(i1[t]) == set(i2[t]):
            same += 1
            m1 = dict(zip(i1[t], g1[t]))
            m2 = dict(zip(i2[t], g2[t]))
            for e in m1:  # identical bits: the bias never enters a gate value
                assert np.float32(m1[e]).view(np.uint32) == np.float32(m2[e]).view(np.uint32)
    assert same > 0
    # the gate is the normalised affinity of the chosen expert
    t = 0
    S = sum(float(s[t, e]) for e in i1[t])
    for j, e in enumerate(i1[t]):
        assert abs(float(g1[t, j]) - float(s[t, e]) / S) <= 2.0 ** -24


def test_gates_k_equals_n_closed_form(orc):
    rng = np.random.default_rng(8)
    s = rng.uniform(0.01, 0.99, (10, 6)).astype(np.float32)
    idx, g = orc.select(s, np.zeros(6, np.float32), 6)
    for t in range(10):
        ref = s[t].astype(np.float64) / s[t].astype(np.float64).sum()
        got = np.empty(6)
        got[idx[t]] = g[t]
        assert np.allclose(got, ref, rtol=2.0 ** -23, atol=0)


def test_single_expert_gate_is_one(orc):
    rng = np.random.default_rng(9)
    x = rng.standard_normal((5, 16)).astype(np.float32)
    E = rng.standard_normal((1, 16)).astype(np.float32)
    r = orc.route(x, E, np.zeros(1, np.float32), 1)
    assert np.all(r["idx"] == 0) and np.all(r["gate"] == 1.0)


# ------------------------------------------------------------------ counts

def test_counts_sum_and_distinct(orc):
    rng = np.random.default_rng(10)
    T, d, N, k = 300, 64, 32, 6
    x = rng.standard_normal((T, d)).astype(np.float32)
    E = (rng.standard_normal((N, d)) / 8).astype(np.float32)
    b = (rng.standard_normal(N) * 1e-3).astype(np.float32)
    r = orc.route(x, E, b, k, 4, 2)
    assert r["counts"].sum() == T * k
    assert np.array_equal(r["counts"], np.bincount(r["idx"].ravel(), minlength=N))
    for t in range(T):
        assert len(set(r["idx"][t])) == k


def test_route_is_composition(orc):
    rng = np.random.default_rng(11)
    T, d, N, k = 40, 48, 16, 4
    x = rng.standard_normal((T, d)).astype(np.float32)
    E = rng.standard_normal((N, d)).astype(np.float32)
    b = (rng.standard_normal(N) * 1e-2).astype(np.float32)
    r = orc.route(x, E, b, k, 4, 2, want_scores=True)
    s = orc.sigmoid(orc.logits(x, E))
    assert np.array_equal(r["scores"], s)
    idx, g = orc.select(s, b, k, 4, 2)
    assert np.array_equal(r["idx"], idx) and np.array_equal(r["gate"], g)


def test_route_shape_errors(orc):
    s = np.zeros((1, 16), np.float32)
    b = np.zeros(16, np.float32)
    with pytest.raises(ValueError):
        orc.select(s, b, 17)
    with pytest.raises(ValueError):
        orc.select(s, b, 2, 5, 2)      # N % G != 0
    with pytest.raises(ValueError):
        orc.select(s, b, 9, 4, 2)      # k > TG * N/G


def test_nan_keys_rank_lowest(orc):
    """NaN is not covered by the pages; the reading: a NaN key (s + b) ranks as
    -inf, below every number, with the lower index first among equals, so a
    token always gets k distinct valid experts."""
    nan = np.float32(np.nan)
    s = np.array([[nan, 0.5, nan, 0.7, 0.1, nan],
                  [nan] * 6,
                  [0.2, nan, 0.9, nan, nan, nan]], np.float32)
    b = np.zeros(6, np.float32)
    idx, gate = orc.select(s, b, 4)
    assert idx[0].tolist() == [3, 1, 4, 0]
    assert idx[1].tolist() == [0, 1, 2, 3]
    assert idx[2].tolist() == [2, 0, 1, 3]
    # gates of a token with a NaN score among its chosen ones are NaN; the others are finite
    assert np.all(np.isnan(gate[1]))
    idx2, gate2 = orc.select(s[:, [1, 3, 4]], np.zeros(3, np.float32), 3)
    assert np.all(np.isfinite(gate2[0]))


def test_nan_group_scores_rank_lowest(orc):
    """Group-limited selection with NaN keys: a group whose two best keys are
    NaN (or whose score is +inf + -inf from the bias) scores -inf and ranks
    below every finite group, lower group index first among equals."""
    nan = np.float32(np.nan)
    N, G, TG, k = 8, 4, 2, 3
    s = np.full((2, N), 0.5, np.float32)
    s[0, 0:2] = nan          # group 0 all NaN
    s[0, 4:6] = [0.9, 0.8]   # group 2 best
    s[1, :] = nan            # every key NaN: groups 0, 1 kept, experts 0, 1, 2
    b = np.zeros(N, np.float32)
    idx, _ = orc.select(s, b, k, G, TG)
    assert idx[0].tolist() == [4, 5, 2]
    assert idx[1].tolist() == [0, 1, 2]
    # +inf bias on expert 7 and -inf on expert 6: group 3 scores inf + -inf = NaN -> -inf
    b2 = np.zeros(N, np.float32)
    b2[6], b2[7] = -np.inf, np.inf
    idx3, _ = orc.select(np.full((1, N), 0.5, np.float32), b2, 2, G, 1)
    assert idx3[0].tolist() == [0, 1]
