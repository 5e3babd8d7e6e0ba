"""Pins for the oracle's sequence-wise balance loss.

The DeepSeek-V3 report reading guide (xyznot.com/de), "Methode" item 2, last
sentence, names a minimal sequence-wise balance loss (alpha = 0.0001) beside
the bias rule; no page prints its formula.  The oracle's reading: per
sequence of S consecutive tokens, alpha * sum_i f_i P_i, with f_i the load of
expert i relative to the uniform share k S / N and P_i the mean over the
sequence of its affinity normalised over all N experts.  The pins below are
what that reading fixes without the oracle's code: closed forms, a worked
example by hand, and invariances (row scaling, token order, expert labels,
sequence locality).
"""
import numpy as np
import pytest

ALPHA = np.float32(1e-4)


def _routing(rng, T, N, k):
    return np.stack([rng.choice(N, k, replace=False) for _ in range(T)]).astype(np.int32)


def _scores(rng, T, N):
    # sigmoid affinities lie in (0, 1)
    return (1.0 / (1.0 + np.exp(-rng.standard_normal((T, N))))).astype(np.float32)


@pytest.mark.parametrize("T,N,k,S", [(64, 16, 2, 16), (96, 64, 8, 32), (40, 256, 8, 8),
                                     (7, 5, 5, 7), (12, 9, 3, 1)])
def test_equal_affinities_give_alpha_for_any_routing(orc, T, N, k, S):
    # P_i = 1/N for every expert, and sum_i f_i = N: the loss is alpha
    rng = np.random.default_rng(T * N + k)
    idx = _routing(rng, T, N, k)
    for c in (1.0, 0.37, 1e-3):
        loss = orc.seq_balance_loss(np.full((T, N), c, np.float32), idx, S)
        assert np.all(loss == ALPHA), loss


@pytest.mark.parametrize("N,k,S", [(16, 2, 4), (256, 8, 16), (64, 1, 3)])
def test_collapsed_sequence_gives_alpha_n_over_k(orc, N, k, S):
    # every token on experts 0..k-1, holding all of its affinity there:
    # f_i = N/k and P_i = 1/k for those k experts -> alpha * N / k
    s = np.zeros((S, N), np.float32)
    s[:, :k] = 0.5
    idx = np.tile(np.arange(k, dtype=np.int32), (S, 1))
    loss = orc.seq_balance_loss(s, idx, S)
    assert loss[0] == np.float32(np.float64(ALPHA) * N / k)


def test_worked_example_by_hand(orc):
    # two tokens, two experts, top-1, one sequence of 2.
    # token 0: affinities (3, 1) -> normalised (3/4, 1/4); token 1: (1, 1) -> (1/2, 1/2)
    # P = ((3/4 + 1/2) / 2, (1/4 + 1/2) / 2) = (5/8, 3/8)
    s = np.array([[3.0, 1.0], [1.0, 1.0]], np.float32)
    # both tokens on expert 0: f = N/(kS) * counts = (2, 0) -> 2 * 5/8 = 5/4
    assert orc.seq_balance_loss(s, np.array([[0], [0]], np.int32), 2)[0] == \
        np.float32(np.float64(ALPHA) * 1.25)
    # one token each: f = (1, 1) -> 5/8 + 3/8 = 1
    assert orc.seq_balance_loss(s, np.array([[0], [1]], np.int32), 2)[0] == ALPHA
    # both on expert 1: f = (0, 2) -> 2 * 3/8 = 3/4
    assert orc.seq_balance_loss(s, np.array([[1], [1]], np.int32), 2)[0] == \
        np.float32(np.float64(ALPHA) * 0.75)
    # each token its own sequence (S = 1): token 0 on expert 0 -> 2 * 3/4 = 3/2;
    # token 1 on expert 0 -> 2 * 1/2 = 1
    got = orc.seq_balance_loss(s, np.array([[0], [0]], np.int32), 1)
    assert got[0] == np.float32(np.float64(ALPHA) * 1.5) and got[1] == ALPHA


def test_row_scaling_invariance(orc):
    # the affinities enter only normalised per token: scaling a token's row by
    # a power of two changes no bit, by any other positive factor only rounding
    rng = np.random.default_rng(1)
    T, N, k, S = 48, 32, 4, 12
    s, idx = _scores(rng, T, N), _routing(rng, T, N, k)
    ref = orc.seq_balance_loss(s, idx, S)
    p2 = s * np.float32(2.0) ** rng.integers(-8, 9, (T, 1)).astype(np.float32)
    assert np.array_equal(orc.seq_balance_loss(p2, idx, S), ref)
    c = s * rng.uniform(0.1, 10.0, (T, 1)).astype(np.float32)
    np.testing.assert_allclose(orc.seq_balance_loss(c, idx, S), ref, rtol=1e-6)


def test_token_order_within_a_sequence(orc):
    rng = np.random.default_rng(2)
    T, N, k, S = 64, 16, 2, 16
    s, idx = _scores(rng, T, N), _routing(rng, T, N, k)
    ref = orc.seq_balance_loss(s, idx, S)
    perm = np.concatenate([b * S + rng.permutation(S) for b in range(T // S)])
    np.testing.assert_allclose(orc.seq_balance_loss(s[perm], idx[perm], S), ref, rtol=1e-6)
    # slot order within a token does not matter either
    np.testing.assert_array_equal(orc.seq_balance_loss(s, idx[:, ::-1].copy(), S), ref)


def test_expert_relabelling(orc):
    rng = np.random.default_rng(3)
    T, N, k, S = 32, 24, 3, 8
    s, idx = _scores(rng, T, N), _routing(rng, T, N, k)
    ref = orc.seq_balance_loss(s, idx, S)
    pi = rng.permutation(N)  # new label of expert i is pi[i]
    s2 = np.empty_like(s)
    s2[:, pi] = s
    np.testing.assert_allclose(orc.seq_balance_loss(s2, pi[idx].astype(np.int32), S), ref,
                               rtol=1e-6)


def test_sequences_are_independent(orc):
    rng = np.random.default_rng(4)
    N, k, S = 16, 2, 10
    a, b = _scores(rng, S, N), _scores(rng, S, N)
    ia, ib = _routing(rng, S, N, k), _routing(rng, S, N, k)
    both = orc.seq_balance_loss(np.concatenate([a, b]), np.concatenate([ia, ib]), S)
    assert both[0] == orc.seq_balance_loss(a, ia, S)[0]
    assert both[1] == orc.seq_balance_loss(b, ib, S)[0]


def test_load_concentration_raises_the_loss(orc):
    # with the affinities held fixed and positive, moving one token's slot
    # onto the expert with the largest mean affinity raises f . P
    rng = np.random.default_rng(5)
    N, k, S = 8, 1, 16
    s = _scores(rng, S, N)
    idx = _routing(rng, S, N, k)
    P = (s / s.sum(1, keepdims=True)).mean(0)
    top = int(np.argmax(P))
    t = int(np.flatnonzero(idx[:, 0] != top)[0])
    moved = idx.copy()
    moved[t, 0] = top
    assert orc.seq_balance_loss(s, moved, S)[0] > orc.seq_balance_loss(s, idx, S)[0]


def test_rejects_partial_sequences(orc):
    with pytest.raises(ValueError):
        orc.seq_balance_loss(np.ones((10, 4), np.float32), np.zeros((10, 1), np.int32), 3)
