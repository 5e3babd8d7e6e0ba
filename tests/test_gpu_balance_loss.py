"""GPU parity of moe_seq_balance_loss (through the C ABI) against the oracle.

The call evaluates the sequence-wise balance loss that the DeepSeek-V3 report
reading guide (xyznot.com/de), "Methode" item 2, last sentence, names beside
the bias rule (alpha = 0.0001), under the reading both sides implement:
per sequence of S consecutive tokens, alpha * sum_i f_i P_i (f_i the load of
expert i relative to the uniform share, P_i its mean normalised affinity).
Inputs are seeded affinities and routings of the layer's shapes; both sides
evaluate in double and round once, so the per-sequence values agree to well
within 1e-6 relative (the fp32 bar of 1e-5).  Cases cover one and many
sequences, sequences shorter than, equal to and ragged against the 64-token
chunks of the partial pass, N up to the ABI limit of 1024 with k = 64, and
the loss of a layer step's own routing.
"""
import numpy as np
import pytest
import torch

import moe_inputs
import sparse_moe_layer_bias_amd as moe
from parity_util import Guards, log
from sparse_moe_layer_bias_amd.layer import MoeLayer

pytestmark = pytest.mark.gpu

RTOL = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the parity tests need the HIP library on an MI355X")
    moe.lib()
    yield
    torch.cuda.synchronize()


def _inputs(T, N, k, seed):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((T, N)) * 2.0
    s = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    # a skewed routing: keys favour low expert indices
    key = rng.random((T, N)) - np.linspace(0.0, 0.5, N)[None, :]
    idx = np.argsort(key, axis=1)[:, :k].astype(np.int32)
    return s, idx


def _gpu_loss(s, idx, S, alpha=1e-4):
    T, N = s.shape
    k = idx.shape[1]
    c = moe.make_cfg(T, 128, N, k, 1, 1, 0, 0, "f32")
    g = Guards()
    loss = g.empty((T // S,), torch.float32, "loss")
    ws = g.empty((max(moe.moe_seq_balance_loss_workspace_size(c, S), 16),), torch.uint8, "ws")
    moe.moe_seq_balance_loss(c, S, alpha, torch.from_numpy(s).cuda(),
                             torch.from_numpy(idx).cuda(), loss, ws)
    torch.cuda.synchronize()
    g.check()
    return loss.cpu().numpy()


CASES = [  # (T, N, k, S)
    (64, 16, 2, 64),       # one sequence, one chunk
    (64, 16, 2, 16),       # four short sequences
    (64, 16, 2, 1),        # every token its own sequence
    (2072, 64, 8, 37),     # sequences shorter than a chunk, odd length
    (2000, 64, 8, 200),    # ragged last chunk of each sequence
    (2048, 64, 8, 2048),
    (8192, 256, 8, 4096),  # V3 routing shape, two sequences of 4096
    (8192, 256, 8, 8192),
    (256, 1024, 64, 128),  # the ABI's largest N and k
    (130, 100, 5, 65),     # N not a multiple of 64
]


@pytest.mark.parametrize("T,N,k,S", CASES)
def test_seq_balance_loss_matches_oracle(orc, T, N, k, S):
    log("seq balance loss T=%d N=%d k=%d S=%d" % (T, N, k, S))
    s, idx = _inputs(T, N, k, seed=T + N + S)
    got = _gpu_loss(s, idx, S)
    ref = orc.seq_balance_loss(s, idx, S)
    np.testing.assert_allclose(got, ref, rtol=RTOL, atol=0)
    # same bits on a second call
    assert np.array_equal(_gpu_loss(s, idx, S), got)


def test_equal_affinities_give_alpha_on_gpu():
    T, N, k, S = 512, 64, 8, 128
    _, idx = _inputs(T, N, k, seed=7)
    got = _gpu_loss(np.full((T, N), 0.25, np.float32), idx, S)
    assert np.all(got == np.float32(1e-4)), got


def test_layer_step_balance_loss(orc):
    # the loss of a bf16 layer step's own routing (scores and idx from moe_route)
    cfg = dict(moe_inputs.CONFIGS["mid_bf16"])
    inp = moe_inputs.make_layer_inputs(cfg, 0, "cpu")
    dev = {n: v.cuda() for n, v in inp.items()}
    layer = MoeLayer(cfg, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"])
    bias = dev["bias"].clone()
    layer.route(dev["x"], dev["centroids"], bias)
    S = 512
    got = layer.seq_balance_loss(S).cpu().numpy()
    torch.cuda.synchronize()
    s = moe_inputs.to_host(layer.scores)
    idx = moe_inputs.to_host(layer.idx)
    ref = orc.seq_balance_loss(s, idx, S)
    np.testing.assert_allclose(got, ref, rtol=RTOL, atol=0)
    assert got.shape == (cfg["T"] // S,)
