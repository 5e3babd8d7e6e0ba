"""HIP graph replay of the layer's forward step (MoeLayer.capture_forward /
replay): every replay equals, bit for bit, the eager step of an identical
layer on the same inputs, over a run of steps whose bias updates feed the
next step's routing.  Each replay reads a fresh batch written into the
captured input buffer, and eager work with host synchronisations runs between
the replays."""
import numpy as np
import pytest
import torch

import moe_inputs
from parity_util import log
from sparse_moe_layer_bias_amd.layer import MoeLayer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the graph tests need the HIP library on an MI355X")
    yield
    torch.cuda.synchronize()


CASES = [
    ("tiny_fp32", {}),
    ("mid_bf16", dict(T=300, G=8, TG=3)),        # gathered token rows, group-limited routing
    ("mid_bf16", dict(T=256, fp8=True)),         # FP8 expert GEMMs
]


def _bits(t):
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    elif t.dtype == torch.float32:
        t = t.view(torch.int32)
    return t.cpu().numpy()


@pytest.mark.parametrize("name,over", CASES)
def test_graph_replay_matches_eager_steps(name, over):
    cfg = dict(moe_inputs.CONFIGS[name])
    cfg.update(over)
    log("graph case", name, over)
    dev = moe_inputs.make_layer_inputs(cfg, 0, "cuda")
    mk = lambda: MoeLayer(cfg, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"])
    eager, graphed = mk(), mk()
    E = dev["centroids"]
    bias_e = dev["bias"].clone()
    bias_g = dev["bias"].clone()
    x_g = torch.empty_like(dev["x"])  # the captured input buffer
    x_g.copy_(dev["x"])
    graphed.capture_forward(x_g, E, bias_g)
    torch.cuda.synchronize()
    for step in range(5):
        x = moe_inputs.make_router_inputs(cfg, 100 + step, "cuda")["x"]
        out_e = eager.forward(x, E, bias_e).clone()
        x_g.copy_(x)
        out_g = graphed.replay().clone()
        torch.cuda.synchronize()
        for what, a, b in (("out", out_e, out_g), ("idx", eager.idx, graphed.idx),
                           ("gate", eager.gate, graphed.gate),
                           ("counts", eager.counts, graphed.counts),
                           ("bias", bias_e, bias_g)):
            assert np.array_equal(_bits(a), _bits(b)), "step %d: %s differs" % (step, what)
        # eager work of the program's own between the replays
        (x.float() * 2.0).sum().item()
        torch.cuda.synchronize()
    # the bias moved: the replays really took the update path
    assert not np.array_equal(_bits(bias_g), _bits(dev["bias"]))


def test_replay_before_capture_is_an_error():
    cfg = dict(moe_inputs.CONFIGS["tiny_fp32"])
    dev = moe_inputs.make_layer_inputs(cfg, 0, "cuda")
    layer = MoeLayer(cfg, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"])
    with pytest.raises(RuntimeError):
        layer.replay()
