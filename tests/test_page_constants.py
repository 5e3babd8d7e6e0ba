"""The printed constants of the pages (tests/golden/page_constants.json) against
the oracle and the workload table."""
import json
import os

import numpy as np

import moe_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")


def _g():
    with open(GOLDEN) as f:
        return json.load(f)


def test_gamma(orc):
    assert orc.GAMMA == np.float32(_g()["gamma"]["value"])


def test_fp8_max_is_largest_code(orc):
    m = _g()["fp8_max"]["value"]
    dec = orc.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert np.nanmax(dec) == m
    assert orc.e4m3_encode(np.array([m], np.float32))[0] == 0x7E


def test_tile_and_block_sizes(orc):
    g = _g()
    assert g["act_tile"]["value"] == [1, 128] and g["weight_block"]["value"] == [128, 128]
    x = np.ones((1, 256), np.float32)
    x[0, 128:] = 2.0
    _, s = orc.quant_act_fp8(x)
    assert s.shape == (1, 2) and s[0, 0] * 2 == s[0, 1]
    w = np.ones((256, 256), np.float32)
    w[128:, :128] = 4.0
    _, sw = orc.quant_weight_fp8(w)
    assert sw.shape == (2, 2) and sw[1, 0] == 4 * sw[0, 0] and sw[0, 1] == sw[0, 0]


def test_v3_shape_matches_pages():
    g = _g()
    c = moe_inputs.CONFIGS["v3_bf16"]
    assert c["N"] == g["n_routed"]["value"] and c["k"] == g["n_active"]["value"]
    assert moe_inputs.CONFIGS["v3_fp8"]["N"] == g["n_routed"]["value"]


def test_seq_balance_alpha(orc):
    # the default coefficient of the sequence-wise balance loss is the pages' alpha
    import inspect
    a = inspect.signature(orc.seq_balance_loss).parameters["alpha"].default
    assert a == _g()["seq_balance_alpha"]["value"]
