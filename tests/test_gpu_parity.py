"""GPU parity: libmoe (HIP, through the C ABI) against the CPU oracle on the
same seeded inputs.

Bit for bit: scores, expert indices, gates, counts, offsets, src_token,
dst_row, permuted rows, FP8 codes and scales, and the bias trajectory.
Within tolerance (see parity_util): expert outputs and the layer output.

Small layers (tiny fp32, mid bf16, ragged and degenerate shapes) are compared
in full.  The DeepSeek-V3-shaped layer is compared on sampled tokens and rows
the oracle computes one by one, plus properties checked at full size.
"""
import numpy as np
import pytest
import torch

import moe_inputs
import sparse_moe_layer_bias_amd as moe
from parity_util import (RTOL, ExpertCodes, RowsOf, assert_bits, assert_close, assert_close_fp8,
                         check_fp8_expert_split, guard_layer, host_inputs, log, small_layer_inputs)
from sparse_moe_layer_bias_amd.layer import MoeLayer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the parity tests need the HIP library on an MI355X")
    moe.lib()
    yield
    torch.cuda.synchronize()


_last_x = [None]


def _check_gathered_rows(layer):
    """moe_expert_ffn_gather (token rows read through src_token) on the state
    of a layer that ran with the permuted copy: y_perm and y_shared bit for
    bit equal to the layer's"""
    import sparse_moe_layer_bias_amd as m
    y = torch.empty_like(layer.y_perm)
    ys = torch.empty_like(layer.y_shared) if layer.y_shared is not None else None
    x = layer.x_q if layer.fp8 else _last_dev_x[0]
    m.moe_expert_ffn_gather(layer.cfg, x, layer.x_s if layer.fp8 else None, layer.src_token,
                            layer.offsets, layer.w13, layer.w13_s, layer.w2, layer.w2_s, y,
                            layer.ws13, layer.ws13_s, layer.ws2, layer.ws2_s, ys, layer.workspace)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.uint8), layer.y_perm.view(torch.uint8)), "y_perm (gathered)"
    if ys is not None:
        assert torch.equal(ys.view(torch.uint8), layer.y_shared.view(torch.uint8)), \
            "y_shared (gathered)"


_last_dev_x = [None]


def _run_small(cfg_name, orc, T=None, residual=True, seed=0, gather_rows=None, **over):
    cfg = dict(moe_inputs.CONFIGS[cfg_name])
    cfg.update(over)
    c, inp, dev = small_layer_inputs(cfg, seed, T)
    _last_x[0] = inp["x"]
    _last_dev_x[0] = dev["x"]
    log("case", cfg_name, "T=%d" % c["T"], over, "seed", seed, "gather_rows", gather_rows)
    layer = MoeLayer(c, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"], gather_rows=gather_rows)
    guards = guard_layer(layer)
    bias = guards.like(dev["bias"], "bias", copy=True)
    out = layer.forward(dev["x"], dev["centroids"], bias, residual=residual)
    torch.cuda.synchronize()
    guards.check()
    ref = orc.layer_forward(host_inputs(inp), c, residual=residual)
    return c, layer, out, bias, ref


LAYER_CASES = [
    ("tiny_fp32", {}),
    ("mid_bf16", {}),
    ("tiny_fp32", dict(T=1)),
    ("tiny_fp32", dict(T=200)),                      # ragged tails
    ("mid_bf16", dict(T=77)),                        # ragged, many empty experts
    ("mid_bf16", dict(T=300, G=8, TG=3)),            # group-limited
    ("mid_bf16", dict(T=96, k=1, N=8)),              # k = 1
    ("mid_bf16", dict(T=130, N=1, k=1)),             # one expert: gate 1
    ("mid_bf16", dict(T=64, d=256, I=128, Is=256)),  # Is != I
    ("mid_bf16", dict(T=64, d=256, I=256, Is=128)),
    ("mid_bf16", dict(T=100, d=384, I=256, Is=128)),  # d % 256 != 0: half a down tile
    ("mid_bf16", dict(T=1000, N=2, k=1)),             # >320 rows per expert: several tiles
    ("mid_bf16", dict(T=96, N=1024, k=64, d=256, I=128, Is=128)),  # largest N and top_k accepted
    ("mid_bf16", dict(T=64, N=100, k=6)),             # N % 64 != 0: a partial router tile
    ("mid_bf16", dict(T=50, N=16, k=16)),             # k = N: every expert chosen
    ("mid_bf16", dict(T=200, N=128, k=8, G=64, TG=4)),  # 64 groups of 2 experts
    # one expert (and the shared one) with exactly T rows: the edges of a
    # wave's 160-row token half and of the 320-row tile
    ("mid_bf16", dict(T=160, N=1, k=1, d=256, I=256, Is=128)),
    ("mid_bf16", dict(T=161, N=1, k=1, d=256, I=256, Is=128)),
    ("mid_bf16", dict(T=320, N=1, k=1, d=256, I=256, Is=128)),
    ("mid_bf16", dict(T=321, N=1, k=1, d=256, I=256, Is=128)),
]


@pytest.mark.parametrize("name,over", LAYER_CASES)
def test_layer_parity_small(orc, name, over):
    over = dict(over)
    T = over.pop("T", None)
    c, layer, out, bias, ref = _run_small(name, orc, T=T, **over)
    dt = c["dtype"]
    rtol = RTOL[dt]
    assert_bits(moe_inputs.to_host(layer.scores), ref["scores"], "scores")
    assert_bits(moe_inputs.to_host(layer.idx), ref["idx"], "idx")
    assert_bits(moe_inputs.to_host(layer.gate), ref["gate"], "gate")
    assert_bits(moe_inputs.to_host(layer.counts), ref["counts"], "counts")
    assert_bits(moe_inputs.to_host(layer.offsets), ref["offsets"], "offsets")
    assert_bits(moe_inputs.to_host(layer.src_token), ref["src_token"], "src_token")
    assert_bits(moe_inputs.to_host(layer.dst_row), ref["dst_row"], "dst_row")
    assert_close(moe_inputs.to_host(layer.y_perm), ref["y_perm"], rtol, "y_perm")
    assert_close(moe_inputs.to_host(layer.y_shared), ref["y_shared"], rtol, "y_shared")
    assert_close(moe_inputs.to_host(out), ref["out"], rtol, "out")
    assert_bits(moe_inputs.to_host(bias), ref["new_bias"], "bias after update")
    if layer.gather_rows:
        # bf16 layers read the token rows through src_token by default: the
        # same layer with the permuted copy must give x_perm bit for bit and
        # the very same expert outputs and layer output
        c2, layer2, out2, _, _ = _run_small(name, orc, T=T, gather_rows=False, **over)
        assert_bits(moe_inputs.to_host(layer2.x_perm), ref["x_perm"], "x_perm")
        for n, a, b in (("y_perm", layer.y_perm, layer2.y_perm),
                        ("y_shared", layer.y_shared, layer2.y_shared), ("out", out, out2)):
            assert_bits(moe_inputs.to_host(a), moe_inputs.to_host(b), n + ": gathered == permuted")
    else:
        assert_bits(moe_inputs.to_host(layer.x_perm), ref["x_perm"], "x_perm")


FP8_CASES = [
    ("mid_bf16", dict(T=256)),
    ("mid_bf16", dict()),                                  # full mid size, T=2048
    ("mid_bf16", dict(T=77)),                              # ragged, empty experts
    ("mid_bf16", dict(T=300, G=8, TG=3)),                  # group-limited
    ("mid_bf16", dict(T=64, d=256, I=128, Is=256)),        # Is != I
    ("mid_bf16", dict(T=700, d=384, N=4, k=2, I=256, Is=128)),  # >256 rows/expert, d%256 != 0
    ("mid_bf16", dict(T=1)),                               # one token: 8 one-row tiles
    ("mid_bf16", dict(T=1000, N=2, k=1)),                  # >320 rows/expert: several tiles
    ("mid_bf16", dict(T=40, d=65536, N=2, k=1, I=128, Is=128)),  # K at the FP8 limit: 512 scale blocks
    ("mid_bf16", dict(T=320, N=1, k=1, d=256, I=256, Is=128)),   # one full 320-row tile
    ("mid_bf16", dict(T=321, N=1, k=1, d=256, I=256, Is=128)),   # and a second tile of one row
]


@pytest.mark.parametrize("name,over", FP8_CASES)
def test_layer_parity_fp8_small(orc, name, over):
    """FP8 E4M3 expert GEMMs (1x128 activation tiles, 128x128 weight blocks,
    fp32 promotion per 128-K block) against the oracle's FP8 path."""
    over = dict(over)
    T = over.pop("T", None)
    c, layer, out, bias, ref = _run_small(name, orc, T=T, fp8=True, gather_rows=False, **over)
    _check_gathered_rows(layer)
    assert_bits(moe_inputs.to_host(layer.idx), ref["idx"], "idx")
    assert_bits(moe_inputs.to_host(layer.gate), ref["gate"], "gate")
    assert_bits(moe_inputs.to_host(layer.x_q), ref["x_q"], "x codes")
    assert_bits(moe_inputs.to_host(layer.x_s).view(np.uint32), ref["x_s"].view(np.uint32),
                "x scales")
    assert_bits(moe_inputs.to_host(layer.x_perm), ref["x_q_perm"], "permuted codes")
    assert_bits(moe_inputs.to_host(layer.x_perm_s).view(np.uint32),
                ref["x_s_perm"].view(np.uint32), "permuted scales")
    assert_bits(moe_inputs.to_host(layer.dst_row), ref["dst_row"], "dst_row")
    check_fp8_expert_split(orc, layer, ref, moe_inputs.to_host(_last_x[0]))
    assert_bits(moe_inputs.to_host(bias), ref["new_bias"], "bias after update")


def test_fp8_block_scales_far_apart(orc):
    """FP8 promotion with block scales that jump by 2^60 from one 128-wide K
    block to the next, all-zero blocks (scale 0) in activations and weights,
    and a block scale at the bottom of the normal fp32 range.  The exact
    block sums scaled by s_x * s_w (oracle) must survive the kernel's
    accumulation order."""
    cfg = dict(moe_inputs.CONFIGS["mid_bf16"], T=160, fp8=True)
    c = dict(cfg)
    inp = moe_inputs.make_layer_inputs(c, 5, "cpu")
    x, w13, w2 = inp["x"].float(), inp["w13"].float(), inp["w2"].float()
    ws13, ws2 = inp["ws13"].float(), inp["ws2"].float()
    d = c["d"]
    # activations: K blocks of very different magnitude, per row pattern
    x[:, 0:128] *= 2.0 ** 30
    x[:, 128:256] *= 2.0 ** -30
    x[::3, 256:384] = 0
    x[1::4, 384:512] *= 2.0 ** -100
    # weights: W1/W3 and W2 blocks scaled the other way, some all-zero blocks
    for w in (w13, ws13):
        w[..., 0:128] *= 2.0 ** -30
        w[..., 128:256] *= 2.0 ** 30
        w[..., :128, 256:384] = 0
    for w in (w2, ws2):
        w[..., :, 0:128] *= 2.0 ** 20
        w[..., :128, 128:256] = 0
    inp.update(x=x.to(torch.bfloat16), w13=w13.to(torch.bfloat16), w2=w2.to(torch.bfloat16),
               ws13=ws13.to(torch.bfloat16), ws2=ws2.to(torch.bfloat16))
    dev = {k: v.cuda() for k, v in inp.items()}
    log("case fp8 far-apart block scales T=%d" % c["T"])
    layer = MoeLayer(c, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"], gather_rows=False)
    out = layer.forward(dev["x"], dev["centroids"], dev["bias"].clone())
    torch.cuda.synchronize()
    ref = orc.layer_forward(host_inputs(inp), c, residual=True)
    assert np.all(np.isfinite(ref["y_perm"].astype(np.float64))), "oracle overflowed"
    assert_bits(moe_inputs.to_host(layer.idx), ref["idx"], "idx")
    assert_bits(moe_inputs.to_host(layer.x_perm), ref["x_q_perm"], "permuted codes")
    check_fp8_expert_split(orc, layer, ref, moe_inputs.to_host(inp["x"]))


def test_layer_without_residual(orc):
    c, layer, out, bias, ref = _run_small("tiny_fp32", orc, residual=False)
    assert_close(moe_inputs.to_host(out), ref["out"], RTOL["f32"], "out (no residual)")


def test_deterministic_bytes(orc):
    cfg = dict(moe_inputs.CONFIGS["mid_bf16"])
    c, inp, dev = small_layer_inputs(cfg, 3, 512)
    outs = []
    for _ in range(2):
        layer = MoeLayer(c, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"])
        b = dev["bias"].clone()
        o = layer.forward(dev["x"], dev["centroids"], b).clone()
        torch.cuda.synchronize()
        outs.append((moe_inputs.to_host(o), moe_inputs.to_host(layer.dst_row),
                     moe_inputs.to_host(b)))
    for a, b in zip(*outs):
        assert_bits(a, b, "run-to-run")


def test_ties_choose_lower_index_on_gpu(orc):
    """Duplicate centroids give identical scores; the lower index must win."""
    cfg = dict(moe_inputs.CONFIGS["mid_bf16"], T=256, N=16, k=3)
    c, inp, dev = small_layer_inputs(cfg, 5)
    E = dev["centroids"].clone()
    E[9] = E[4]
    E[13] = E[4]
    bias = torch.zeros(16, device="cuda")
    layer = MoeLayer(c, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"])
    layer.route(dev["x"], E, bias)
    torch.cuda.synchronize()
    h = host_inputs(inp)
    r = orc.route(h["x"], moe_inputs.to_host(E), np.zeros(16, np.float32), 3)
    assert_bits(moe_inputs.to_host(layer.idx), r["idx"], "idx with ties")
    idx = moe_inputs.to_host(layer.idx)
    assert any(4 in row for row in idx)
    for row in idx:
        if 9 in row:
            assert 4 in row


def test_bias_forces_expert(orc):
    cfg = dict(moe_inputs.CONFIGS["mid_bf16"], T=128)
    c, inp, dev = small_layer_inputs(cfg, 6)
    bias = torch.zeros(cfg["N"], device="cuda")
    bias[37] = 1.0
    layer = MoeLayer(c, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"])
    layer.route(dev["x"], dev["centroids"], bias)
    torch.cuda.synchronize()
    assert np.all(moe_inputs.to_host(layer.idx)[:, 0] == 37)


def test_zero_tokens():
    cfg = dict(moe_inputs.CONFIGS["mid_bf16"])
    c, inp, dev = small_layer_inputs(cfg, 0, 1)
    c0 = dict(c, T=0)
    layer = MoeLayer(c0, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"])
    x = torch.empty((0, c["d"]), dtype=torch.bfloat16, device="cuda")
    b = dev["bias"].clone()
    layer.forward(x, dev["centroids"], b)
    torch.cuda.synchronize()
    assert np.all(moe_inputs.to_host(layer.counts) == 0)
    assert np.all(moe_inputs.to_host(layer.offsets) == 0)
    # every expert is underloaded against a mean of 0?  mean = 0: counts == mean -> unchanged
    assert_bits(moe_inputs.to_host(b), moe_inputs.to_host(dev["bias"]), "bias (T=0)")


# ------------------------------------------------------------------ FP8 bytes

def test_fp8_activation_codes_bit_exact(orc):
    cfg = dict(moe_inputs.CONFIGS["mid_bf16"], T=96, fp8=True)
    c, inp, dev = small_layer_inputs(cfg, 7)
    x = dev["x"].clone()
    x[3, 128:256] = 0          # an all-zero tile
    x[5, :] *= 1000
    x[6, :] *= 1e-3
    layer = MoeLayer(c, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"], gather_rows=False)
    layer.route(x, dev["centroids"], dev["bias"])
    layer.permute(x)
    torch.cuda.synchronize()
    xh = moe_inputs.to_host(x)
    q, s = orc.quant_act_fp8(xh)
    assert_bits(moe_inputs.to_host(layer.x_q), q, "x codes")
    assert_bits(moe_inputs.to_host(layer.x_s).view(np.uint32), s.view(np.uint32), "x scales")
    r = orc.route(xh, moe_inputs.to_host(dev["centroids"]), moe_inputs.to_host(dev["bias"]),
                  c["k"])
    off, src, dst = orc.permute(r["idx"], c["N"])
    assert_bits(moe_inputs.to_host(layer.x_perm), orc.gather_rows(q, src), "permuted codes")
    assert_bits(moe_inputs.to_host(layer.x_perm_s).view(np.uint32),
                orc.gather_rows(s, src).view(np.uint32), "permuted scales")


def test_fp8_weight_codes_bit_exact(orc):
    from sparse_moe_layer_bias_amd.layer import quantize_weights_fp8
    g = torch.Generator().manual_seed(11)
    w = (torch.randn((3, 256, 384), generator=g) / 20).to(torch.bfloat16)
    w[1, :128, :128] = 0
    w[2, 128:, 256:] *= 300
    wd = w.cuda()
    q, s = quantize_weights_fp8(wd)
    torch.cuda.synchronize()
    rq, rs = orc.quant_weight_fp8(moe_inputs.to_host(w))
    assert_bits(moe_inputs.to_host(q), rq, "weight codes")
    assert_bits(moe_inputs.to_host(s).view(np.uint32), rs.view(np.uint32), "weight scales")


def test_e4m3_encoder_every_midpoint(orc):
    """The GPU quantiser at every E4M3 code midpoint and its neighbours: rows
    whose amax is 448 give scale 1, so the codes are the encoder's own."""
    table = orc.e4m3_decode(np.arange(128, dtype=np.uint8))
    pos = np.sort(table[np.isfinite(table)].astype(np.float64))
    vals = []
    for a, b in zip(pos[:-1], pos[1:]):
        m = np.float32((a + b) / 2)
        vals += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(1e9)),
                 np.float32(a)]
    vals = np.array(vals, np.float32)
    vals = np.concatenate([vals, -vals])
    n = int(np.ceil(vals.size / 127))
    rows = np.zeros((n, 128), np.float32)
    flat = np.zeros(n * 127, np.float32)
    flat[:vals.size] = vals
    rows[:, :127] = flat.reshape(n, 127)
    rows[:, 127] = 448.0
    # bf16 activations cannot hold these values exactly, so run the weight
    # quantiser path on an fp32-exact subset: values representable in bf16
    bf = (rows.view(np.uint32) & 0xFFFF0000).view(np.float32)
    exact = bf == rows
    xb = torch.from_numpy(bf).to(torch.bfloat16)
    pad = torch.zeros((128 * ((n + 127) // 128), 128), dtype=torch.bfloat16)
    pad[:n] = xb
    q, s = __import__("sparse_moe_layer_bias_amd.layer", fromlist=["x"]).quantize_weights_fp8(
        pad.cuda())
    torch.cuda.synchronize()
    rq, rs = orc.quant_weight_fp8(moe_inputs.to_host(pad))
    assert_bits(moe_inputs.to_host(q), rq, "codes at midpoints")
    assert exact.sum() > 100


def test_e4m3_encoder_fp32_midpoint_neighbours(orc):
    """The quantisation step as the kernels apply it (moe_inspect_e4m3: the FP8
    gate/up epilogue's quotient + four-value conversion, and the activation /
    weight quantisers' one-value conversion) on fp32 values the bf16 paths
    cannot carry: every E4M3 midpoint, its fp32 neighbours one ulp either
    side, the codes themselves, signed zeros, values past +-448 and below the
    smallest subnormal.  Each 1x128 row's scale comes from the oracle's own
    quantiser of that row; with an amax of 448 the scale is 1 and the codes are
    the converter's own.  Rows scaled by 0.37 and 3e-5 exercise the divide."""
    table = orc.e4m3_decode(np.arange(128, dtype=np.uint8)).astype(np.float64)
    pos = np.sort(table[np.isfinite(table)])
    vals = []
    for a, b in zip(pos[:-1], pos[1:]):
        m = np.float32((a + b) / 2)
        vals += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(1e9)),
                 np.float32(a), np.nextafter(np.float32(a), np.float32(1e9))]
    vals += [0.0, 2.0 ** -11, 2.0 ** -10, 3 * 2.0 ** -11, 448.0]
    vals = np.array(vals, np.float32)
    vals = np.concatenate([vals, -vals, np.array([-0.0], np.float32)])
    n = int(np.ceil(vals.size / 127))
    flat = np.zeros(n * 127, np.float32)
    flat[:vals.size] = vals
    base = np.zeros((n, 128), np.float32)
    base[:, :127] = np.clip(flat.reshape(n, 127), -448, 448)
    base[:, 127] = 448.0
    for f in (1.0, 0.37, 3e-5):
        rows = (base * np.float32(f)).astype(np.float32)
        q_ref, s_ref = orc.quant_act_fp8(rows)
        if f == 1.0:
            assert np.all(s_ref == 1.0)
        for r in range(n):
            v = torch.from_numpy(rows[r]).cuda()
            c4 = torch.empty(128, dtype=torch.uint8, device="cuda")
            c1 = torch.empty(128, dtype=torch.uint8, device="cuda")
            moe.moe_inspect_e4m3(v, float(s_ref[r, 0]), c4, c1)
            torch.cuda.synchronize()
            assert_bits(moe_inputs.to_host(c4), q_ref[r], "epilogue codes, row %d, x%g" % (r, f))
            assert_bits(moe_inputs.to_host(c1), q_ref[r], "quantiser codes, row %d, x%g" % (r, f))
    # quotients past +-448 are clamped (scale 1: the quotient is the value)
    big = np.array([448.0, np.nextafter(np.float32(448), 1e9), 449.0, 464.0, 480.0, 1e6, 3e38],
                   np.float32)
    big = np.concatenate([big, -big, np.zeros(2, np.float32)])
    v = torch.from_numpy(big).cuda()
    c4 = torch.empty(big.size, dtype=torch.uint8, device="cuda")
    c1 = torch.empty(big.size, dtype=torch.uint8, device="cuda")
    moe.moe_inspect_e4m3(v, 1.0, c4, c1)
    torch.cuda.synchronize()
    ref = orc.e4m3_encode(np.clip(big, -448, 448))
    assert_bits(moe_inputs.to_host(c4), ref, "clamped (epilogue)")
    assert_bits(moe_inputs.to_host(c1), ref, "clamped (quantiser)")
    # an all-zero tile: scale 0, codes 0
    z = torch.zeros(128, device="cuda")
    c4 = torch.full((128,), 7, dtype=torch.uint8, device="cuda")
    c1 = torch.full((128,), 7, dtype=torch.uint8, device="cuda")
    moe.moe_inspect_e4m3(z, 0.0, c4, c1)
    torch.cuda.synchronize()
    assert not moe_inputs.to_host(c4).any() and not moe_inputs.to_host(c1).any()


# ------------------------------------------------------------------ bias trajectory

def test_skew_balance_trajectory(orc):
    """Zipf-skewed router, 100 steps of route + end-of-step bias update: the
    bias after every step is bit-identical to the oracle's."""
    cfg = dict(moe_inputs.CONFIGS["skew_balance"])
    steps = cfg["steps"]
    E = moe_inputs.make_skew_centroids(cfg, 0, "cpu")
    Eh = moe_inputs.to_host(E)
    Ed = E.cuda()
    c = moe.cfg_from_dict(cfg)
    T, N, k = cfg["T"], cfg["N"], cfg["k"]
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, k), dtype=torch.float32, device="cuda")
    counts = torch.empty((N,), dtype=torch.int32, device="cuda")
    scores = torch.empty((T, N), dtype=torch.float32, device="cuda")
    bias = torch.zeros(N, device="cuda")
    bh = np.zeros(N, np.float32)
    imb = []
    for step in range(steps):
        x = moe_inputs.make_skew_tokens(cfg, step, 0, "cpu")
        moe.moe_route(c, x.cuda(), Ed, bias, scores, idx, gate, counts)
        moe.moe_bias_update(N, T * k, counts, 0.001, bias)
        torch.cuda.synchronize()
        r = orc.route(moe_inputs.to_host(x), Eh, bh, k)
        assert_bits(moe_inputs.to_host(idx), r["idx"], "idx step %d" % step)
        assert_bits(moe_inputs.to_host(counts), r["counts"], "counts step %d" % step)
        bh = orc.bias_update(r["counts"], T * k, bh)
        assert_bits(moe_inputs.to_host(bias).view(np.uint32), bh.view(np.uint32),
                    "bias step %d" % step)
        imb.append(r["counts"].max() / (T * k / N))
        if step % 20 == 0:
            log("step", step, "max/mean load %.2f" % imb[-1])
    assert np.mean(imb[-10:]) < np.mean(imb[:10])


def test_bias_state_resumes_exactly():
    """The bias is the layer's only state across steps: 30 steps in one go and
    15 + 15 steps with the bias saved to host memory and restored into a
    fresh buffer in between end with the same bias bits."""
    cfg = dict(moe_inputs.CONFIGS["skew_balance"])
    E = moe_inputs.make_skew_centroids(cfg, 0, "cpu").cuda()
    c = moe.cfg_from_dict(cfg)
    T, N, k = cfg["T"], cfg["N"], cfg["k"]
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, k), dtype=torch.float32, device="cuda")
    counts = torch.empty((N,), dtype=torch.int32, device="cuda")
    scores = torch.empty((T, N), dtype=torch.float32, device="cuda")

    def run(bias, steps):
        for step in steps:
            x = moe_inputs.make_skew_tokens(cfg, step, 0, "cpu").cuda()
            moe.moe_route(c, x, E, bias, scores, idx, gate, counts)
            moe.moe_bias_update(N, T * k, counts, 0.001, bias)
        torch.cuda.synchronize()
        return bias

    straight = run(torch.zeros(N, device="cuda"), range(30))
    saved = moe_inputs.to_host(run(torch.zeros(N, device="cuda"), range(15))).copy()
    resumed = run(torch.from_numpy(saved).cuda(), range(15, 30))
    assert_bits(moe_inputs.to_host(resumed).view(np.uint32),
                moe_inputs.to_host(straight).view(np.uint32), "bias after resume")
    assert np.any(moe_inputs.to_host(straight) != 0)


# ------------------------------------------------------------------ V3 shape, sampled

@pytest.fixture(scope="module")
def v3_run():
    cfg = dict(moe_inputs.CONFIGS["v3_bf16"])
    log("generating V3-shaped inputs on the GPU")
    dev = moe_inputs.make_layer_inputs(cfg, 0, "cuda")
    layer = MoeLayer(cfg, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"])
    bias0 = dev["bias"].clone()
    bias = dev["bias"].clone()
    layer.forward(dev["x"], dev["centroids"], bias)
    torch.cuda.synchronize()
    log("V3 forward done")
    return cfg, dev, layer, bias0, bias


@pytest.fixture(scope="module")
def v3_fp8_run():
    cfg = dict(moe_inputs.CONFIGS["v3_fp8"])
    log("generating V3-shaped inputs on the GPU (FP8 layer)")
    dev = moe_inputs.make_layer_inputs(cfg, 0, "cuda")
    layer = MoeLayer(cfg, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"], gather_rows=False)
    bias0 = dev["bias"].clone()
    bias = dev["bias"].clone()
    layer.forward(dev["x"], dev["centroids"], bias)
    torch.cuda.synchronize()
    log("V3 FP8 forward done")
    yield cfg, dev, layer, bias0, bias
    del layer, dev
    torch.cuda.empty_cache()


def _v3_tokens(cfg, idx, seed, n=64):
    """n tokens at random plus the first and last, covering all expert groups"""
    rng = np.random.default_rng(seed)
    tok = np.unique(np.concatenate([rng.choice(cfg["T"], n, replace=False), [0, cfg["T"] - 1]]))
    gs = cfg["N"] // cfg["G"]
    assert len(np.unique(idx[tok] // gs)) == cfg["G"], "sample misses a group"
    return tok


def _check_v3_routing(orc, cfg, dev, layer, bias0, with_scores):
    """scores (when kept), idx, gates and counts of the whole batch against the
    oracle, bit for bit; then offsets, src_token and dst_row against the
    oracle's permutation of the oracle's indices."""
    xh = moe_inputs.to_host(dev["x"])
    r = orc.route(xh, moe_inputs.to_host(dev["centroids"]), moe_inputs.to_host(bias0),
                  cfg["k"], cfg["G"], cfg["TG"], want_scores=with_scores)
    log("oracle routed the whole batch")
    if with_scores:
        assert_bits(moe_inputs.to_host(layer.scores), r["scores"], "scores (all tokens)")
    assert_bits(moe_inputs.to_host(layer.idx), r["idx"], "idx (all tokens)")
    assert_bits(moe_inputs.to_host(layer.gate), r["gate"], "gate (all tokens)")
    assert_bits(moe_inputs.to_host(layer.counts), r["counts"], "counts")
    off, src, dst = orc.permute(r["idx"], cfg["N"])
    assert_bits(moe_inputs.to_host(layer.offsets), off, "offsets")
    assert_bits(moe_inputs.to_host(layer.src_token), src, "src_token")
    assert_bits(moe_inputs.to_host(layer.dst_row), dst, "dst_row")
    r.update(offsets=off, src_token=src, dst_row=dst)
    return xh, r


@pytest.mark.timeout(900)
def test_v3_fp8_layer_parity(orc, v3_fp8_run):
    """The V3-shaped FP8 layer: routing of all 8192 tokens and the activation
    codes and scales of every token bit for bit; the expert FFN step by step
    (fp32 h, h bytes, y, out) on the routed rows of 64+ tokens that cover all
    8 groups, and every shared-expert row of those tokens."""
    cfg, dev, layer, bias0, bias = v3_fp8_run
    xh, r = _check_v3_routing(orc, cfg, dev, layer, bias0, with_scores=False)
    xq, xs = orc.quant_act_fp8(xh)
    assert_bits(moe_inputs.to_host(layer.x_q), xq, "x codes (all tokens)")
    assert_bits(moe_inputs.to_host(layer.x_s).view(np.uint32), xs.view(np.uint32),
                "x scales (all tokens)")
    src = r["src_token"]
    rows = np.random.default_rng(4).choice(cfg["T"] * cfg["k"], 4096, replace=False)
    rt = torch.from_numpy(rows).cuda()
    assert_bits(moe_inputs.to_host(layer.x_perm[rt]), xq[src[rows]], "permuted codes (rows)")
    assert_bits(moe_inputs.to_host(layer.x_perm_s[rt]).view(np.uint32),
                xs[src[rows]].view(np.uint32), "permuted scales (rows)")
    tok = _v3_tokens(cfg, r["idx"], 3)
    rows = np.sort(r["dst_row"][tok].ravel())
    ref = dict(r, x_q=xq, x_s=xs,
               w13_q=ExpertCodes(orc, dev["w13"], 0), w13_s=ExpertCodes(orc, dev["w13"], 1),
               w2_q=ExpertCodes(orc, dev["w2"], 0), w2_s=ExpertCodes(orc, dev["w2"], 1))
    ref["x_q_perm"] = RowsOf(xq, src)
    ref["x_s_perm"] = RowsOf(xs, src)
    ref["ws13_q"], ref["ws13_s"] = orc.quant_weight_fp8(moe_inputs.to_host(dev["ws13"]))
    ref["ws2_q"], ref["ws2_s"] = orc.quant_weight_fp8(moe_inputs.to_host(dev["ws2"]))
    log("checking the expert FFN on %d routed rows of %d tokens" % (len(rows), len(tok)))
    check_fp8_expert_split(orc, layer, ref, xh, rows=rows, what="V3 FP8: ")
    new_b = orc.bias_update(r["counts"], cfg["T"] * cfg["k"], moe_inputs.to_host(bias0))
    assert_bits(moe_inputs.to_host(bias).view(np.uint32), new_b.view(np.uint32), "bias update")


def _full_permute(cfg, x, layer):
    """moe_permute with the permuted copy, on the layer's routing"""
    T, k, d, N = cfg["T"], cfg["k"], cfg["d"], cfg["N"]
    i32 = dict(dtype=torch.int32, device="cuda")
    offs = torch.empty((N + 1,), **i32)
    src = torch.empty((T * k,), **i32)
    dst = torch.empty((T, k), **i32)
    x_perm = torch.empty((T * k, d), dtype=torch.bfloat16, device="cuda")
    moe.moe_permute(layer.cfg, x, layer.idx, offs, src, dst, x_perm, None, None, None,
                    layer.workspace)
    return offs, src, dst, x_perm


def test_v3_gathered_rows_equal_permuted_rows(orc, v3_run):
    """At the V3 shape the expert FFN on the gathered rows (the layer's path)
    equals moe_expert_ffn on the permuted copy, bit for bit."""
    cfg, dev, layer, bias0, bias = v3_run
    assert layer.gather_rows
    offs, src, dst, x_perm = _full_permute(cfg, dev["x"], layer)
    y = torch.empty_like(layer.y_perm)
    ys = torch.empty_like(layer.y_shared)
    moe.moe_expert_ffn(layer.cfg, x_perm, None, offs, layer.w13, None, layer.w2, None, y,
                       dev["x"], None, layer.ws13, None, layer.ws2, None, ys, layer.workspace)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), layer.y_perm.view(torch.int16)), "y_perm"
    assert torch.equal(ys.view(torch.int16), layer.y_shared.view(torch.int16)), "y_shared"


def test_v3_fp8_gathered_rows_equal_permuted_rows(orc, v3_fp8_run):
    """The V3-shaped FP8 expert FFN on rows gathered from x_q, x_s through
    src_token (the inference layer's path) equals the one on the permuted
    codes, bit for bit."""
    cfg, dev, layer, bias0, bias = v3_fp8_run
    _check_gathered_rows(layer)


def test_v3_routing_all_tokens(orc, v3_run):
    cfg, dev, layer, bias0, bias = v3_run
    _check_v3_routing(orc, cfg, dev, layer, bias0, with_scores=True)


def test_v3_permutation_properties(orc, v3_run):
    cfg, dev, layer, bias0, bias = v3_run
    N, T, k = cfg["N"], cfg["T"], cfg["k"]
    idx = moe_inputs.to_host(layer.idx)
    counts = moe_inputs.to_host(layer.counts)
    assert counts.sum() == T * k
    for row in idx[:: 97]:
        assert len(set(row)) == k
    # group limit: each token's experts lie in at most TG groups
    gs = N // cfg["G"]
    assert max(len(set(row // gs)) for row in idx) <= cfg["TG"]
    src = moe_inputs.to_host(layer.src_token)
    # the layer's permutation wrote indices only (its GEMM gathers the rows):
    # the full permutation gives the same indices and the rows they name
    offs, srcf, dstf, x_perm = _full_permute(cfg, dev["x"], layer)
    assert_bits(moe_inputs.to_host(offs), moe_inputs.to_host(layer.offsets), "offsets")
    assert_bits(moe_inputs.to_host(srcf), src, "src_token")
    assert_bits(moe_inputs.to_host(dstf), moe_inputs.to_host(layer.dst_row), "dst_row")
    rows = np.random.default_rng(1).choice(T * k, 4000, replace=False)
    xp = moe_inputs.to_host(x_perm[torch.from_numpy(rows).cuda()])
    xs = moe_inputs.to_host(dev["x"][torch.from_numpy(src[rows]).long().cuda()])
    assert_bits(xp, xs, "x_perm rows")
    new_b = orc.bias_update(counts, T * k, moe_inputs.to_host(bias0))
    assert_bits(moe_inputs.to_host(bias).view(np.uint32), new_b.view(np.uint32), "bias update")


@pytest.mark.timeout(900)
def test_v3_layer_output_sampled_tokens(orc, v3_run):
    """Expert outputs and the layer output of 64+ tokens that cover all 8
    groups (every routed row of those tokens, one expert at a time)."""
    cfg, dev, layer, bias0, bias = v3_run
    xh_all = moe_inputs.to_host(dev["x"])
    r = orc.route(xh_all, moe_inputs.to_host(dev["centroids"]), moe_inputs.to_host(bias0),
                  cfg["k"], cfg["G"], cfg["TG"])
    assert_bits(moe_inputs.to_host(layer.idx), r["idx"], "idx (all tokens)")
    tok = _v3_tokens(cfg, r["idx"], 2)
    tt = torch.from_numpy(tok).cuda()
    xh = xh_all[tok]
    ws13 = moe_inputs.to_host(dev["ws13"])
    ws2 = moe_inputs.to_host(dev["ws2"])
    ys = orc.swiglu_ffn(xh, ws13, ws2)
    assert_close(moe_inputs.to_host(layer.y_shared[tt]), ys, RTOL["bf16"], "y_shared (sampled)")
    # routed expert outputs for the sampled tokens, one expert at a time
    idx = r["idx"][tok]
    yp_ref = np.zeros((len(tok), cfg["k"], cfg["d"]), np.uint16)
    experts = np.unique(idx)
    log("oracle: %d experts for %d tokens" % (len(experts), len(tok)))
    for n, e in enumerate(experts):
        sel = np.argwhere(idx == e)
        y = orc.swiglu_ffn(xh[sel[:, 0]], moe_inputs.to_host(dev["w13"][int(e)]),
                           moe_inputs.to_host(dev["w2"][int(e)]))
        yp_ref[sel[:, 0], sel[:, 1]] = y
        if n % 32 == 0:
            log("  expert %d of %d" % (n, len(experts)))
    dst = moe_inputs.to_host(layer.dst_row)[tok]
    yp_gpu = moe_inputs.to_host(layer.y_perm[torch.from_numpy(dst.ravel()).long().cuda()])
    assert_close(yp_gpu.reshape(yp_ref.shape), yp_ref, RTOL["bf16"], "y_perm (sampled)")
    # combine from the oracle's own expert outputs
    k = cfg["k"]
    fake_dst = np.arange(len(tok) * k, dtype=np.int32).reshape(len(tok), k)
    out_ref = orc.combine(xh, ys, yp_ref.reshape(-1, cfg["d"]), r["gate"][tok], fake_dst, "bf16")
    assert_close(moe_inputs.to_host(layer.out[tt]), out_ref, RTOL["bf16"], "out (sampled)")


@pytest.mark.timeout(900)
def test_decode_batch_layer_v3_weights(orc, v3_run):
    """The skewed decode-step workload as a whole layer: T = 128 tokens of the
    Zipf-skewed router (no group limit) over the V3-shaped experts, with the
    bias the oracle's own 100 balancing steps reach, so that most experts get
    1-10 rows (a few rows per 320-row tile).  idx, gates and counts of all
    tokens bit for bit; routed and shared expert outputs and the layer output
    of 24 tokens (every routed row of each) within the bf16 tolerance."""
    cfg5 = dict(moe_inputs.CONFIGS["skew_balance"])
    _, dev, _, _, _ = v3_run
    T, N, k = cfg5["T"], cfg5["N"], cfg5["k"]
    E = moe_inputs.make_skew_centroids(cfg5, 0, "cpu")
    Eh = moe_inputs.to_host(E)
    bh = np.zeros(N, np.float32)
    for step in range(cfg5["steps"]):
        r = orc.route(moe_inputs.to_host(moe_inputs.make_skew_tokens(cfg5, step, 0, "cpu")), Eh,
                      bh, k)
        bh = orc.bias_update(r["counts"], T * k, bh)
    x = moe_inputs.make_skew_tokens(cfg5, cfg5["steps"], 0, "cpu")
    xh = moe_inputs.to_host(x)
    xd = x.cuda()
    layer = MoeLayer(cfg5, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"])
    bias = torch.from_numpy(bh.copy()).cuda()
    out = layer.forward(xd, E.cuda(), bias)
    torch.cuda.synchronize()
    r = orc.route(xh, Eh, bh, k)
    assert_bits(moe_inputs.to_host(layer.idx), r["idx"], "idx")
    assert_bits(moe_inputs.to_host(layer.gate), r["gate"], "gate")
    assert_bits(moe_inputs.to_host(layer.counts), r["counts"], "counts")
    touched = int((r["counts"] > 0).sum())
    log("decode batch: %d of %d experts touched, max rows %d" % (touched, N, r["counts"].max()))
    assert touched > N // 2
    off, src, dst = orc.permute(r["idx"], N)
    assert_bits(moe_inputs.to_host(layer.dst_row), dst, "dst_row")
    tok = np.sort(np.random.default_rng(7).choice(T, 24, replace=False))
    tt = torch.from_numpy(tok).cuda()
    ys = orc.swiglu_ffn(xh[tok], moe_inputs.to_host(dev["ws13"]), moe_inputs.to_host(dev["ws2"]))
    assert_close(moe_inputs.to_host(layer.y_shared[tt]), ys, RTOL["bf16"], "y_shared")
    idx = r["idx"][tok]
    yp_ref = np.zeros((len(tok), k, cfg5["d"]), np.uint16)
    for e in np.unique(idx):
        sel = np.argwhere(idx == e)
        yp_ref[sel[:, 0], sel[:, 1]] = orc.swiglu_ffn(
            xh[tok][sel[:, 0]], moe_inputs.to_host(dev["w13"][int(e)]),
            moe_inputs.to_host(dev["w2"][int(e)]))
    yp_gpu = moe_inputs.to_host(layer.y_perm[torch.from_numpy(dst[tok].ravel()).long().cuda()])
    assert_close(yp_gpu.reshape(yp_ref.shape), yp_ref, RTOL["bf16"], "y_perm")
    fake = np.arange(len(tok) * k, dtype=np.int32).reshape(len(tok), k)
    out_ref = orc.combine(xh[tok], ys, yp_ref.reshape(-1, cfg5["d"]), r["gate"][tok], fake,
                          "bf16")
    assert_close(moe_inputs.to_host(out[tt]), out_ref, RTOL["bf16"], "out")
    assert_bits(moe_inputs.to_host(bias).view(np.uint32),
                orc.bias_update(r["counts"], T * k, bh).view(np.uint32), "bias update")
    del layer
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_decode_batch_layer_v3_fp8(orc, v3_fp8_run):
    """The skewed decode-step batch (T = 128, no group limit, the bias of the
    oracle's own 100 balancing steps) through the FP8 layer with the V3-shaped
    weights: 1-10 rows in most 320-row FP8 tiles.  idx, gates and counts of all
    tokens and the activation codes and scales bit for bit; the expert FFN step
    by step (fp32 h, h bytes, y, out) on every routed row of 24 tokens and
    their shared-expert rows."""
    cfg5 = dict(moe_inputs.CONFIGS["skew_balance"], fp8=True)
    _, dev, _, _, _ = v3_fp8_run
    T, N, k = cfg5["T"], cfg5["N"], cfg5["k"]
    E = moe_inputs.make_skew_centroids(cfg5, 0, "cpu")
    Eh = moe_inputs.to_host(E)
    bh = np.zeros(N, np.float32)
    for step in range(cfg5["steps"]):
        r = orc.route(moe_inputs.to_host(moe_inputs.make_skew_tokens(cfg5, step, 0, "cpu")), Eh,
                      bh, k)
        bh = orc.bias_update(r["counts"], T * k, bh)
    x = moe_inputs.make_skew_tokens(cfg5, cfg5["steps"], 0, "cpu")
    xh = moe_inputs.to_host(x)
    layer = MoeLayer(cfg5, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"], gather_rows=False)
    bias = torch.from_numpy(bh.copy()).cuda()
    layer.forward(x.cuda(), E.cuda(), bias)
    torch.cuda.synchronize()
    r = orc.route(xh, Eh, bh, k)
    assert_bits(moe_inputs.to_host(layer.idx), r["idx"], "idx")
    assert_bits(moe_inputs.to_host(layer.gate), r["gate"], "gate")
    assert_bits(moe_inputs.to_host(layer.counts), r["counts"], "counts")
    touched = int((r["counts"] > 0).sum())
    log("FP8 decode batch: %d of %d experts touched, max rows %d" % (touched, N,
                                                                      r["counts"].max()))
    assert touched > N // 2
    off, src, dst = orc.permute(r["idx"], N)
    assert_bits(moe_inputs.to_host(layer.offsets), off, "offsets")
    assert_bits(moe_inputs.to_host(layer.dst_row), dst, "dst_row")
    xq, xs = orc.quant_act_fp8(xh)
    assert_bits(moe_inputs.to_host(layer.x_q), xq, "x codes")
    assert_bits(moe_inputs.to_host(layer.x_s).view(np.uint32), xs.view(np.uint32), "x scales")
    tok = np.sort(np.random.default_rng(9).choice(T, 24, replace=False))
    rows = np.sort(dst[tok].ravel())
    ref = dict(r, offsets=off, src_token=src, dst_row=dst, x_q=xq, x_s=xs,
               w13_q=ExpertCodes(orc, dev["w13"], 0), w13_s=ExpertCodes(orc, dev["w13"], 1),
               w2_q=ExpertCodes(orc, dev["w2"], 0), w2_s=ExpertCodes(orc, dev["w2"], 1))
    ref["x_q_perm"] = RowsOf(xq, src)
    ref["x_s_perm"] = RowsOf(xs, src)
    ref["ws13_q"], ref["ws13_s"] = orc.quant_weight_fp8(moe_inputs.to_host(dev["ws13"]))
    ref["ws2_q"], ref["ws2_s"] = orc.quant_weight_fp8(moe_inputs.to_host(dev["ws2"]))
    log("checking the FP8 expert FFN on %d routed rows of %d tokens" % (len(rows), len(tok)))
    check_fp8_expert_split(orc, layer, ref, xh, rows=rows, what="FP8 decode: ")
    assert_bits(moe_inputs.to_host(bias).view(np.uint32),
                orc.bias_update(r["counts"], T * k, bh).view(np.uint32), "bias update")
    del layer
    torch.cuda.empty_cache()
