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
from parity_util import (RTOL, assert_bits, assert_close, assert_close_fp8, host_inputs, log,
                         small_layer_inputs)
from sparse_moe_layer_bias_amd.layer import MoeLayer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the parity tests need the HIP library on an MI355X")
    moe.lib()
    yield
    torch.cuda.synchronize()


def _run_small(cfg_name, orc, T=None, residual=True, seed=0, **over):
    cfg = dict(moe_inputs.CONFIGS[cfg_name])
    cfg.update(over)
    c, inp, dev = small_layer_inputs(cfg, seed, T)
    log("case", cfg_name, "T=%d" % c["T"], over, "seed", seed)
    layer = MoeLayer(c, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"])
    bias = dev["bias"].clone()
    out = layer.forward(dev["x"], dev["centroids"], bias, residual=residual)
    torch.cuda.synchronize()
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
    assert_bits(moe_inputs.to_host(layer.x_perm), ref["x_perm"], "x_perm")
    assert_close(moe_inputs.to_host(layer.y_perm), ref["y_perm"], rtol, "y_perm")
    assert_close(moe_inputs.to_host(layer.y_shared), ref["y_shared"], rtol, "y_shared")
    assert_close(moe_inputs.to_host(out), ref["out"], rtol, "out")
    assert_bits(moe_inputs.to_host(bias), ref["new_bias"], "bias after update")


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
]


@pytest.mark.parametrize("name,over", FP8_CASES)
def test_layer_parity_fp8_small(orc, name, over):
    """FP8 E4M3 expert GEMMs (1x128 activation tiles, 128x128 weight blocks,
    fp32 promotion per 128-K block) against the oracle's FP8 path."""
    over = dict(over)
    T = over.pop("T", None)
    c, layer, out, bias, ref = _run_small(name, orc, T=T, fp8=True, **over)
    rtol = RTOL["fp8"]
    assert_bits(moe_inputs.to_host(layer.idx), ref["idx"], "idx")
    assert_bits(moe_inputs.to_host(layer.x_q), ref["x_q"], "x codes")
    assert_bits(moe_inputs.to_host(layer.x_s).view(np.uint32), ref["x_s"].view(np.uint32),
                "x scales")
    assert_bits(moe_inputs.to_host(layer.x_perm), ref["x_q_perm"], "permuted codes")
    assert_close_fp8(moe_inputs.to_host(layer.y_perm), ref["y_perm"], "y_perm")
    assert_close_fp8(moe_inputs.to_host(layer.y_shared), ref["y_shared"], "y_shared")
    assert_close_fp8(moe_inputs.to_host(out), ref["out"], "out")
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
    layer = MoeLayer(c, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"])
    out = layer.forward(dev["x"], dev["centroids"], dev["bias"].clone())
    torch.cuda.synchronize()
    ref = orc.layer_forward(host_inputs(inp), c, residual=True)
    assert np.all(np.isfinite(ref["y_perm"].astype(np.float64))), "oracle overflowed"
    assert_bits(moe_inputs.to_host(layer.idx), ref["idx"], "idx")
    assert_bits(moe_inputs.to_host(layer.x_perm), ref["x_q_perm"], "permuted codes")
    assert_close_fp8(moe_inputs.to_host(layer.y_perm), ref["y_perm"], "y_perm")
    assert_close_fp8(moe_inputs.to_host(layer.y_shared), ref["y_shared"], "y_shared")
    assert_close_fp8(moe_inputs.to_host(out), ref["out"], "out")


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
    layer = MoeLayer(c, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"])
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
    layer = MoeLayer(cfg, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"])
    bias0 = dev["bias"].clone()
    bias = dev["bias"].clone()
    layer.forward(dev["x"], dev["centroids"], bias)
    torch.cuda.synchronize()
    log("V3 FP8 forward done")
    yield cfg, dev, layer, bias0, bias
    del layer, dev
    torch.cuda.empty_cache()


def test_v3_fp8_layer_output_sampled_tokens(orc, v3_fp8_run):
    cfg, dev, layer, bias0, bias = v3_fp8_run
    rng = np.random.default_rng(3)
    tok = np.unique(np.concatenate([rng.choice(cfg["T"], 6, replace=False), [cfg["T"] - 1]]))
    ti = torch.from_numpy(tok).cuda()
    xh = moe_inputs.to_host(dev["x"][ti])
    r = orc.route(xh, moe_inputs.to_host(dev["centroids"]), moe_inputs.to_host(bias0),
                  cfg["k"], cfg["G"], cfg["TG"])
    assert_bits(moe_inputs.to_host(layer.idx)[tok], r["idx"], "idx (sampled)")
    xq, xs = orc.quant_act_fp8(xh)
    assert_bits(moe_inputs.to_host(layer.x_q[ti]), xq, "x codes (sampled)")
    q13, s13 = orc.quant_weight_fp8(moe_inputs.to_host(dev["ws13"]))
    q2, s2 = orc.quant_weight_fp8(moe_inputs.to_host(dev["ws2"]))
    ys = orc.swiglu_ffn_fp8(xq, xs, q13, s13, q2, s2)
    assert_close_fp8(moe_inputs.to_host(layer.y_shared[ti]), ys, "y_shared (sampled)")
    yp_ref = np.zeros((len(tok), cfg["k"], cfg["d"]), np.uint16)
    for e in np.unique(r["idx"]):
        sel = np.argwhere(r["idx"] == e)
        q13, s13 = orc.quant_weight_fp8(moe_inputs.to_host(dev["w13"][int(e)]))
        q2, s2 = orc.quant_weight_fp8(moe_inputs.to_host(dev["w2"][int(e)]))
        yp_ref[sel[:, 0], sel[:, 1]] = orc.swiglu_ffn_fp8(xq[sel[:, 0]], xs[sel[:, 0]], q13, s13,
                                                          q2, s2)
    dst = moe_inputs.to_host(layer.dst_row)[tok]
    yp_gpu = moe_inputs.to_host(layer.y_perm[torch.from_numpy(dst.ravel()).long().cuda()])
    assert_close_fp8(yp_gpu.reshape(-1, cfg["d"]), yp_ref.reshape(-1, cfg["d"]),
                     "y_perm (sampled)")
    k = cfg["k"]
    fake_dst = np.arange(len(tok) * k, dtype=np.int32).reshape(len(tok), k)
    out_ref = orc.combine(xh, ys, yp_ref.reshape(-1, cfg["d"]), r["gate"], fake_dst, "bf16")
    assert_close_fp8(moe_inputs.to_host(layer.out[ti]), out_ref, "out (sampled)")


def test_v3_routing_sampled_tokens(orc, v3_run):
    cfg, dev, layer, bias0, bias = v3_run
    rng = np.random.default_rng(0)
    tok = np.sort(rng.choice(cfg["T"], 384, replace=False))
    tok = np.unique(np.concatenate([tok, [0, cfg["T"] - 1]]))
    xh = moe_inputs.to_host(dev["x"][torch.from_numpy(tok).cuda()])
    r = orc.route(xh, moe_inputs.to_host(dev["centroids"]), moe_inputs.to_host(bias0),
                  cfg["k"], cfg["G"], cfg["TG"], want_scores=True)
    assert_bits(moe_inputs.to_host(layer.scores)[tok], r["scores"], "scores (sampled)")
    assert_bits(moe_inputs.to_host(layer.idx)[tok], r["idx"], "idx (sampled)")
    assert_bits(moe_inputs.to_host(layer.gate)[tok], r["gate"], "gate (sampled)")


def test_v3_permutation_properties(orc, v3_run):
    cfg, dev, layer, bias0, bias = v3_run
    N, T, k = cfg["N"], cfg["T"], cfg["k"]
    idx = moe_inputs.to_host(layer.idx)
    counts = moe_inputs.to_host(layer.counts)
    assert counts.sum() == T * k
    assert_bits(counts, np.bincount(idx.ravel(), minlength=N).astype(np.int32), "counts")
    for row in idx[:: 97]:
        assert len(set(row)) == k
    # group limit: each token's experts lie in at most TG groups
    gs = N // cfg["G"]
    assert max(len(set(row // gs)) for row in idx) <= cfg["TG"]
    off, src, dst = orc.permute(idx, N)
    assert_bits(moe_inputs.to_host(layer.offsets), off, "offsets")
    assert_bits(moe_inputs.to_host(layer.src_token), src, "src_token")
    assert_bits(moe_inputs.to_host(layer.dst_row), dst, "dst_row")
    rows = np.random.default_rng(1).choice(T * k, 2000, replace=False)
    xp = moe_inputs.to_host(layer.x_perm[torch.from_numpy(rows).cuda()])
    xs = moe_inputs.to_host(dev["x"][torch.from_numpy(src[rows]).long().cuda()])
    assert_bits(xp, xs, "x_perm rows")
    new_b = orc.bias_update(counts, T * k, moe_inputs.to_host(bias0))
    assert_bits(moe_inputs.to_host(bias).view(np.uint32), new_b.view(np.uint32), "bias update")


def test_v3_layer_output_sampled_tokens(orc, v3_run):
    cfg, dev, layer, bias0, bias = v3_run
    rng = np.random.default_rng(2)
    tok = np.unique(np.concatenate([rng.choice(cfg["T"], 10, replace=False),
                                    [0, cfg["T"] - 1]]))
    h = {"x": moe_inputs.to_host(dev["x"][torch.from_numpy(tok).cuda()])}
    r = orc.route(h["x"], moe_inputs.to_host(dev["centroids"]), moe_inputs.to_host(bias0),
                  cfg["k"], cfg["G"], cfg["TG"])
    ws13 = moe_inputs.to_host(dev["ws13"])
    ws2 = moe_inputs.to_host(dev["ws2"])
    ys = orc.swiglu_ffn(h["x"], ws13, ws2)
    assert_close(moe_inputs.to_host(layer.y_shared[torch.from_numpy(tok).cuda()]), ys,
                 RTOL["bf16"], "y_shared (sampled)")
    # routed expert outputs for the sampled tokens, one expert at a time
    yp_ref = np.zeros((len(tok), cfg["k"], cfg["d"]), np.uint16)
    for e in np.unique(r["idx"]):
        sel = np.argwhere(r["idx"] == e)
        rows = h["x"][sel[:, 0]]
        y = orc.swiglu_ffn(rows, moe_inputs.to_host(dev["w13"][int(e)]),
                           moe_inputs.to_host(dev["w2"][int(e)]))
        yp_ref[sel[:, 0], sel[:, 1]] = y
    dst = moe_inputs.to_host(layer.dst_row)[tok]
    yp_gpu = moe_inputs.to_host(layer.y_perm[torch.from_numpy(dst.ravel()).long().cuda()])
    assert_close(yp_gpu.reshape(yp_ref.shape), yp_ref, RTOL["bf16"], "y_perm (sampled)")
    # combine from the oracle's own expert outputs
    k = cfg["k"]
    fake_dst = np.arange(len(tok) * k, dtype=np.int32).reshape(len(tok), k)
    out_ref = orc.combine(h["x"], ys, yp_ref.reshape(-1, cfg["d"]), r["gate"], fake_dst, "bf16")
    assert_close(moe_inputs.to_host(layer.out[torch.from_numpy(tok).cuda()]), out_ref,
                 RTOL["bf16"], "out (sampled)")
