"""Helpers shared by the GPU parity tests: input preparation on both sides and
the tolerance rule.

Tolerance (floating outputs): |gpu - ref| <= rtol * (|ref| + rms(ref row)),
elementwise, with rtol 1e-5 (fp32), 2e-2 (bf16), 6e-2 (FP8 GEMMs).
Integer, index and byte outputs are compared bit for bit.

Gradients of fp32 layers use the same rtol against the RMS of the whole
tensor instead of the row: |gpu - ref| <= rtol * (|ref| + rms(ref)).  Their
entries are differences and cancelling sums (silu' vanishes near a = -1.28,
dL/dz = (dg_j - sum_i dg_i g_i) s (1-s) / S, dot products with small
results); fp32 evaluation of such a quantity errs by about eps times the size
of its terms, which is the tensor's typical magnitude, not by eps times the
result.  With one token the weight gradient rows are single products
da[n] * x, so a row is one such quantity and the row RMS gives no scale.
"""
import sys

import numpy as np
import torch

import moe_inputs
from moe_inputs import to_host

RTOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2}


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def assert_close(got, ref, rtol, what=""):
    g, r = to_f64(got), to_f64(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    if r.size == 0:
        return
    r2 = r.reshape(-1, r.shape[-1]) if r.ndim > 1 else r.reshape(1, -1)
    g2 = g.reshape(r2.shape)
    rms = np.sqrt(np.mean(r2 ** 2, axis=1, keepdims=True))
    bound = rtol * (np.abs(r2) + rms)
    err = np.abs(g2 - r2)
    bad = ~(err <= bound)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("%s: %d/%d elements out of tolerance %g; first at %s: gpu=%r ref=%r"
                             " (max rel err %.3g)" % (what, bad.sum(), bad.size, rtol, tuple(i),
                                                      g2[tuple(i)], r2[tuple(i)],
                                                      float(np.nanmax(err / (np.abs(r2) + rms)))))


def assert_close_tensor(got, ref, rtol, what=""):
    g, r = to_f64(got), to_f64(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    if r.size == 0:
        return
    rms = float(np.sqrt(np.mean(r ** 2)))
    err = np.abs(g - r)
    bad = ~(err <= rtol * (np.abs(r) + rms))
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("%s: %d/%d elements out of tolerance %g (tensor rms %.3g); first at "
                             "%s: gpu=%r ref=%r" % (what, bad.sum(), bad.size, rtol, rms, tuple(i),
                                                    g[tuple(i)], r[tuple(i)]))


def assert_close_fp8(got, ref, what="", rtol=RTOL["fp8"]):
    """FP8 outputs: the plain elementwise rule at rtol = 6e-2."""
    assert_close(got, ref, rtol, what)


# GPU fp32 h = silu(a) * b before its 1x128 quantisation against the oracle's
# fp32 h from the same codes.  gfx950's FP8 MFMA sums each group of 8
# consecutive products keeping about 14 bits below the group's largest
# product, then adds the group into its fp32 accumulator with fp32 rounding
# (measured with exact-value cases: in 448^2 + 7 x 1.0 the seven ones vanish;
# 2^20 + eight group sums of 2^-6 stays 2^20).  Per group that is an error of
# up to ~2^-12 of its largest product; over K/8 groups of random-signed
# errors a and b move by ~2^-12 sqrt(K/8) of a typical group maximum, ~1e-4
# of the row's RMS at K = 7168 (measured worst 2.9e-4 over the test cases).
# The oracle sums exactly.  The bound leaves a factor 3.
H_RTOL = 1e-3


def max_rule_err(got, ref):
    """largest |gpu - ref| / (|ref| + rms(ref row)): the smallest rtol the
    elementwise rule would pass with"""
    g, r = to_f64(got), to_f64(ref)
    if r.size == 0:
        return 0.0
    r2 = r.reshape(-1, r.shape[-1])
    g2 = g.reshape(r2.shape)
    den = np.abs(r2) + np.sqrt(np.mean(r2 ** 2, axis=1, keepdims=True))
    err = np.abs(g2 - r2)
    return float(np.max(np.where(den > 0, err / np.where(den > 0, den, 1.0),
                                 np.where(err > 0, np.inf, 0.0))))


def row_rel_l2(got, ref):
    g, r = to_f64(got), to_f64(ref)
    r2 = r.reshape(-1, r.shape[-1])
    g2 = g.reshape(r2.shape)
    return np.linalg.norm(g2 - r2, axis=1) / np.maximum(np.linalg.norm(r2, axis=1), 1e-30)


def check_fp8_expert_split(orc, layer, ref, x_host, rows=None, residual=True, what=""):
    """The FP8 expert FFN checked step by step against the oracle, for the
    routed rows `rows` of x_perm (None: all) and every shared-expert row of
    the tokens those rows belong to (all tokens when rows is None).

    1. The gate/up epilogue's fp32 h (moe_expert_ffn_inspect) against the
       oracle's gate/up half on the same codes: within H_RTOL.
    2. h's E4M3 codes and tile scales, as the down GEMM read them, bit for bit
       against the oracle's 1x128 quantiser applied to that GPU h.
    3. y against the oracle's down half fed those codes: 6e-2, plain rule.
    4. The layer output against the oracle's combine of those y: 6e-2.
    5. Beside the contract: y against the fully independent oracle (its own
       h), row-wise relative L2 within 6e-2 (a code at a rounding midpoint of
       h may differ there, moving single elements by up to a code step).
    `ref` is orc.layer_forward's result (routing, permutation, x and weight
    codes bit-exact against the GPU's are asserted by the caller)."""
    c = layer.c
    T, k, d, N = c["T"], c["k"], c["d"], c["N"]
    y_before = to_host(layer.y_perm).copy()
    ys_before = to_host(layer.y_shared).copy() if layer.y_shared is not None else None
    ins = layer.expert_ffn_inspect()
    torch.cuda.synchronize()
    assert_bits(to_host(layer.y_perm), y_before, what + "y_perm: inspect call == moe_expert_ffn")
    if ys_before is not None:
        assert_bits(to_host(layer.y_shared), ys_before, what + "y_shared: inspect call")
    offsets = ref["offsets"]
    if rows is None:
        rows = np.arange(T * k)
    rows = np.asarray(rows, np.int64)
    rt = torch.from_numpy(rows).cuda()
    hf = to_host(ins["h_f32"][rt])
    hq = to_host(ins["h_q"][rt])
    hs = to_host(ins["h_s"][rt])
    # 2. bytes
    q_o, s_o = orc.quant_act_fp8(hf)
    assert_bits(hq, q_o, what + "h codes (routed)")
    assert_bits(hs.view(np.uint32), s_o.view(np.uint32), what + "h tile scales (routed)")
    # 3. and 1., expert by expert
    expert = np.searchsorted(offsets, rows, side="right") - 1
    h_ref = np.empty_like(hf)
    y_ref = np.empty((len(rows), d), np.uint16)
    for e in np.unique(expert):
        sel = np.nonzero(expert == e)[0]
        r = rows[sel]
        h_ref[sel] = orc.swiglu_gateup_fp8(ref["x_q_perm"][r], ref["x_s_perm"][r],
                                           ref["w13_q"][e], ref["w13_s"][e])
        y_ref[sel] = orc.ffn_down_fp8(hq[sel], hs[sel], ref["w2_q"][e], ref["w2_s"][e])
    y_gpu = y_before[rows]
    l2 = (row_rel_l2(y_gpu, ref["y_perm"][rows]) if ref.get("y_perm") is not None
          else np.zeros(1))
    log(what + "routed rows %d: h max err %.2e, y max err %.2e (row rule); y max row-L2 vs "
        "independent oracle %.2e" % (len(rows), max_rule_err(hf, h_ref), max_rule_err(y_gpu, y_ref),
                                     float(l2.max(initial=0.0))))
    assert_close_fp8(y_gpu, y_ref, what + "y_perm")
    assert np.all(l2 <= RTOL["fp8"]), (what + "y_perm vs independent oracle: row L2 %.3g" %
                                       float(l2.max()))
    assert_close(hf, h_ref, H_RTOL, what + "h fp32 (routed)")
    # the tokens of those rows: shared expert and layer output
    src = ref["src_token"]
    tok = np.unique(src[rows])
    ys_ref = None
    if layer.y_shared is not None:
        tt = torch.from_numpy(tok).cuda()
        hfs = to_host(ins["h_f32_shared"][tt])
        hqs = to_host(ins["h_q_shared"][tt])
        hss = to_host(ins["h_s_shared"][tt])
        q_o, s_o = orc.quant_act_fp8(hfs)
        assert_bits(hqs, q_o, what + "h codes (shared)")
        assert_bits(hss.view(np.uint32), s_o.view(np.uint32), what + "h tile scales (shared)")
        hs_ref = orc.swiglu_gateup_fp8(ref["x_q"][tok], ref["x_s"][tok], ref["ws13_q"],
                                       ref["ws13_s"])
        ys_ref = orc.ffn_down_fp8(hqs, hss, ref["ws2_q"], ref["ws2_s"])
        log(what + "shared rows %d: h max err %.2e, y max err %.2e (row rule)" %
            (len(tok), max_rule_err(hfs, hs_ref), max_rule_err(ys_before[tok], ys_ref)))
        assert_close_fp8(ys_before[tok], ys_ref, what + "y_shared")
        assert_close(hfs, hs_ref, H_RTOL, what + "h fp32 (shared)")
        if ref.get("y_shared") is not None:
            assert np.all(row_rel_l2(ys_before[tok], ref["y_shared"][tok]) <= RTOL["fp8"])
    # layer output of the tokens whose every routed row was checked
    pos = {int(r): i for i, r in enumerate(rows)}
    dst = ref["dst_row"][tok]
    full = np.array([all(int(q) in pos for q in row) for row in dst])
    if full.any():
        tk = tok[full]
        yk = np.stack([y_ref[[pos[int(q)] for q in row]] for row in dst[full]])
        fake = np.arange(len(tk) * k, dtype=np.int32).reshape(len(tk), k)
        out_ref = orc.combine(x_host[tk] if residual else None,
                              ys_ref[full] if ys_ref is not None else None,
                              yk.reshape(-1, d), ref["gate"][tk], fake, "bf16")
        assert_close_fp8(to_host(layer.out)[tk], out_ref, what + "out")
    return ins


def assert_bits(got, ref, what=""):
    g, r = np.asarray(got), np.asarray(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    if g.dtype != r.dtype:
        g = g.view(r.dtype) if g.itemsize == r.itemsize else g.astype(r.dtype)
    neq = g != r
    if neq.any():
        i = np.argwhere(neq)[0]
        raise AssertionError("%s: %d/%d mismatches; first at %s: gpu=%r ref=%r" %
                             (what, neq.sum(), neq.size, tuple(i), g[tuple(i)], r[tuple(i)]))


# ------------------------------------------------------------------ canaries

GUARD_BYTES = 4096      # keeps every guarded view 256-byte aligned
GUARD_PATTERN = 0xA5


class Guards:
    """Device buffers with guard bands: each buffer is a view into an
    allocation that holds GUARD_BYTES bytes of GUARD_PATTERN before and after
    it; check() asserts every band is still untouched, so a kernel that writes
    past either end of an output shows up even when the stray bytes land in
    memory no other check reads."""

    def __init__(self):
        self.items = []

    def empty(self, shape, dtype, label, device="cuda"):
        esz = torch.tensor([], dtype=dtype).element_size()
        n = int(np.prod(shape)) * esz
        back = torch.full((n + 2 * GUARD_BYTES,), GUARD_PATTERN, dtype=torch.uint8,
                          device=device)
        view = back[GUARD_BYTES:GUARD_BYTES + n].view(dtype).view(shape)
        self.items.append((label, back, n))
        return view

    def like(self, t, label, copy=False):
        if t is None:
            return None
        v = self.empty(tuple(t.shape), t.dtype, label, t.device)
        if copy:
            v.copy_(t)
        return v

    def check(self):
        torch.cuda.synchronize()
        for label, back, n in self.items:
            head = back[:GUARD_BYTES]
            tail = back[GUARD_BYTES + n:]
            bad_h = int((head != GUARD_PATTERN).sum())
            bad_t = int((tail != GUARD_PATTERN).sum())
            assert bad_h == 0 and bad_t == 0, ("%s: %d bytes before and %d bytes after the "
                                               "buffer were overwritten" % (label, bad_h, bad_t))
        return len(self.items)


LAYER_OUTPUTS = ("scores", "idx", "gate", "counts", "offsets", "src_token", "dst_row", "x_perm",
                 "x_perm_s", "x_q", "x_s", "y_perm", "y_shared", "out", "workspace", "saved")


def guard_layer(layer, guards=None):
    """Replace every output and scratch buffer of a MoeLayer (and the gradient
    buffers of its backward) by guarded ones of the same shape."""
    g = guards or Guards()
    for name in LAYER_OUTPUTS:
        t = getattr(layer, name, None)
        if isinstance(t, torch.Tensor):
            setattr(layer, name, g.like(t, name))
    return g


def guard_grads(layer, centroids, g):
    """Pre-allocate the backward's buffers of a training MoeLayer, guarded."""
    grads = layer._grad_buffers(centroids)
    layer.grads = {k: (g.like(v, "grad " + k) if isinstance(v, torch.Tensor) else v)
                   for k, v in grads.items()}
    return layer.grads


def host_inputs(inp):
    """torch dict -> numpy dict in the oracle's conventions"""
    return {k: (to_host(v) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def small_layer_inputs(cfg, seed=0, T=None):
    """generate on the host (so CPU and GPU tests see the same bytes), copy to GPU"""
    c = dict(cfg)
    if T is not None:
        c["T"] = T
    inp = moe_inputs.make_layer_inputs(c, seed, "cpu")
    dev = {k: v.cuda() for k, v in inp.items()}
    return c, inp, dev


class ExpertCodes:
    """The oracle's 128x128 block quantisation of one expert's weights at a time
    (host copy of the bf16 weights -> oracle quantiser), for ref["w13_q"][e]
    and the like; the last expert is kept."""

    def __init__(self, orc, w, part):
        self.orc, self.w, self.part = orc, w, part
        self.e, self.val = None, None

    def __getitem__(self, e):
        e = int(e)
        if self.e != e:
            self.val = self.orc.quant_weight_fp8(to_host(self.w[e]))
            self.e = e
        return self.val[self.part]


class RowsOf:
    """rows of a host array through an index map (a gather the oracle did)"""

    def __init__(self, a, src):
        self.a, self.src = a, src

    def __getitem__(self, r):
        return self.a[self.src[r]]


# ------------------------------------------------------------------ FP8 backward, step by step

def _ws_view(ws, off, n, dtype, shape):
    esz = torch.tensor([], dtype=dtype).element_size()
    return ws[off:off + n * esz].view(dtype).view(shape)


def check_fp8_backward_split(orc, layer, fwd, x_host, dout_host, what="", groups=None):
    """The FP8 expert backward checked step by step against the oracle's steps
    fed the GPU's own inputs (moe_expert_ffn_backward_fp8's workspace through
    moe_expert_ffn_backward_fp8_offsets):
      bytes, bit for bit: dY, [da db] 1x128 row tiles; the 128x1 row-direction
        tiles of dY, h, [da db] and x (oracle quantisers on the GPU's bf16 values)
      dh, dX, dW2, dW13: the oracle's GEMM on those codes, 6e-2 plain rule
      [da db]: the oracle's SwiGLU derivative of the GPU's dh, a, b, bf16 rule
      a, b, h (bf16): the oracle's recompute from the same codes, bf16 rule
    Groups: the routed experts (rows of x_perm) and the shared expert (index
    N); `groups` limits the check to some (default: all).  `fwd` holds the
    oracle's offsets, src_token, x_q_perm / x_s_perm (row-indexable), x_q /
    x_s, and the weight codes (w13_q[e] ..., ws13_q ...)."""
    import sparse_moe_layer_bias_amd as moe
    c = layer.c
    T, k, d, N, I = c["T"], c["k"], c["d"], c["N"], c["I"]
    Is = layer.cfg.inter_shared
    R, S = T * k, (T if Is > 0 else 0)
    Im = max(I, Is)
    g = layer.grads
    ws = g["workspace"]
    off = moe.moe_expert_ffn_backward_fp8_offsets(layer.cfg)
    Vd = lambda name, n, dt, shape: _ws_view(ws, off[name], n, dt, shape)
    if layer.saved is not None:
        so = moe.moe_expert_ffn_saved_offsets(layer.cfg)
        src, ab_o, h_o, abs_o, hs_o = layer.saved, so["ab"], so["h"], so["ab_sh"], so["h_sh"]
    else:
        src, ab_o, h_o, abs_o, hs_o = ws, off["ab"], off["h"], off["ab_sh"], off["h_sh"]
    dev = dict(
        ab=_ws_view(src, ab_o, R * 2 * I, torch.bfloat16, (R, 2 * I)),
        h=_ws_view(src, h_o, R * I, torch.bfloat16, (R, I)),
        dy=g["dy_perm"],
        dy_q=Vd("dy_q", R * d, torch.uint8, (R, d)),
        dy_s=Vd("dy_s", R * d // 128, torch.float32, (R, d // 128)),
        dh=Vd("dh", R * I, torch.bfloat16, (R, I)),
        dab=Vd("dab", R * 2 * I, torch.bfloat16, (R, 2 * I)),
        dab_q=Vd("dab_q", R * 2 * I, torch.uint8, (R, 2 * I)),
        dab_s=Vd("dab_s", R * 2 * I // 128, torch.float32, (R, 2 * I // 128)),
        dx=g["dx_perm"])
    if S:
        dev_sh = dict(
            ab=_ws_view(src, abs_o, S * 2 * Is, torch.bfloat16, (S, 2 * Is)),
            h=_ws_view(src, hs_o, S * Is, torch.bfloat16, (S, Is)),
            dy_q=Vd("dy_q_sh", S * d, torch.uint8, (S, d)),
            dy_s=Vd("dy_s_sh", S * d // 128, torch.float32, (S, d // 128)),
            dh=Vd("dh_sh", S * Is, torch.bfloat16, (S, Is)),
            dab=Vd("dab_sh", S * 2 * Is, torch.bfloat16, (S, 2 * Is)),
            dab_q=Vd("dab_q_sh", S * 2 * Is, torch.uint8, (S, 2 * Is)),
            dab_s=Vd("dab_s_sh", S * 2 * Is // 128, torch.float32, (S, 2 * Is // 128)),
            dx=g["dx_shared"])
    poff = to_host(Vd("poff", N + 2, torch.int32, (N + 2,)))
    offsets = np.asarray(fwd["offsets"], np.int64)
    M_g = [int(offsets[e + 1] - offsets[e]) for e in range(N)] + [S]
    assert_bits(poff, np.concatenate([[0], np.cumsum([(m + 127) // 128 * 128 for m in M_g])])
                .astype(np.int32), what + "padded offsets")
    P = int(poff[-1])
    col = {}
    for name, F in (("col_dy", d), ("col_h", Im), ("col_dab", 2 * Im), ("col_x", d)):
        col[name] = (Vd(name, P * F, torch.uint8, (P // 128, F, 128)),
                     Vd(name + "_s", P // 128 * F, torch.float32, (P // 128, F)))

    def cols_of(name, gi, C):
        q, s = col[name]
        pb0, M = int(poff[gi]) // 128, M_g[gi]
        nb = (M + 127) // 128
        qh = to_host(q[pb0:pb0 + nb, :C, :])
        codes = qh.transpose(0, 2, 1).reshape(nb * 128, C)[:M]
        return np.ascontiguousarray(codes), np.ascontiguousarray(to_host(s[pb0:pb0 + nb, :C]))

    def bits(a, b, label):
        if a.dtype == np.float32:
            a, b = a.view(np.uint32), b.view(np.uint32)
        assert_bits(a, b, what + label)

    src_tok = fwd["src_token"]
    dw2, dw13 = g["dw2"], g["dw13"]
    err = {"dh": 0.0, "dab": 0.0, "dx": 0.0, "dw2": 0.0, "dw13": 0.0, "ab": 0.0}
    if groups is None:
        groups = range(N + (1 if S else 0))
    for e in groups:
        shared = e == N
        M = M_g[e]
        if M == 0:
            assert not torch.any(dw2[e]) and not torch.any(dw13[e])
            continue
        if shared:
            Ie, w13q, w13s, w2q, w2s = Is, fwd["ws13_q"], fwd["ws13_s"], fwd["ws2_q"], fwd["ws2_s"]
            a_in, as_in = fwd["x_q"], fwd["x_s"]
            G = {n: to_host(v) for n, v in dev_sh.items()}
            G["dy"] = dout_host
            x_e = x_host
            dw2_e, dw13_e = to_host(g["dws2"]), to_host(g["dws13"])
        else:
            a0, a1 = int(offsets[e]), int(offsets[e + 1])
            Ie, w13q, w13s, w2q, w2s = I, fwd["w13_q"][e], fwd["w13_s"][e], fwd["w2_q"][e], \
                fwd["w2_s"][e]
            rows = np.arange(a0, a1)
            a_in, as_in = fwd["x_q_perm"][rows], fwd["x_s_perm"][rows]
            G = {n: to_host(v[a0:a1]) for n, v in dev.items()}
            x_e = x_host[src_tok[a0:a1]]
            dw2_e, dw13_e = to_host(dw2[e]), to_host(dw13[e])
        label = "(group %d)" % e
        for vals, codes, scales, nm in ((G["dy"], G["dy_q"], G["dy_s"], "dY"),
                                        (G["dab"], G["dab_q"], G["dab_s"], "[da db]")):
            q, s = orc.quant_act_fp8(vals)
            bits(codes, q, "%s row-tile codes %s" % (nm, label))
            bits(scales, s, "%s row-tile scales %s" % (nm, label))
        ab_ref, h_ref = orc.fp8_recompute_ab(a_in, as_in, w13q, w13s)
        err["ab"] = max(err["ab"], max_rule_err(G["ab"], ab_ref), max_rule_err(G["h"], h_ref))
        assert_close(G["ab"], ab_ref, RTOL["bf16"], what + "a, b " + label)
        assert_close(G["h"], h_ref, RTOL["bf16"], what + "h " + label)
        dh_ref = orc.fp8_dgrad(G["dy_q"], G["dy_s"], w2q, w2s)
        dab_ref = orc.swiglu_bwd_bf16(G["dh"], G["ab"])
        dx_ref = orc.fp8_dgrad(G["dab_q"], G["dab_s"], w13q, w13s)
        for n, (gv, rv) in (("dh", (G["dh"], dh_ref)), ("dab", (G["dab"], dab_ref)),
                            ("dx", (G["dx"], dx_ref))):
            err[n] = max(err[n], max_rule_err(gv, rv))
        assert_close_fp8(G["dh"], dh_ref, what + "dh " + label)
        assert_close(G["dab"], dab_ref, RTOL["bf16"], what + "[da db] " + label)
        assert_close_fp8(G["dx"], dx_ref, what + "dX " + label)
        cdy = cols_of("col_dy", e, d)
        ch = cols_of("col_h", e, Ie)
        ct = cols_of("col_dab", e, 2 * Ie)
        cx = cols_of("col_x", e, d)
        for (cq, cs), v, nm in ((cdy, G["dy"], "dY"), (ch, G["h"], "h"),
                                (ct, G["dab"], "[da db]"), (cx, x_e, "x")):
            q, s = orc.quant_cols_fp8(v)
            bits(cq, q, "%s row-direction codes %s" % (nm, label))
            bits(cs, s, "%s row-direction scales %s" % (nm, label))
        w2_ref = orc.fp8_wgrad(*cdy, *ch)
        w13_ref = orc.fp8_wgrad(*ct, *cx)
        err["dw2"] = max(err["dw2"], max_rule_err(dw2_e, w2_ref))
        err["dw13"] = max(err["dw13"], max_rule_err(dw13_e, w13_ref))
        assert_close_fp8(dw2_e, w2_ref, what + "dW2 " + label)
        assert_close_fp8(dw13_e, w13_ref, what + "dW13 " + label)
    log(what + "FP8 backward steps, max error (row rule): " +
        ", ".join("%s %.2e" % kv for kv in err.items()))
    return err
