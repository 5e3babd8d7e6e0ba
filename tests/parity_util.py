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


def assert_close_fp8(got, ref, what="", rtol=RTOL["fp8"], elem=2.0):
    """FP8 expert outputs.  Both sides re-quantise h = silu(a)*b to E4M3 per
    1x128 tile from fp32 values that differ in the last bits (the kernel sums
    in MFMA order, the oracle exactly), so an h code at a rounding midpoint can
    legitimately differ and move the outputs of its row by up to a code step.
    Criterion: every element within elem*rtol (elem = 2), at least 99.99%
    within rtol (elementwise rule as in assert_close; an element that is zero
    on both sides, e.g. the gradient of an expert without rows, agrees), and
    each row's relative L2 error within rtol."""
    g, r = to_f64(got), to_f64(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    if r.size == 0:
        return
    r2 = r.reshape(-1, r.shape[-1])
    g2 = g.reshape(r2.shape)
    rms = np.sqrt(np.mean(r2 ** 2, axis=1, keepdims=True))
    den = np.abs(r2) + rms
    err = np.abs(g2 - r2)
    rel = np.where(den > 0, err / np.where(den > 0, den, 1.0), np.where(err > 0, np.inf, 0.0))
    frac_out = float(np.mean(rel > rtol))
    assert np.all(rel <= elem * rtol), "%s: max elementwise rel err %.3g > %g" % (
        what, float(rel.max()), elem * rtol)
    assert frac_out <= 1e-4, "%s: %.2e of elements beyond %g" % (what, frac_out, rtol)
    row = np.linalg.norm(g2 - r2, axis=1) / np.maximum(np.linalg.norm(r2, axis=1), 1e-30)
    assert np.all(row <= rtol), "%s: row L2 rel err %.3g > %g" % (what, float(row.max()), rtol)


def assert_close_fp8_grad(got, ref, what="", rtol=RTOL["fp8"], elem=3.0):
    """FP8 weight gradients [experts..., rows, cols].  Criterion as
    assert_close_fp8 (elem = 3, see the FP8 backward tests), with each
    element's scale the larger of its row's RMS and its expert matrix's RMS,
    and the relative L2 error taken per expert matrix.  A weight-gradient row
    of an expert with few rows is nearly an outer product scaled by one
    gradient value, which may be a near-cancelling sum: such a row can be far
    below the matrix's scale, and its own RMS is then no measure of the error
    (as for the fp32 gradients)."""
    g, r = to_f64(got), to_f64(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    if r.size == 0:
        return
    g3 = g.reshape((-1,) + g.shape[-2:])
    r3 = r.reshape(g3.shape)
    rms_row = np.sqrt(np.mean(r3 ** 2, axis=2, keepdims=True))
    rms_mat = np.sqrt(np.mean(r3 ** 2, axis=(1, 2), keepdims=True))
    den = np.abs(r3) + np.maximum(rms_row, rms_mat)
    err = np.abs(g3 - r3)
    rel = np.where(den > 0, err / np.where(den > 0, den, 1.0), np.where(err > 0, np.inf, 0.0))
    assert np.all(rel <= elem * rtol), "%s: max elementwise rel err %.3g > %g at %s" % (
        what, float(rel.max()), elem * rtol, np.unravel_index(int(np.argmax(rel)), rel.shape))
    frac_out = float(np.mean(rel > rtol))
    assert frac_out <= 1e-4, "%s: %.2e of elements beyond %g" % (what, frac_out, rtol)
    for i in range(r3.shape[0]):
        nr = np.linalg.norm(r3[i])
        ne = np.linalg.norm(g3[i] - r3[i])
        assert ne <= rtol * nr or (nr == 0 and ne == 0), "%s[%d]: L2 rel err %.3g" % (
            what, i, ne / max(nr, 1e-300))


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
