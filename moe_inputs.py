"""Seeded synthetic inputs for the DeepSeekMoE layer, shared by the HIP path's
tests/benchmark and by the CPU oracle.

This module holds no arithmetic of the layer itself: only the workload table
and random-number recipes.  Every tensor is drawn from its own seeded
``torch.Generator`` (one per tensor and, for expert weights, one per expert),
as fp32 normals times the stated standard deviation, then cast to the storage
dtype (bf16 round-to-nearest-even).  The same bytes go to both sides.

Workload shapes follow DeepSeek-V3's MoE layer as the pages state it (1 shared
+ 256 routed experts, 8 active; reading guide "Kernideen", first bullet), at
the five sizes below.  No dataset is involved: the layer forward is
token-wise, so synthetic hidden states of the right shape and distribution
stand in for real activations.
"""
import hashlib
import math

import torch

CONFIGS = {
    # small case the oracle finishes in seconds; fp32 throughout
    "tiny_fp32": dict(T=64, d=128, N=16, k=2, G=1, TG=1, I=64, Is=64, dtype="f32",
                      fp8=False, bias_std=0.0, w_std="d"),
    # mid size, bf16, no group limit
    "mid_bf16": dict(T=2048, d=1024, N=64, k=8, G=1, TG=1, I=512, Is=512, dtype="bf16",
                     fp8=False, bias_std=1e-3, w_std="fan_in"),
    # DeepSeek-V3 layer shape, bf16 expert GEMMs
    "v3_bf16": dict(T=8192, d=7168, N=256, k=8, G=8, TG=4, I=2048, Is=2048, dtype="bf16",
                    fp8=False, bias_std=1e-3, w_std="fan_in"),
    # same shape, FP8 E4M3 expert GEMMs (1x128 activation tiles, 128x128 weight blocks)
    "v3_fp8": dict(T=8192, d=7168, N=256, k=8, G=8, TG=4, I=2048, Is=2048, dtype="bf16",
                   fp8=True, bias_std=1e-3, w_std="fan_in"),
    # decode-step batches with Zipf-skewed expert popularity, 100 balancing steps
    "skew_balance": dict(T=128, d=7168, N=256, k=8, G=1, TG=1, I=2048, Is=2048,
                         dtype="bf16", fp8=False, bias_std=0.0, w_std="fan_in",
                         steps=100, zipf_s=1.2),
}


def _seed(seed, *key):
    h = hashlib.sha256(("%d|" % seed + "|".join(str(k) for k in key)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, seed, *key):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, *key))
    return g


def normal(shape, std, device, seed, *key):
    """fp32 N(0, std^2) draws from a generator keyed by (seed, *key)."""
    t = torch.randn(shape, generator=_gen(device, seed, *key), device=device,
                    dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def storage(t, dtype):
    return t.to(torch.bfloat16) if dtype == "bf16" else t.to(torch.float32)


def _wstd(cfg, fan_in):
    return 1.0 / math.sqrt(cfg["d"] if cfg["w_std"] == "d" else fan_in)


def make_router_inputs(cfg, seed=0, device="cpu"):
    """x [T,d], centroids [N,d] fp32, bias [N] fp32."""
    T, d, N = cfg["T"], cfg["d"], cfg["N"]
    x = storage(normal((T, d), 1.0, device, seed, "x"), cfg["dtype"])
    centroids = normal((N, d), 1.0 / math.sqrt(d), device, seed, "centroids")
    if cfg["bias_std"] > 0:
        bias = normal((N,), cfg["bias_std"], device, seed, "bias")
    else:
        bias = torch.zeros(N, dtype=torch.float32, device=device)
    return dict(x=x, centroids=centroids, bias=bias)


def make_expert_weights(cfg, experts, seed=0, device="cpu"):
    """w13 [len(experts), 2I, d] (W1 rows then W3 rows) and w2 [len(experts), d, I],
    each expert from its own generator, so any subset can be regenerated alone."""
    d, I, dt = cfg["d"], cfg["I"], cfg["dtype"]
    n = len(experts)
    w13 = torch.empty((n, 2 * I, d), dtype=torch.bfloat16 if dt == "bf16" else torch.float32,
                      device=device)
    w2 = torch.empty((n, d, I), dtype=w13.dtype, device=device)
    for j, e in enumerate(experts):
        w13[j] = storage(normal((2 * I, d), _wstd(cfg, d), device, seed, "w13", e), dt)
        w2[j] = storage(normal((d, I), _wstd(cfg, I), device, seed, "w2", e), dt)
    return w13, w2


def make_shared_weights(cfg, seed=0, device="cpu"):
    d, Is, dt = cfg["d"], cfg["Is"], cfg["dtype"]
    ws13 = storage(normal((2 * Is, d), _wstd(cfg, d), device, seed, "ws13"), dt)
    ws2 = storage(normal((d, Is), _wstd(cfg, Is), device, seed, "ws2"), dt)
    return ws13, ws2


def make_layer_inputs(cfg, seed=0, device="cpu"):
    inp = make_router_inputs(cfg, seed, device)
    w13, w2 = make_expert_weights(cfg, range(cfg["N"]), seed, device)
    ws13, ws2 = make_shared_weights(cfg, seed, device)
    inp.update(w13=w13, w2=w2, ws13=ws13, ws2=ws2)
    return inp


def make_upstream_grad(cfg, seed=0, device="cpu", T=None):
    """dL/dh' [T, d] for the backward: N(0, 1) in the storage dtype."""
    T = cfg["T"] if T is None else T
    return storage(normal((T, cfg["d"]), 1.0, device, seed, "dout"), cfg["dtype"])


# ------------------------------------------------------------------ skewed routing

def make_skew_centroids(cfg, seed=0, device="cpu", c=1.0):
    """Centroids for Zipf-skewed expert popularity.  Hidden coordinate 0 of every
    token is held at 1.0; the expert at popularity rank r (1-based, ranks are a
    seeded random permutation of the expert ids) gets centroid coordinate 0 equal
    to -c * s * ln(r), so its logit is that offset plus the N(0, ~1) contribution
    of the other coordinates.  Other coordinates ~ N(0, 1/d)."""
    N, d = cfg["N"], cfg["d"]
    e = normal((N, d), 1.0 / math.sqrt(d), device, seed, "skew_centroids")
    perm = torch.randperm(N, generator=_gen("cpu", seed, "skew_rank"))
    rank = torch.empty(N, dtype=torch.float64)
    rank[perm] = torch.arange(1, N + 1, dtype=torch.float64)
    offs = (-c * cfg["zipf_s"] * torch.log(rank)).to(torch.float32)
    e[:, 0] = offs.to(device)
    return e


def make_skew_tokens(cfg, step, seed=0, device="cpu"):
    """A fresh decode batch for each step: x ~ N(0,1) with coordinate 0 = 1.0."""
    x = normal((cfg["T"], cfg["d"]), 1.0, device, seed, "skew_x", step)
    x[:, 0] = 1.0
    return storage(x, cfg["dtype"])


# ------------------------------------------------------------------ host views

def to_host(t):
    """torch tensor -> numpy in the oracle's conventions (bf16 as uint16 bits)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()
