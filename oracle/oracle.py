"""Python face of the CPU oracle (test infrastructure only).

Only the test-suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  It loads ``oracle/liboracle.so`` (built
from ``moe_oracle.c`` by ``oracle/build.py``) through ctypes and works on numpy
arrays in host memory.  It never imports the HIP library and shares no code
with it.

Array conventions: fp32 tensors are ``np.float32``; bf16 tensors are carried
as their bit patterns in ``np.uint16``; FP8 E4M3 codes are ``np.uint8``;
indices are ``np.int32``.

What each function computes, and the passage it follows, is stated in
``moe_oracle.c``.  Sources: the DeepSeek-V3 report reading guide
(xyznot.com/de, "Methode" item 2 for the layer; "Kernideen" FP8 bullet for the
tiles and blocks) and the singularity-lens summary's formula paragraph (bias
sign rule, FP8 scale rule).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1

GAMMA = np.float32(0.001)  # [P4] end-of-step bias step, as the nearest fp32

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build()
        _lib = ctypes.CDLL(_LIB_PATH)
        _declare(_lib)
    return _lib


def set_threads(n):
    """OpenMP threads of the oracle's next calls (timing only); returns the
    previous maximum."""
    L = lib()
    L.orc_set_threads.argtypes = [ctypes.c_int]
    L.orc_set_threads.restype = ctypes.c_int
    return int(L.orc_set_threads(int(n)))


def _declare(L):
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    F = ctypes.c_float
    sig = {
        "orc_logits": [I64, I64, I64, I, P, P, P],
        "orc_sigmoid": [I64, P, P],
        "orc_select": [I64, I64, I64, I64, I64, P, P, P, P],
        "orc_histogram": [I64, I64, I64, P, P],
        "orc_route": [I64, I64, I64, I64, I64, I64, I, P, P, P, P, P, P, P],
        "orc_permute": [I64, I64, I64, P, P, P, P],
        "orc_gather_rows": [I64, I64, P, P, P],
        "orc_swiglu_ffn": [I64, I64, I64, I, P, P, P, P],
        "orc_e4m3_encode_array": [I64, P, P],
        "orc_e4m3_decode_array": [I64, P, P],
        "orc_quant_act_fp8": [I64, I64, I, P, P, P],
        "orc_quant_weight_fp8": [I64, I64, I64, I, P, P, P],
        "orc_swiglu_ffn_fp8": [I64, I64, I64, P, P, P, P, P, P, P],
        "orc_swiglu_gateup_fp8": [I64, I64, I64, P, P, P, P, P],
        "orc_ffn_down_fp8": [I64, I64, I64, P, P, P, P, P],
        "orc_combine": [I64, I64, I64, I, P, P, P, P, P, P],
        "orc_bias_update": [I64, I64, P, F, P],
        "orc_seq_balance_loss": [I64, I64, I64, I64, F, P, P, P],
        "orc_round_to_dtype": [I64, I, P, P],
        "orc_combine_backward": [I64, I64, I64, I, P, P, P, P, P, P],
        "orc_swiglu_ffn_backward": [I64, I64, I64, I, P, P, P, P, P, P, P],
        "orc_route_backward": [I64, I64, I64, P, P, P, P],
        "orc_centroid_grad": [I64, I64, I64, I64, I, P, P, P, P],
        "orc_input_grad": [I64, I64, I64, I, P, P, P, P, P, P, P, P],
        "orc_quant_cols_fp8": [I64, I64, I, P, P, P],
        "orc_swiglu_ffn_backward_fp8": [I64, I64, I64] + [P] * 11,
        "orc_fp8_recompute_ab": [I64, I64, I64, P, P, P, P, P, P],
        "orc_fp8_dgrad": [I64, I64, I64, P, P, P, P, P],
        "orc_swiglu_bwd_bf16": [I64, I64, P, P, P],
        "orc_fp8_wgrad": [I64, I64, I64, P, P, P, P, P],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = None


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    return a


def dtype_code(arr):
    if arr.dtype == np.uint16:
        return BF16
    if arr.dtype == np.float32:
        return F32
    raise TypeError("activations/weights must be float32 or bf16 bits (uint16)")


# ---------------------------------------------------------------- routing

def logits(x, centroids):
    """z[t,i]: fixed-order fp32 FMA chain of x[t,:] against centroid i."""
    x = np.ascontiguousarray(x)
    E = _c(centroids, np.float32)
    T, d = x.shape
    N = E.shape[0]
    z = np.empty((T, N), np.float32)
    lib().orc_logits(T, d, N, dtype_code(x), _p(x), _p(E), _p(z))
    return z


def sigmoid(z):
    z = _c(z, np.float32)
    s = np.empty_like(z)
    lib().orc_sigmoid(z.size, _p(z), _p(s))
    return s


def select(s, bias, k, n_group=1, topk_group=1):
    """Biased top-k (group-limited when n_group > 1) and normalised gates."""
    s = _c(s, np.float32)
    b = _c(bias, np.float32)
    T, N = s.shape
    _check_route_shape(N, k, n_group, topk_group)
    idx = np.empty((T, k), np.int32)
    gate = np.empty((T, k), np.float32)
    lib().orc_select(T, N, k, n_group, topk_group, _p(s), _p(b), _p(idx), _p(gate))
    return idx, gate


def _check_route_shape(N, k, G, TG):
    if G < 1 or N % G or (G > 1 and (N // G < 2 or TG < 1 or TG > G or G > 1024)):
        raise ValueError("bad group shape")
    if G > 1 and k > TG * (N // G):
        raise ValueError("k exceeds the experts in the kept groups")
    if not (1 <= k <= N):
        raise ValueError("bad k")


def histogram(idx, N):
    idx = _c(idx, np.int32)
    T, k = idx.shape
    counts = np.empty(N, np.int32)
    lib().orc_histogram(T, k, N, _p(idx), _p(counts))
    return counts


def route(x, centroids, bias, k, n_group=1, topk_group=1, want_scores=False):
    x = np.ascontiguousarray(x)
    E = _c(centroids, np.float32)
    b = _c(bias, np.float32)
    T, d = x.shape
    N = E.shape[0]
    _check_route_shape(N, k, n_group, topk_group)
    scores = np.empty((T, N), np.float32) if want_scores else None
    idx = np.empty((T, k), np.int32)
    gate = np.empty((T, k), np.float32)
    counts = np.empty(N, np.int32)
    lib().orc_route(T, d, N, k, n_group, topk_group, dtype_code(x), _p(x), _p(E), _p(b),
                    _p(scores), _p(idx), _p(gate), _p(counts))
    out = {"idx": idx, "gate": gate, "counts": counts}
    if want_scores:
        out["scores"] = scores
    return out


# ---------------------------------------------------------------- permute

def permute(idx, N):
    """Stable counting sort by expert -> offsets[N+1], src_token[T*k], dst_row[T,k]."""
    idx = _c(idx, np.int32)
    T, k = idx.shape
    offsets = np.empty(N + 1, np.int32)
    src = np.empty(T * k, np.int32)
    dst = np.empty((T, k), np.int32)
    lib().orc_permute(T, k, N, _p(idx), _p(offsets), _p(src), _p(dst))
    return offsets, src, dst


def gather_rows(x, src):
    x = np.ascontiguousarray(x)
    src = _c(src, np.int32)
    rows = src.shape[0]
    out = np.empty((rows,) + x.shape[1:], x.dtype)
    row_bytes = x[0].nbytes if x.shape[0] else 0
    lib().orc_gather_rows(rows, row_bytes, _p(src), _p(x), _p(out))
    return out


# ---------------------------------------------------------------- expert FFN

def swiglu_ffn(A, w13, w2):
    """One expert over the rows A [M,d]; w13 [2I,d] (W1 rows then W3 rows), w2 [d,I]."""
    A = np.ascontiguousarray(A)
    w13 = np.ascontiguousarray(w13)
    w2 = np.ascontiguousarray(w2)
    dt = dtype_code(A)
    assert dtype_code(w13) == dt and dtype_code(w2) == dt
    M, d = A.shape
    I = w13.shape[0] // 2
    assert w13.shape == (2 * I, d) and w2.shape == (d, I)
    y = np.empty((M, d), A.dtype)
    lib().orc_swiglu_ffn(M, d, I, dt, _p(A), _p(w13), _p(w2), _p(y))
    return y


# ---------------------------------------------------------------- FP8

def e4m3_encode(v):
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().orc_e4m3_encode_array(v.size, _p(v), _p(out))
    return out


def e4m3_decode(c):
    c = _c(c, np.uint8)
    out = np.empty(c.shape, np.float32)
    lib().orc_e4m3_decode_array(c.size, _p(c), _p(out))
    return out


def quant_act_fp8(x):
    """1x128 tiles along the last axis -> codes [rows, cols], scales [rows, cols/128]."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    assert cols % 128 == 0
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, cols // 128), np.float32)
    lib().orc_quant_act_fp8(rows, cols, dtype_code(x), _p(x), _p(q), _p(s))
    return q, s


def quant_weight_fp8(w):
    """128x128 blocks of each matrix -> codes, scales [.., rows/128, cols/128]."""
    w = np.ascontiguousarray(w)
    lead = w.shape[:-2]
    rows, cols = w.shape[-2:]
    assert rows % 128 == 0 and cols % 128 == 0
    n = int(np.prod(lead)) if lead else 1
    q = np.empty(w.shape, np.uint8)
    s = np.empty(lead + (rows // 128, cols // 128), np.float32)
    lib().orc_quant_weight_fp8(n, rows, cols, dtype_code(w), _p(w), _p(q), _p(s))
    return q, s


def quant_cols_fp8(x):
    """128x1 tiles down the rows (blocks of 128 rows from row 0, the last one
    partial) -> codes [rows, cols], scales [ceil(rows/128), cols]."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty(((rows + 127) // 128, cols), np.float32)
    lib().orc_quant_cols_fp8(rows, cols, dtype_code(x), _p(x), _p(q), _p(s))
    return q, s


def swiglu_ffn_fp8(Aq, As, w13q, w13s, w2q, w2s):
    Aq = _c(Aq, np.uint8)
    As = _c(As, np.float32)
    w13q = _c(w13q, np.uint8)
    w13s = _c(w13s, np.float32)
    w2q = _c(w2q, np.uint8)
    w2s = _c(w2s, np.float32)
    M, d = Aq.shape
    I = w13q.shape[0] // 2
    y = np.empty((M, d), np.uint16)
    lib().orc_swiglu_ffn_fp8(M, d, I, _p(Aq), _p(As), _p(w13q), _p(w13s), _p(w2q), _p(w2s),
                             _p(y))
    return y


def swiglu_gateup_fp8(Aq, As, w13q, w13s):
    """The gate/up half of the FP8 expert: h = silu(a) * b in fp32 [M, I], from
    block-scaled sums a, b rounded to fp32."""
    Aq = _c(Aq, np.uint8)
    As = _c(As, np.float32)
    w13q = _c(w13q, np.uint8)
    w13s = _c(w13s, np.float32)
    M, d = Aq.shape
    I = w13q.shape[0] // 2
    assert w13q.shape == (2 * I, d) and As.shape == (M, d // 128)
    h = np.empty((M, I), np.float32)
    lib().orc_swiglu_gateup_fp8(M, d, I, _p(Aq), _p(As), _p(w13q), _p(w13s), _p(h))
    return h


def ffn_down_fp8(hq, hs, w2q, w2s):
    """The down half of the FP8 expert from h's 1x128 codes and tile scales:
    y [M, d] as bf16 bits."""
    hq = _c(hq, np.uint8)
    hs = _c(hs, np.float32)
    w2q = _c(w2q, np.uint8)
    w2s = _c(w2s, np.float32)
    M, I = hq.shape
    d = w2q.shape[0]
    assert w2q.shape == (d, I) and hs.shape == (M, I // 128)
    y = np.empty((M, d), np.uint16)
    lib().orc_ffn_down_fp8(M, I, d, _p(hq), _p(hs), _p(w2q), _p(w2s), _p(y))
    return y


# ---------------------------------------------------------------- combine, bias

def combine(x, y_shared, y_perm, gate, dst_row, dtype):
    """out = x + y_shared + sum_j gate_j * y_perm[dst_row_j]; x / y_shared may be None."""
    y_perm = np.ascontiguousarray(y_perm)
    gate = _c(gate, np.float32)
    dst = _c(dst_row, np.int32)
    T, k = gate.shape
    d = y_perm.shape[1]
    dt = BF16 if dtype == "bf16" else F32
    npdt = np.uint16 if dt == BF16 else np.float32
    if x is not None:
        x = _c(x, npdt)
    if y_shared is not None:
        y_shared = _c(y_shared, npdt)
    out = np.empty((T, d), npdt)
    lib().orc_combine(T, d, k, dt, _p(x), _p(y_shared), _p(y_perm), _p(gate), _p(dst), _p(out))
    return out


def bias_update(counts, tokens_times_k, bias, gamma=GAMMA):
    """Return the bias after one end-of-step update (the input is not modified)."""
    counts = _c(counts, np.int32)
    b = np.array(bias, dtype=np.float32, copy=True)
    lib().orc_bias_update(counts.size, int(tokens_times_k), _p(counts),
                          ctypes.c_float(float(gamma)), _p(b))
    return b


def seq_balance_loss(scores, idx, seq_len, alpha=1e-4):
    """Per-sequence balance loss [T / seq_len] fp32 of moe_oracle.c's reading
    (sequences of seq_len consecutive tokens; alpha taken as fp32)."""
    scores = _c(scores, np.float32)
    idx = _c(idx, np.int32)
    T, N = scores.shape
    k = idx.shape[1]
    if seq_len < 1 or T % seq_len:
        raise ValueError("T must be a multiple of seq_len")
    out = np.empty(T // seq_len, np.float32)
    lib().orc_seq_balance_loss(T, N, k, int(seq_len), ctypes.c_float(float(alpha)),
                               _p(scores), _p(idx), _p(out))
    return out


def round_to_dtype(v, dtype):
    v = _c(np.asarray(v, np.float64), np.float64)
    dt = BF16 if dtype == "bf16" else F32
    out = np.empty(v.shape, np.uint16 if dt == BF16 else np.float32)
    lib().orc_round_to_dtype(v.size, dt, _p(v), _p(out))
    return out


# ---------------------------------------------------------------- whole layer

def layer_forward(inp, cfg, residual=True):
    """Every step of the layer on host arrays, in order.  ``inp`` holds numpy
    arrays: x, centroids, bias, w13 [N,2I,d], w2 [N,d,I], ws13 [2Is,d], ws2 [d,Is]
    (bf16 as uint16 bits, or float32).  Returns a dict of every intermediate."""
    k, G, TG = cfg["k"], cfg["G"], cfg["TG"]
    N = cfg["N"]
    x = inp["x"]
    r = route(x, inp["centroids"], inp["bias"], k, G, TG, want_scores=True)
    offsets, src, dst = permute(r["idx"], N)
    T, d = x.shape
    fp8 = cfg.get("fp8", False)
    dt = "bf16" if x.dtype == np.uint16 else "f32"
    if fp8:
        xq, xs = quant_act_fp8(x)
        xq_perm = gather_rows(xq, src)
        xs_perm = gather_rows(xs, src)
        w13q, w13s = quant_weight_fp8(inp["w13"])
        w2q, w2s = quant_weight_fp8(inp["w2"])
        ws13q, ws13s = quant_weight_fp8(inp["ws13"])
        ws2q, ws2s = quant_weight_fp8(inp["ws2"])
        y_perm = np.empty((T * k, d), np.uint16)
        for e in range(N):
            a, b = offsets[e], offsets[e + 1]
            if b > a:
                y_perm[a:b] = swiglu_ffn_fp8(xq_perm[a:b], xs_perm[a:b], w13q[e], w13s[e],
                                             w2q[e], w2s[e])
        y_shared = swiglu_ffn_fp8(xq, xs, ws13q, ws13s, ws2q, ws2s)
        x_perm = None
    else:
        x_perm = gather_rows(x, src)
        y_perm = np.empty((T * k, d), x.dtype)
        for e in range(N):
            a, b = offsets[e], offsets[e + 1]
            if b > a:
                y_perm[a:b] = swiglu_ffn(x_perm[a:b], inp["w13"][e], inp["w2"][e])
        y_shared = swiglu_ffn(x, inp["ws13"], inp["ws2"]) if inp.get("ws13") is not None else None
    out = combine(x if residual else None, y_shared, y_perm, r["gate"], dst, dt)
    new_bias = bias_update(r["counts"], T * k, inp["bias"])
    res = dict(r)
    res.update(offsets=offsets, src_token=src, dst_row=dst, x_perm=x_perm, y_perm=y_perm,
               y_shared=y_shared, out=out, new_bias=new_bias)
    if fp8:
        res.update(x_q=xq, x_s=xs, x_q_perm=xq_perm, x_s_perm=xs_perm, w13_q=w13q, w13_s=w13s,
                   w2_q=w2q, w2_s=w2s, ws13_q=ws13q, ws13_s=ws13s, ws2_q=ws2q, ws2_s=ws2s)
    return res


# ---------------------------------------------------------------- backward

def combine_backward(dout, y_perm, gate, dst_row):
    """dy_perm[dst[t,j]] = gate[t,j] * dout[t] (dtype), dgate[t,j] = dout[t] . y_perm[dst[t,j]]."""
    dout = np.ascontiguousarray(dout)
    y_perm = _c(y_perm, dout.dtype)
    gate = _c(gate, np.float32)
    dst = _c(dst_row, np.int32)
    T, k = gate.shape
    d = dout.shape[1]
    dy_perm = np.empty((T * k, d), dout.dtype)
    dgate = np.empty((T, k), np.float32)
    lib().orc_combine_backward(T, d, k, dtype_code(dout), _p(dout), _p(y_perm), _p(gate),
                               _p(dst), _p(dy_perm), _p(dgate))
    return dy_perm, dgate


def swiglu_ffn_backward(A, w13, w2, dY):
    """One expert's backward: (dA [M,d], dw13 [2I,d], dw2 [d,I]) for the rows A
    and the output gradient dY."""
    A = np.ascontiguousarray(A)
    dt = dtype_code(A)
    w13 = _c(w13, A.dtype)
    w2 = _c(w2, A.dtype)
    dY = _c(dY, A.dtype)
    M, d = A.shape
    I = w13.shape[0] // 2
    assert w13.shape == (2 * I, d) and w2.shape == (d, I) and dY.shape == (M, d)
    dA = np.empty((M, d), A.dtype)
    dw13 = np.empty((2 * I, d), A.dtype)
    dw2 = np.empty((d, I), A.dtype)
    lib().orc_swiglu_ffn_backward(M, d, I, dt, _p(A), _p(w13), _p(w2), _p(dY), _p(dA),
                                  _p(dw13), _p(dw2))
    return dA, dw13, dw2


def swiglu_ffn_backward_fp8(Aq, As, A, w13q, w13s, w2q, w2s, dY):
    """One FP8 expert's backward: (dA [M,d], dw13 [2I,d], dw2 [d,I]) in bf16
    bits, from the forward's activation tiles (Aq, As), the same rows in bf16
    (A), the forward's weight blocks and the bf16 output gradient dY."""
    Aq = _c(Aq, np.uint8)
    As = _c(As, np.float32)
    A = _c(A, np.uint16)
    w13q = _c(w13q, np.uint8)
    w13s = _c(w13s, np.float32)
    w2q = _c(w2q, np.uint8)
    w2s = _c(w2s, np.float32)
    dY = _c(dY, np.uint16)
    M, d = Aq.shape
    I = w13q.shape[0] // 2
    assert A.shape == (M, d) and dY.shape == (M, d) and w2q.shape == (d, I)
    dA = np.empty((M, d), np.uint16)
    dw13 = np.empty((2 * I, d), np.uint16)
    dw2 = np.empty((d, I), np.uint16)
    lib().orc_swiglu_ffn_backward_fp8(M, d, I, _p(Aq), _p(As), _p(A), _p(w13q), _p(w13s),
                                      _p(w2q), _p(w2s), _p(dY), _p(dA), _p(dw13), _p(dw2))
    return dA, dw13, dw2


def fp8_recompute_ab(Aq, As, w13q, w13s):
    """The FP8 forward's a, b kept in bf16 ([M, 2I] = [a | b]) and h = bf16(silu(a) b)."""
    Aq, As = _c(Aq, np.uint8), _c(As, np.float32)
    w13q, w13s = _c(w13q, np.uint8), _c(w13s, np.float32)
    M, d = Aq.shape
    I = w13q.shape[0] // 2
    ab = np.empty((M, 2 * I), np.uint16)
    h = np.empty((M, I), np.uint16)
    lib().orc_fp8_recompute_ab(M, d, I, _p(Aq), _p(As), _p(w13q), _p(w13s), _p(ab), _p(h))
    return ab, h


def fp8_dgrad(gq, gs, wq, ws):
    """bf16(g W) for gradient rows g in 1x128 tiles along K (codes [M, K], scales
    [M, K/128]) and a weight matrix W [K, N] in 128x128 blocks (codes, scales
    [K/128, N/128])."""
    gq, gs = _c(gq, np.uint8), _c(gs, np.float32)
    wq, ws = _c(wq, np.uint8), _c(ws, np.float32)
    M, K = gq.shape
    N = wq.shape[1]
    assert wq.shape == (K, N) and gs.shape == (M, K // 128) and ws.shape == (K // 128, N // 128)
    out = np.empty((M, N), np.uint16)
    lib().orc_fp8_dgrad(M, K, N, _p(gq), _p(gs), _p(wq), _p(ws), _p(out))
    return out


def swiglu_bwd_bf16(dh, ab):
    """[da | db] in bf16 from bf16 dh [M, I] and [a | b] [M, 2I]."""
    dh, ab = _c(dh, np.uint16), _c(ab, np.uint16)
    M, I = dh.shape
    assert ab.shape == (M, 2 * I)
    dab = np.empty((M, 2 * I), np.uint16)
    lib().orc_swiglu_bwd_bf16(M, I, _p(dh), _p(ab), _p(dab))
    return dab


def fp8_wgrad(Aq, As, Bq, Bs):
    """bf16(A^T B) over the M rows, both in 128x1 row-direction tiles (codes
    [M, F], scales [ceil(M/128), F])."""
    Aq, As = _c(Aq, np.uint8), _c(As, np.float32)
    Bq, Bs = _c(Bq, np.uint8), _c(Bs, np.float32)
    M, FA = Aq.shape
    FB = Bq.shape[1]
    nb = (M + 127) // 128
    assert Bq.shape[0] == M and As.shape == (nb, FA) and Bs.shape == (nb, FB)
    out = np.empty((FA, FB), np.uint16)
    lib().orc_fp8_wgrad(M, FA, FB, _p(Aq), _p(As), _p(Bq), _p(Bs), _p(out))
    return out


def route_backward(scores, idx, dgate):
    """dz[t,j]: gradient of the chosen logits from the gate gradient."""
    scores = _c(scores, np.float32)
    idx = _c(idx, np.int32)
    dgate = _c(dgate, np.float32)
    T, N = scores.shape
    k = idx.shape[1]
    dz = np.empty((T, k), np.float32)
    lib().orc_route_backward(T, N, k, _p(scores), _p(idx), _p(dgate), _p(dz))
    return dz


def centroid_grad(x, idx, dz, N):
    x = np.ascontiguousarray(x)
    idx = _c(idx, np.int32)
    dz = _c(dz, np.float32)
    T, d = x.shape
    k = idx.shape[1]
    dE = np.empty((N, d), np.float32)
    lib().orc_centroid_grad(T, d, N, k, dtype_code(x), _p(x), _p(idx), _p(dz), _p(dE))
    return dE


def input_grad(dout, dx_shared, dx_perm, dst_row, dz, idx, centroids):
    """dx = dout (residual; None = no residual) + dx_shared (None = no shared
    expert) + the routed rows' gradients + the logits' gradients."""
    dx_perm = np.ascontiguousarray(dx_perm)
    dt = dtype_code(dx_perm)
    dst = _c(dst_row, np.int32)
    dz = _c(dz, np.float32)
    idx = _c(idx, np.int32)
    E = _c(centroids, np.float32)
    T, k = dst.shape
    d = dx_perm.shape[1]
    if dout is not None:
        dout = _c(dout, dx_perm.dtype)
    if dx_shared is not None:
        dx_shared = _c(dx_shared, dx_perm.dtype)
    dx = np.empty((T, d), dx_perm.dtype)
    lib().orc_input_grad(T, d, k, dt, _p(dout), _p(dx_shared), _p(dx_perm), _p(dst), _p(dz),
                         _p(idx), _p(E), _p(dx))
    return dx


def layer_backward(inp, cfg, fwd, dout, residual=True):
    """Gradients of the layer for the upstream gradient ``dout`` [T,d], given
    the inputs ``inp`` and the forward's results ``fwd`` (from layer_forward).
    bf16 / fp32 layers differentiate the stored-precision experts; FP8 layers
    run every expert GEMM of the backward in E4M3 (swiglu_ffn_backward_fp8).
    Returns dx, dcentroids, dw13 [N,2I,d], dw2 [N,d,I], dws13, dws2 and the
    intermediates dy_perm, dgate, dz, dx_perm, dx_shared."""
    fp8 = cfg.get("fp8", False)
    N = cfg["N"]
    x = inp["x"]
    T, d = x.shape
    dout = _c(dout, x.dtype)
    offsets = fwd["offsets"]
    dy_perm, dgate = combine_backward(dout, fwd["y_perm"], fwd["gate"], fwd["dst_row"])
    x_perm = fwd["x_perm"] if not fp8 else gather_rows(x, fwd["src_token"])
    dx_perm = np.empty_like(x_perm)
    dw13 = np.empty_like(inp["w13"])
    dw2 = np.empty_like(inp["w2"])
    if fp8:
        w13q, w13s = quant_weight_fp8(inp["w13"])
        w2q, w2s = quant_weight_fp8(inp["w2"])
    for e in range(N):
        a, b = offsets[e], offsets[e + 1]
        if fp8:
            dA, dw13[e], dw2[e] = swiglu_ffn_backward_fp8(
                fwd["x_q_perm"][a:b], fwd["x_s_perm"][a:b], x_perm[a:b], w13q[e], w13s[e],
                w2q[e], w2s[e], dy_perm[a:b])
        else:
            dA, dw13[e], dw2[e] = swiglu_ffn_backward(x_perm[a:b], inp["w13"][e], inp["w2"][e],
                                                      dy_perm[a:b])
        dx_perm[a:b] = dA
    has_shared = inp.get("ws13") is not None and fwd.get("y_shared") is not None
    dx_shared = dws13 = dws2 = None
    if has_shared and fp8:
        ws13q, ws13s = quant_weight_fp8(inp["ws13"])
        ws2q, ws2s = quant_weight_fp8(inp["ws2"])
        dx_shared, dws13, dws2 = swiglu_ffn_backward_fp8(fwd["x_q"], fwd["x_s"], x, ws13q, ws13s,
                                                         ws2q, ws2s, dout)
    elif has_shared:
        dx_shared, dws13, dws2 = swiglu_ffn_backward(x, inp["ws13"], inp["ws2"], dout)
    dz = route_backward(fwd["scores"], fwd["idx"], dgate)
    dE = centroid_grad(x, fwd["idx"], dz, N)
    dx = input_grad(dout if residual else None, dx_shared, dx_perm, fwd["dst_row"], dz,
                    fwd["idx"], inp["centroids"])
    return dict(dx=dx, dcentroids=dE, dw13=dw13, dw2=dw2, dws13=dws13, dws2=dws2,
                dy_perm=dy_perm, dgate=dgate, dz=dz, dx_perm=dx_perm, dx_shared=dx_shared)
