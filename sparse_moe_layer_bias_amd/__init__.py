"""Python binding of libmoe (include/moe.h): argument marshalling only.

Every step of the layer runs in the HIP kernels of ``libmoe.so``; this module
turns torch tensors into device pointers and the current HIP stream into a
``hipStream_t``, and raises ``MoeError`` on a non-zero status.  PyTorch is used
for device memory and streams only.  There is no fallback: if ``libmoe.so`` is
missing, importing the functions fails loudly.

The functions carry the C names: moe_route, moe_permute, moe_expert_ffn,
moe_combine, moe_bias_update, moe_seq_balance_loss, moe_quantize_weights_fp8,
the backward calls of
include/moe_backward.h (moe_expert_ffn_train, moe_combine_backward,
moe_expert_ffn_backward, moe_expert_ffn_train_fp8, moe_expert_ffn_backward_fp8,
moe_route_backward, moe_input_grad), the FFN inspection calls of
include/moe_inspect.h, plus the workspace size queries.
``MoeLayer`` (in layer.py) strings them together for one step.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2


class MoeError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("libmoe error %d: %s" % (code, msg))
        self.code = code


class MoeCfg(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("hidden", ctypes.c_int64),
                ("n_experts", ctypes.c_int64), ("top_k", ctypes.c_int64),
                ("n_group", ctypes.c_int64), ("topk_group", ctypes.c_int64),
                ("inter", ctypes.c_int64), ("inter_shared", ctypes.c_int64),
                ("act_dtype", ctypes.c_int32), ("gemm_dtype", ctypes.c_int32)]


def make_cfg(T, d, N, k, G=1, TG=1, I=0, Is=0, dtype="bf16", fp8=False):
    act = MOE_BF16 if dtype == "bf16" else MOE_F32
    return MoeCfg(T, d, N, k, G, TG, I, Is, act, MOE_FP8_E4M3 if fp8 else act)


def cfg_from_dict(c, T=None):
    return make_cfg(c["T"] if T is None else T, c["d"], c["N"], c["k"], c["G"], c["TG"],
                    c["I"], c["Is"], c["dtype"], c.get("fp8", False))


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libmoe.so is not built (run `python -m sparse_moe_layer_bias_amd.build`"
                              " or __graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32, SZ, F = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t,
                              ctypes.c_float)
        C = ctypes.POINTER(MoeCfg)
        sigs = {
            "moe_route_workspace_size": ([C], SZ),
            "moe_route": ([C, P, P, P, P, P, P, P, P, SZ, P], ctypes.c_int),
            "moe_permute_workspace_size": ([C], SZ),
            "moe_permute": ([C, P, P, P, P, P, P, P, P, P, P, SZ, P], ctypes.c_int),
            "moe_expert_ffn_workspace_size": ([C], SZ),
            "moe_expert_ffn": ([C] + [P] * 15 + [P, SZ, P], ctypes.c_int),
            "moe_expert_ffn_gather": ([C] + [P] * 14 + [P, SZ, P], ctypes.c_int),
            "moe_combine": ([C, P, P, P, P, P, P, P], ctypes.c_int),
            "moe_packed_weights_size": ([C, ctypes.c_int], SZ),
            "moe_pack_weights": ([C, ctypes.c_int, P, P, P], ctypes.c_int),
            "moe_bias_update": ([I64, I64, P, F, P, P], ctypes.c_int),
            "moe_seq_balance_loss_workspace_size": ([C, I64], SZ),
            "moe_seq_balance_loss": ([C, I64, F, P, P, P, P, SZ, P], ctypes.c_int),
            "moe_quantize_weights_fp8": ([I64, I64, I64, P, P, P, P], ctypes.c_int),
            "moe_combine_backward": ([C, P, P, P, P, P, P, P], ctypes.c_int),
            "moe_expert_ffn_backward_workspace_size": ([C], SZ),
            "moe_expert_ffn_backward": ([C] + [P] * 18 + [SZ, P, SZ, P], ctypes.c_int),
            "moe_expert_ffn_backward_fp8_workspace_size": ([C], SZ),
            "moe_expert_ffn_backward_fp8": ([C] + [P] * 26 + [SZ, P, SZ, P], ctypes.c_int),
            "moe_expert_ffn_train_fp8": ([C] + [P] * 16 + [SZ, P, SZ, P], ctypes.c_int),
            "moe_expert_ffn_saved_size": ([C], SZ),
            "moe_expert_ffn_train": ([C] + [P] * 10 + [SZ, P, SZ, P], ctypes.c_int),
            "moe_route_backward_workspace_size": ([C], SZ),
            "moe_route_backward": ([C] + [P] * 10 + [SZ, P], ctypes.c_int),
            "moe_input_grad": ([C] + [P] * 8 + [P], ctypes.c_int),
            "moe_expert_ffn_h_offsets": ([C, ctypes.POINTER(SZ)], ctypes.c_int),
            "moe_expert_ffn_inspect": ([C] + [P] * 17 + [P, SZ, P], ctypes.c_int),
            "moe_inspect_e4m3": ([P, I64, F, P, P, P], ctypes.c_int),
            "moe_expert_ffn_backward_fp8_offsets": ([C, ctypes.POINTER(SZ)], ctypes.c_int),
            "moe_expert_ffn_saved_offsets": ([C, ctypes.POINTER(SZ)], ctypes.c_int),
            "moe_permute_noalloc_max_bytes": ([], SZ),
            "moe_permute_noalloc": ([C, P, P, P, P, P, P, P, P, P, P], ctypes.c_int),
            "moe_last_error": ([], ctypes.c_char_p),
            "moe_abi_version": ([], ctypes.c_int),
        }
        for name, (args, res) in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(rc):
    if rc != MOE_OK:
        raise MoeError(rc, lib().moe_last_error().decode())


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


# ------------------------------------------------------------------ C calls

def moe_route_workspace_size(cfg):
    return lib().moe_route_workspace_size(ctypes.byref(cfg))


def moe_route(cfg, x, centroids, bias, scores, idx, gate, counts, workspace=None, stream=None):
    _check(lib().moe_route(ctypes.byref(cfg), _p(x), _p(centroids), _p(bias), _p(scores), _p(idx),
                           _p(gate), _p(counts), _p(workspace), _nbytes(workspace),
                           _stream(stream)))


def moe_permute_workspace_size(cfg):
    return lib().moe_permute_workspace_size(ctypes.byref(cfg))


def moe_permute(cfg, x, idx, offsets, src_token, dst_row, x_perm, x_perm_scale=None, x_q=None,
                x_s=None, workspace=None, stream=None):
    _check(lib().moe_permute(ctypes.byref(cfg), _p(x), _p(idx), _p(offsets), _p(src_token),
                             _p(dst_row), _p(x_perm), _p(x_perm_scale), _p(x_q), _p(x_s),
                             _p(workspace), _nbytes(workspace), _stream(stream)))


def moe_permute_noalloc_max_bytes():
    return lib().moe_permute_noalloc_max_bytes()


def moe_permute_noalloc(cfg, x, idx, offsets, src_token, dst_row, x_perm, x_perm_scale=None,
                        x_q=None, x_s=None, stream=None):
    _check(lib().moe_permute_noalloc(ctypes.byref(cfg), _p(x), _p(idx), _p(offsets),
                                     _p(src_token), _p(dst_row), _p(x_perm), _p(x_perm_scale),
                                     _p(x_q), _p(x_s), _stream(stream)))


def moe_expert_ffn_workspace_size(cfg):
    return lib().moe_expert_ffn_workspace_size(ctypes.byref(cfg))


def moe_expert_ffn(cfg, x_perm, x_perm_scale, offsets, w13, w13_scale, w2, w2_scale, y_perm,
                   x_sh, x_sh_scale, ws13, ws13_scale, ws2, ws2_scale, y_shared,
                   workspace=None, stream=None):
    _check(lib().moe_expert_ffn(ctypes.byref(cfg), _p(x_perm), _p(x_perm_scale), _p(offsets),
                                _p(w13), _p(w13_scale), _p(w2), _p(w2_scale), _p(y_perm),
                                _p(x_sh), _p(x_sh_scale), _p(ws13), _p(ws13_scale), _p(ws2),
                                _p(ws2_scale), _p(y_shared), _p(workspace), _nbytes(workspace),
                                _stream(stream)))


def moe_expert_ffn_gather(cfg, x, x_scale, src_token, offsets, w13, w13_scale, w2, w2_scale,
                          y_perm, ws13, ws13_scale, ws2, ws2_scale, y_shared, workspace=None,
                          stream=None):
    _check(lib().moe_expert_ffn_gather(ctypes.byref(cfg), _p(x), _p(x_scale), _p(src_token),
                                       _p(offsets), _p(w13), _p(w13_scale), _p(w2),
                                       _p(w2_scale), _p(y_perm), _p(ws13), _p(ws13_scale),
                                       _p(ws2), _p(ws2_scale), _p(y_shared), _p(workspace),
                                       _nbytes(workspace), _stream(stream)))


def moe_expert_ffn_h_offsets(cfg):
    """include/moe_inspect.h: byte offsets of h (routed, shared) and of its FP8
    tile scales (routed, shared; None for other layers) in the FFN workspace."""
    off = (ctypes.c_size_t * 4)()
    _check(lib().moe_expert_ffn_h_offsets(ctypes.byref(cfg), off))
    none = ctypes.c_size_t(-1).value
    return [None if v == none else int(v) for v in off]


def moe_expert_ffn_inspect(cfg, x_perm, x_perm_scale, offsets, w13, w13_scale, w2, w2_scale,
                           y_perm, x_sh, x_sh_scale, ws13, ws13_scale, ws2, ws2_scale, y_shared,
                           h_f32, h_f32_shared, workspace=None, stream=None):
    _check(lib().moe_expert_ffn_inspect(
        ctypes.byref(cfg), _p(x_perm), _p(x_perm_scale), _p(offsets), _p(w13), _p(w13_scale),
        _p(w2), _p(w2_scale), _p(y_perm), _p(x_sh), _p(x_sh_scale), _p(ws13), _p(ws13_scale),
        _p(ws2), _p(ws2_scale), _p(y_shared), _p(h_f32), _p(h_f32_shared), _p(workspace),
        _nbytes(workspace), _stream(stream)))


BWD8_NAMES = ("dy_q", "dy_s", "dy_q_sh", "dy_s_sh", "dh", "dh_sh", "dab", "dab_sh", "dab_q",
              "dab_s", "dab_q_sh", "dab_s_sh", "col_dy", "col_dy_s", "col_h", "col_h_s",
              "col_dab", "col_dab_s", "col_x", "col_x_s", "poff", "ab", "h", "ab_sh", "h_sh")


def moe_expert_ffn_backward_fp8_offsets(cfg):
    """include/moe_inspect.h: byte offsets of the FP8 backward's intermediates
    in its workspace, as a dict keyed by BWD8_NAMES."""
    off = (ctypes.c_size_t * len(BWD8_NAMES))()
    _check(lib().moe_expert_ffn_backward_fp8_offsets(ctypes.byref(cfg), off))
    return {n: int(v) for n, v in zip(BWD8_NAMES, off)}


def moe_expert_ffn_saved_offsets(cfg):
    off = (ctypes.c_size_t * 4)()
    _check(lib().moe_expert_ffn_saved_offsets(ctypes.byref(cfg), off))
    return dict(zip(("ab", "h", "ab_sh", "h_sh"), (int(v) for v in off)))


def moe_inspect_e4m3(v, scale, codes4, codes1, stream=None):
    _check(lib().moe_inspect_e4m3(_p(v), int(v.numel()), ctypes.c_float(float(scale)),
                                  _p(codes4), _p(codes1), _stream(stream)))


def moe_packed_weights_size(cfg, which):
    return lib().moe_packed_weights_size(ctypes.byref(cfg), int(which))


def moe_pack_weights(cfg, which, w, w_packed, stream=None):
    _check(lib().moe_pack_weights(ctypes.byref(cfg), int(which), _p(w), _p(w_packed),
                                  _stream(stream)))


def moe_combine(cfg, x_residual, y_shared, y_perm, gate, dst_row, out, stream=None):
    _check(lib().moe_combine(ctypes.byref(cfg), _p(x_residual), _p(y_shared), _p(y_perm),
                             _p(gate), _p(dst_row), _p(out), _stream(stream)))


def moe_bias_update(n_experts, tokens_times_k, counts, gamma, bias, stream=None):
    _check(lib().moe_bias_update(int(n_experts), int(tokens_times_k), _p(counts),
                                 ctypes.c_float(float(gamma)), _p(bias), _stream(stream)))


def moe_seq_balance_loss_workspace_size(cfg, seq_len):
    return int(lib().moe_seq_balance_loss_workspace_size(ctypes.byref(cfg), int(seq_len)))


def moe_seq_balance_loss(cfg, seq_len, alpha, scores, idx, loss, workspace=None, stream=None):
    _check(lib().moe_seq_balance_loss(ctypes.byref(cfg), int(seq_len), ctypes.c_float(float(alpha)),
                                      _p(scores), _p(idx), _p(loss), _p(workspace),
                                      _nbytes(workspace), _stream(stream)))


def moe_quantize_weights_fp8(n_mats, rows, cols, w_bf16, w_q, w_scale, stream=None):
    _check(lib().moe_quantize_weights_fp8(int(n_mats), int(rows), int(cols), _p(w_bf16), _p(w_q),
                                          _p(w_scale), _stream(stream)))


# ------------------------------------------------------------------ backward

def moe_combine_backward(cfg, dout, y_perm, gate, dst_row, dy_perm, dgate, stream=None):
    _check(lib().moe_combine_backward(ctypes.byref(cfg), _p(dout), _p(y_perm), _p(gate),
                                      _p(dst_row), _p(dy_perm), _p(dgate), _stream(stream)))


def moe_expert_ffn_backward_workspace_size(cfg):
    return lib().moe_expert_ffn_backward_workspace_size(ctypes.byref(cfg))


def moe_expert_ffn_saved_size(cfg):
    return lib().moe_expert_ffn_saved_size(ctypes.byref(cfg))


def moe_expert_ffn_train(cfg, x_perm, offsets, w13, w2, y_perm, x_sh, ws13, ws2, y_shared, saved,
                         workspace, stream=None):
    _check(lib().moe_expert_ffn_train(ctypes.byref(cfg), _p(x_perm), _p(offsets), _p(w13),
                                      _p(w2), _p(y_perm), _p(x_sh), _p(ws13), _p(ws2),
                                      _p(y_shared), _p(saved), _nbytes(saved), _p(workspace),
                                      _nbytes(workspace), _stream(stream)))


def moe_expert_ffn_backward(cfg, x_perm, offsets, w13, w13t, w2t, dy_perm, x_sh, ws13, ws13t,
                            ws2t, dy_shared, dx_perm, dx_shared, dw13, dw2, dws13, dws2, saved,
                            workspace, stream=None):
    _check(lib().moe_expert_ffn_backward(
        ctypes.byref(cfg), _p(x_perm), _p(offsets), _p(w13), _p(w13t), _p(w2t), _p(dy_perm),
        _p(x_sh), _p(ws13), _p(ws13t), _p(ws2t), _p(dy_shared), _p(dx_perm), _p(dx_shared),
        _p(dw13), _p(dw2), _p(dws13), _p(dws2), _p(saved), _nbytes(saved), _p(workspace),
        _nbytes(workspace), _stream(stream)))


def moe_expert_ffn_backward_fp8_workspace_size(cfg):
    return lib().moe_expert_ffn_backward_fp8_workspace_size(ctypes.byref(cfg))


def moe_expert_ffn_backward_fp8(cfg, x, src_token, offsets, x_perm, x_perm_scale, x_q, x_scale,
                                w13, w13t, w13_scale, w2t, w2_scale, ws13, ws13t, ws13_scale,
                                ws2t, ws2_scale, dy_perm, dy_shared, dx_perm, dx_shared, dw13,
                                dw2, dws13, dws2, saved, workspace, stream=None):
    _check(lib().moe_expert_ffn_backward_fp8(
        ctypes.byref(cfg), _p(x), _p(src_token), _p(offsets), _p(x_perm), _p(x_perm_scale),
        _p(x_q), _p(x_scale), _p(w13), _p(w13t), _p(w13_scale), _p(w2t), _p(w2_scale), _p(ws13),
        _p(ws13t), _p(ws13_scale), _p(ws2t), _p(ws2_scale), _p(dy_perm), _p(dy_shared),
        _p(dx_perm), _p(dx_shared), _p(dw13), _p(dw2), _p(dws13), _p(dws2), _p(saved),
        _nbytes(saved), _p(workspace), _nbytes(workspace), _stream(stream)))


def moe_expert_ffn_train_fp8(cfg, x_perm, x_perm_scale, offsets, w13, w13_scale, w2, w2_scale,
                             y_perm, x_sh, x_sh_scale, ws13, ws13_scale, ws2, ws2_scale,
                             y_shared, saved, workspace, stream=None):
    _check(lib().moe_expert_ffn_train_fp8(
        ctypes.byref(cfg), _p(x_perm), _p(x_perm_scale), _p(offsets), _p(w13), _p(w13_scale),
        _p(w2), _p(w2_scale), _p(y_perm), _p(x_sh), _p(x_sh_scale), _p(ws13), _p(ws13_scale),
        _p(ws2), _p(ws2_scale), _p(y_shared), _p(saved), _nbytes(saved), _p(workspace),
        _nbytes(workspace), _stream(stream)))


def moe_route_backward_workspace_size(cfg):
    return lib().moe_route_backward_workspace_size(ctypes.byref(cfg))


def moe_route_backward(cfg, x, scores, idx, dgate, offsets, src_token, dst_row, dz, dcentroids,
                       workspace, stream=None):
    _check(lib().moe_route_backward(ctypes.byref(cfg), _p(x), _p(scores), _p(idx), _p(dgate),
                                    _p(offsets), _p(src_token), _p(dst_row), _p(dz),
                                    _p(dcentroids), _p(workspace), _nbytes(workspace),
                                    _stream(stream)))


def moe_input_grad(cfg, dout, dx_shared, dx_perm, dst_row, dz, idx, centroids, dx, stream=None):
    _check(lib().moe_input_grad(ctypes.byref(cfg), _p(dout), _p(dx_shared), _p(dx_perm),
                                _p(dst_row), _p(dz), _p(idx), _p(centroids), _p(dx),
                                _stream(stream)))


def moe_abi_version():
    return lib().moe_abi_version()
