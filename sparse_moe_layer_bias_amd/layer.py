"""One DeepSeekMoE layer step through libmoe: buffers (torch device memory) and
the five calls in order on one stream.

    route -> permute -> expert_ffn (routed + shared) -> combine -> bias_update

and, for layers built with ``train=True``, the backward calls of
include/moe_backward.h:

    combine_backward -> expert_ffn_backward (FP8 layers: expert_ffn_backward_fp8)
        -> route_backward -> input_grad

(DeepSeek-V3 report reading guide, xyznot.com/de, "Methode" item 2: the layer
output h'_t, the biased Topk routing and the end-of-step bias rule.)
"""
import torch

from . import (MoeCfg, cfg_from_dict, moe_bias_update, moe_combine, moe_combine_backward,
               moe_expert_ffn, moe_expert_ffn_backward, moe_expert_ffn_backward_fp8,
               moe_expert_ffn_gather,
               moe_expert_ffn_backward_fp8_workspace_size, moe_expert_ffn_backward_workspace_size,
               moe_expert_ffn_train_fp8, moe_expert_ffn_h_offsets, moe_expert_ffn_inspect,
               moe_expert_ffn_saved_size, moe_expert_ffn_train,
               moe_expert_ffn_workspace_size, moe_input_grad, moe_pack_weights,
               moe_packed_weights_size, moe_permute, moe_permute_workspace_size,
               moe_quantize_weights_fp8, moe_route, moe_route_backward,
               moe_route_backward_workspace_size, moe_route_workspace_size,
               moe_seq_balance_loss, moe_seq_balance_loss_workspace_size)

GAMMA = 0.001  # end-of-step bias step (reading guide, "Methode" item 2)


# the gathered-rows expert GEMM addresses a row of x (bf16, or its FP8 codes)
# by a 32-bit byte offset
GATHER_MAX_X_BYTES = (1 << 32) - 1


def can_gather_rows(c, train):
    """Whether a layer of config dict c can run its expert GEMM on gathered
    token rows (moe_expert_ffn_gather): inference with bf16 activations and an
    x (bf16, or its FP8 codes) below 2^32 bytes."""
    x_bytes = c["T"] * c["d"] * (1 if c.get("fp8", False) else 2)
    return c["dtype"] == "bf16" and not train and x_bytes <= GATHER_MAX_X_BYTES


def pack_weights(cfg, which, w, stream=None):
    """The expert GEMM's streaming layout of one weight stack (moe_pack_weights)."""
    out = torch.empty((moe_packed_weights_size(cfg, which),), dtype=torch.uint8,
                      device=w.device)
    moe_pack_weights(cfg, which, w, out, stream)
    return out


def quantize_weights_fp8(w, stream=None):
    """128x128 block E4M3 codes and scales of a bf16 weight stack [..., rows, cols]."""
    rows, cols = w.shape[-2:]
    n = w.numel() // (rows * cols)
    q = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    s = torch.empty(w.shape[:-2] + (rows // 128, cols // 128), dtype=torch.float32,
                    device=w.device)
    moe_quantize_weights_fp8(n, rows, cols, w, q, s, stream)
    return q, s


class MoeLayer:
    """Holds the expert weights (and their FP8 form when the config asks for it)
    and every per-step buffer for a batch of T tokens.

    gather_rows (inference layers with bf16 activations, bf16 or FP8 GEMMs,
    whose x stays below 2^32 bytes; default on for them): the permutation
    writes only its indices (FP8: and the codes of x) and the expert GEMM
    reads the token rows through src_token (moe_expert_ffn_gather), so x_perm
    is not kept.  Larger batches use the permuted copy x_perm."""

    def __init__(self, cfg, w13, w2, ws13=None, ws2=None, T=None, device="cuda",
                 train=False, save_activations=True, gather_rows=None):
        self.c = dict(cfg)
        if T is not None:
            self.c["T"] = T
        c = self.c
        self.cfg: MoeCfg = cfg_from_dict(c)
        self.fp8 = bool(c.get("fp8", False))
        T, d, N, k = c["T"], c["d"], c["N"], c["k"]
        TK = T * k
        act = torch.bfloat16 if c["dtype"] == "bf16" else torch.float32
        dev = torch.device(device)
        has_shared = ws13 is not None and c["Is"] > 0
        if not has_shared:
            self.cfg.inter_shared = 0
        if self.fp8:
            # 128x128 block quantisation, then the GEMM's streaming order
            # (training: also the transposed packs of the same codes for the
            # backward's data-gradient GEMMs)
            q13, self.w13_s = quantize_weights_fp8(w13)
            q2, self.w2_s = quantize_weights_fp8(w2)
            self.w13 = pack_weights(self.cfg, 0, q13)
            self.w2 = pack_weights(self.cfg, 1, q2)
            self.w13t_fp8 = pack_weights(self.cfg, 4, q13) if train else None
            self.w2t_fp8 = pack_weights(self.cfg, 5, q2) if train else None
            del q13, q2
            self.ws13 = self.ws13_s = self.ws2 = self.ws2_s = None
            self.ws13t_fp8 = self.ws2t_fp8 = None
            if has_shared:
                qs13, self.ws13_s = quantize_weights_fp8(ws13)
                qs2, self.ws2_s = quantize_weights_fp8(ws2)
                self.ws13 = pack_weights(self.cfg, 2, qs13)
                self.ws2 = pack_weights(self.cfg, 3, qs2)
                if train:
                    self.ws13t_fp8 = pack_weights(self.cfg, 6, qs13)
                    self.ws2t_fp8 = pack_weights(self.cfg, 7, qs2)
        else:
            self.w13 = pack_weights(self.cfg, 0, w13)
            self.w2 = pack_weights(self.cfg, 1, w2)
            self.ws13 = pack_weights(self.cfg, 2, ws13) if has_shared else None
            self.ws2 = pack_weights(self.cfg, 3, ws2) if has_shared else None
            self.w13_s = self.w2_s = self.ws13_s = self.ws2_s = None
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        self.scores = torch.empty((T, N), **f32)
        self.idx = torch.empty((T, k), **i32)
        self.gate = torch.empty((T, k), **f32)
        self.counts = torch.empty((N,), **i32)
        self.offsets = torch.empty((N + 1,), **i32)
        self.src_token = torch.empty((TK,), **i32)
        self.dst_row = torch.empty((T, k), **i32)
        can_gather = can_gather_rows(c, train)
        self.gather_rows = can_gather if gather_rows is None else bool(gather_rows)
        if self.gather_rows and not can_gather:
            raise ValueError("gather_rows needs an inference layer with bf16 activations "
                             "and x below 2^32 bytes")
        if self.fp8:
            if self.gather_rows:
                self.x_perm = self.x_perm_s = None
            else:
                self.x_perm = torch.empty((TK, d), dtype=torch.uint8, device=dev)
                self.x_perm_s = torch.empty((TK, d // 128), **f32)
            self.x_q = torch.empty((T, d), dtype=torch.uint8, device=dev)
            self.x_s = torch.empty((T, d // 128), **f32)
        elif self.gather_rows:
            self.x_perm = self.x_perm_s = self.x_q = self.x_s = None
        else:
            self.x_perm = torch.empty((TK, d), dtype=act, device=dev)
            self.x_perm_s = self.x_q = self.x_s = None
        self.y_perm = torch.empty((TK, d), dtype=act, device=dev)
        self.y_shared = torch.empty((T, d), dtype=act, device=dev) if has_shared else None
        self.out = torch.empty((T, d), dtype=act, device=dev)
        ws = max(moe_route_workspace_size(self.cfg), moe_permute_workspace_size(self.cfg),
                 moe_expert_ffn_workspace_size(self.cfg), 256)
        self.workspace = torch.empty((ws,), dtype=torch.uint8, device=dev)
        # the backward's dgrad GEMMs stream the weights transposed
        self.train = bool(train)
        self.w_shapes = (tuple(w13.shape), tuple(w2.shape),
                         tuple(ws13.shape) if has_shared else None,
                         tuple(ws2.shape) if has_shared else None)
        self.w13t = self.w2t = self.ws13t = self.ws2t = None
        if self.train and self.fp8:
            self.w13t, self.w2t = self.w13t_fp8, self.w2t_fp8
            self.ws13t, self.ws2t = self.ws13t_fp8, self.ws2t_fp8
        elif self.train:
            self.w13t = pack_weights(self.cfg, 4, w13)
            self.w2t = pack_weights(self.cfg, 5, w2)
            if has_shared:
                self.ws13t = pack_weights(self.cfg, 6, ws13)
                self.ws2t = pack_weights(self.cfg, 7, ws2)
        self.grads = None
        # a training forward keeps a, b and h for the backward (else recomputed)
        self.saved = None
        self.graph = None  # capture_forward
        if self.train and save_activations:
            self.saved = torch.empty((moe_expert_ffn_saved_size(self.cfg),), dtype=torch.uint8,
                                     device=dev)

    # the five calls -------------------------------------------------------
    def route(self, x, centroids, bias, stream=None):
        moe_route(self.cfg, x, centroids, bias, self.scores, self.idx, self.gate, self.counts,
                  None, stream)

    def seq_balance_loss(self, seq_len, alpha=1e-4, stream=None):
        """The sequence-wise balance loss of this step's routing (moe_seq_balance_loss:
        one fp32 value per sequence of seq_len consecutive tokens), from the
        affinities and indices of the last route()."""
        T = self.c["T"]
        loss = torch.empty(T // seq_len if seq_len > 0 else 0, dtype=torch.float32,
                           device=self.scores.device)
        ws = torch.empty(max(moe_seq_balance_loss_workspace_size(self.cfg, seq_len), 16),
                         dtype=torch.uint8, device=self.scores.device)
        moe_seq_balance_loss(self.cfg, seq_len, alpha, self.scores, self.idx, loss, ws, stream)
        return loss

    def permute(self, x, stream=None):
        moe_permute(self.cfg, x, self.idx, self.offsets, self.src_token, self.dst_row,
                    self.x_perm, self.x_perm_s, self.x_q, self.x_s, self.workspace, stream)

    def expert_ffn(self, x, stream=None):
        if self.saved is not None and self.fp8:
            shared = self.y_shared is not None
            moe_expert_ffn_train_fp8(
                self.cfg, self.x_perm, self.x_perm_s, self.offsets, self.w13, self.w13_s, self.w2,
                self.w2_s, self.y_perm, self.x_q if shared else None,
                self.x_s if shared else None, self.ws13, self.ws13_s, self.ws2, self.ws2_s,
                self.y_shared, self.saved, self.workspace, stream)
            return
        if self.saved is not None:
            shared = self.y_shared is not None
            moe_expert_ffn_train(self.cfg, self.x_perm, self.offsets, self.w13, self.w2,
                                 self.y_perm, x if shared else None, self.ws13, self.ws2,
                                 self.y_shared, self.saved, self.workspace, stream)
            return
        if self.gather_rows:
            src = (self.x_q, self.x_s) if self.fp8 else (x, None)
            moe_expert_ffn_gather(self.cfg, src[0], src[1], self.src_token, self.offsets,
                                  self.w13, self.w13_s, self.w2, self.w2_s, self.y_perm,
                                  self.ws13, self.ws13_s, self.ws2, self.ws2_s, self.y_shared,
                                  self.workspace, stream)
            return
        shared_in = self.x_q if self.fp8 else x
        moe_expert_ffn(self.cfg, self.x_perm, self.x_perm_s, self.offsets, self.w13, self.w13_s,
                       self.w2, self.w2_s, self.y_perm, shared_in if self.y_shared is not None
                       else None, self.x_s if self.y_shared is not None else None, self.ws13,
                       self.ws13_s, self.ws2, self.ws2_s, self.y_shared, self.workspace, stream)

    def expert_ffn_inspect(self, stream=None):
        """FP8 layers: the expert FFN again through moe_expert_ffn_inspect (same
        results as expert_ffn) on this step's permuted rows.  Returns a dict:
        h_f32 / h_f32_shared, the gate/up epilogue's fp32 h before quantisation,
        and h_q / h_s / h_q_shared / h_s_shared, the E4M3 codes and 1x128 tile
        scales the down GEMM read (views into the workspace, valid until the
        next call that uses it)."""
        if not self.fp8:
            raise ValueError("expert_ffn_inspect covers FP8 layers")
        c = self.c
        T, k, I, Is = c["T"], c["k"], c["I"], self.cfg.inter_shared
        dev = self.out.device
        shared = self.y_shared is not None
        hf = torch.empty((T * k, I), dtype=torch.float32, device=dev)
        hfs = torch.empty((T, Is), dtype=torch.float32, device=dev) if shared else None
        moe_expert_ffn_inspect(self.cfg, self.x_perm, self.x_perm_s, self.offsets, self.w13,
                               self.w13_s, self.w2, self.w2_s, self.y_perm,
                               self.x_q if shared else None, self.x_s if shared else None,
                               self.ws13, self.ws13_s, self.ws2, self.ws2_s, self.y_shared, hf,
                               hfs, self.workspace, stream)
        off = moe_expert_ffn_h_offsets(self.cfg)
        ws = self.workspace

        def view(o, n, dtype, shape):
            b = ws[o:o + n * torch.tensor([], dtype=dtype).element_size()]
            return b.view(dtype).view(shape)

        out = dict(h_f32=hf, h_f32_shared=hfs,
                   h_q=view(off[0], T * k * I, torch.uint8, (T * k, I)),
                   h_s=view(off[2], T * k * (I // 128), torch.float32, (T * k, I // 128)))
        if shared:
            out.update(h_q_shared=view(off[1], T * Is, torch.uint8, (T, Is)),
                       h_s_shared=view(off[3], T * (Is // 128), torch.float32, (T, Is // 128)))
        return out

    def combine(self, x, residual=True, stream=None):
        moe_combine(self.cfg, x if residual else None, self.y_shared, self.y_perm, self.gate,
                    self.dst_row, self.out, stream)

    def bias_update(self, bias, stream=None):
        moe_bias_update(self.c["N"], self.c["T"] * self.c["k"], self.counts, GAMMA, bias, stream)

    def forward(self, x, centroids, bias, residual=True, update_bias=True, stream=None):
        """One step; returns ``self.out``.  ``bias`` is updated in place at the
        end when ``update_bias`` (the routing of this step used the old value)."""
        self.route(x, centroids, bias, stream)
        self.permute(x, stream)
        self.expert_ffn(x, stream)
        self.combine(x, residual, stream)
        if update_bias:
            self.bias_update(bias, stream)
        return self.out

    # HIP graph ----------------------------------------------------------------
    def capture_forward(self, x, centroids, bias, residual=True, update_bias=True):
        """Record one forward step -- the same five calls on the same buffers --
        into a HIP graph and keep it; ``replay()`` runs it.  Every replay reads
        x, centroids and bias from the tensors given here (write new values into
        them in place between replays) and leaves its result in ``self.out``;
        with ``update_bias`` each replay also updates ``bias`` in place.  None
        of the calls allocates, synchronises or copies through the host, so a
        whole step is one graph launch.  One untimed step (without the bias
        update) runs first on the capture stream."""
        s = torch.cuda.Stream()  # default priority
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.forward(x, centroids, bias, residual, update_bias=False)
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            self.forward(x, centroids, bias, residual, update_bias)
        torch.cuda.current_stream().wait_stream(s)
        self.graph = g
        return g

    def replay(self):
        """Run the captured forward step on the current stream."""
        if self.graph is None:
            raise RuntimeError("replay() needs capture_forward() first")
        self.graph.replay()
        return self.out

    # the backward ------------------------------------------------------------
    def _grad_buffers(self, centroids):
        c = self.c
        T, d, k = c["T"], c["d"], c["k"]
        dev = self.out.device
        act = self.out.dtype
        s13, s2, ss13, ss2 = self.w_shapes
        f32 = dict(dtype=torch.float32, device=dev)
        a = dict(dtype=act, device=dev)
        g = dict(dy_perm=torch.empty((T * k, d), **a),
                 dgate=torch.empty((T, k), **f32),
                 dx_perm=torch.empty((T * k, d), **a),
                 dx_shared=torch.empty((T, d), **a) if ss13 is not None else None,
                 dw13=torch.empty(s13, **a), dw2=torch.empty(s2, **a),
                 dws13=torch.empty(ss13, **a) if ss13 is not None else None,
                 dws2=torch.empty(ss2, **a) if ss2 is not None else None,
                 dz=torch.empty((T, k), **f32),
                 dcentroids=torch.empty_like(centroids),
                 dx=torch.empty((T, d), **a))
        ffn_ws = (moe_expert_ffn_backward_fp8_workspace_size(self.cfg) if self.fp8 else
                  moe_expert_ffn_backward_workspace_size(self.cfg))
        # separate workspaces: the expert backward's keeps its intermediates
        # (readable through moe_expert_ffn_backward_fp8_offsets) until the
        # next backward call
        g["workspace"] = torch.empty((max(ffn_ws, 256),), dtype=torch.uint8, device=dev)
        g["route_workspace"] = torch.empty((max(moe_route_backward_workspace_size(self.cfg), 256),),
                                           dtype=torch.uint8, device=dev)
        return g

    def expert_ffn_backward(self, dout, x, stream=None):
        """moe_expert_ffn_backward on the buffers of the last backward call
        (dy_perm from its combine backward)."""
        g = self.grads
        shared = self.ws13t is not None
        if self.fp8:
            moe_expert_ffn_backward_fp8(
                self.cfg, x, self.src_token, self.offsets, self.x_perm, self.x_perm_s,
                self.x_q if shared else None, self.x_s if shared else None, self.w13, self.w13t,
                self.w13_s, self.w2t, self.w2_s, self.ws13, self.ws13t, self.ws13_s, self.ws2t,
                self.ws2_s, g["dy_perm"], dout if shared else None, g["dx_perm"], g["dx_shared"],
                g["dw13"], g["dw2"], g["dws13"], g["dws2"], self.saved, g["workspace"], stream)
            return
        moe_expert_ffn_backward(self.cfg, self.x_perm, self.offsets, self.w13, self.w13t,
                                self.w2t, g["dy_perm"], x if shared else None, self.ws13,
                                self.ws13t, self.ws2t, dout if shared else None, g["dx_perm"],
                                g["dx_shared"], g["dw13"], g["dw2"], g["dws13"], g["dws2"],
                                self.saved, g["workspace"], stream)

    def backward(self, dout, x, centroids, residual=True, stream=None, events=None):
        """Gradients of the last forward step for the upstream gradient ``dout``
        [T, d]: returns a dict with dx, dcentroids, dw13, dw2, dws13, dws2 (plus
        the intermediates dy_perm, dgate, dx_perm, dx_shared, dz).  The buffers
        are reused across calls.  ``events``: 5 torch.cuda.Events recorded
        around the four calls (on the current stream)."""
        if not self.train:
            raise RuntimeError("the backward needs the transposed weight packs: build the "
                               "layer with train=True")
        if self.grads is None:
            self.grads = self._grad_buffers(centroids)
        g = self.grads
        mark = (lambda i: events[i].record()) if events is not None else (lambda i: None)
        mark(0)
        moe_combine_backward(self.cfg, dout, self.y_perm, self.gate, self.dst_row, g["dy_perm"],
                             g["dgate"], stream)
        mark(1)
        self.expert_ffn_backward(dout, x, stream)
        mark(2)
        moe_route_backward(self.cfg, x, self.scores, self.idx, g["dgate"], self.offsets,
                           self.src_token, self.dst_row, g["dz"], g["dcentroids"],
                           g["route_workspace"], stream)
        mark(3)
        moe_input_grad(self.cfg, dout if residual else None, g["dx_shared"], g["dx_perm"],
                       self.dst_row, g["dz"], self.idx, centroids, g["dx"], stream)
        mark(4)
        return g
