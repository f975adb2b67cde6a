"""Buffers and call order of one MoE layer forward on one GPU.

``MoELayerBuffers`` allocates (with torch, once) every buffer the five entry points write, sized
for the worst case of T*top_k rows; ``forward`` enqueues the five calls on one stream with no
host synchronisation. Nothing here computes: all arithmetic runs in libmoe's kernels.
"""
from __future__ import annotations

from typing import Dict, Optional

import torch

from . import _lib as L


class MoELayerBuffers:
    def __init__(self, d: L.moe_dims, device="cuda", logits: bool = False, x_perm: bool = True):
        """x_perm=False: no permuted copy of x; the forward's up-projection gathers its rows from x
        (``moe_expert_ffn_up_gather``; in training ``moe_expert_ffn_up_train_gather``, and the backward
        gathers the same rows into its transposed operand)."""
        self.d = d
        dt = torch.bfloat16 if d.dtype == L.MOE_BF16 else torch.float32
        P = d.T * d.top_k
        i32 = dict(dtype=torch.int32, device=device)
        self.topk_idx = torch.empty(P, **i32)
        self.topk_gate = torch.empty(P, dtype=torch.float32, device=device)
        self.logits = torch.empty(d.T * d.E, dtype=torch.float32, device=device) if logits else None
        self.expert_counts = torch.empty(d.E, **i32)
        self.expert_offsets = torch.empty(d.E + 1, **i32)
        self.rank_counts = torch.empty(d.ep_size, **i32)
        self.rank_offsets = torch.empty(d.ep_size + 1, **i32)
        self.pair_to_row = torch.empty(P, **i32)
        self.row_to_pair = torch.empty(P, **i32)
        ws = (L.moe_workspace_size(d, L.MOE_STAGE_LAYOUT) + 255) // 256 * 256
        self.layout_ws = torch.empty(max(256, ws), dtype=torch.uint8, device=device)
        self.x_perm = torch.empty((P, d.D), dtype=dt, device=device) if x_perm else None
        self.h = torch.empty((P, d.F), dtype=dt, device=device)
        self.y_perm = torch.empty((P, d.D), dtype=dt, device=device)
        self.y = torch.empty((d.T, d.D), dtype=dt, device=device)
        # split-K scratch of moe_expert_ffn_down_splitk, for dims whose down-projection has too few tiles
        n = L.moe_workspace_size(d, L.MOE_STAGE_FFN_DOWN)
        self.down_ws = torch.empty(n, dtype=torch.uint8, device=device) if n > 0 else None

    def as_dict(self) -> Dict[str, Optional[torch.Tensor]]:
        return {k: v for k, v in self.__dict__.items() if isinstance(v, torch.Tensor) or v is None}


def _ptr(t):
    return None if t is None else t.data_ptr()


def _layer_args(buf: MoELayerBuffers, x, w_gate, bias, w1, w3, w2, pre=None) -> L.moe_layer_args:
    a = L.moe_layer_args()
    a.x, a.w_gate, a.bias, a.w1, a.w3, a.w2, a.y = _ptr(x), _ptr(w_gate), _ptr(bias), _ptr(w1), _ptr(w3), _ptr(w2), \
        _ptr(buf.y)
    for n in ("topk_idx", "topk_gate", "pair_to_row", "row_to_pair", "x_perm", "h", "y_perm", "expert_counts",
              "expert_offsets", "rank_counts", "rank_offsets", "layout_ws", "logits"):
        setattr(a, n, _ptr(getattr(buf, n)))
    a.layout_ws_bytes = buf.layout_ws.numel()
    a.pre = _ptr(pre)
    if buf.down_ws is not None:
        a.down_ws, a.down_ws_bytes = buf.down_ws.data_ptr(), buf.down_ws.numel()
    return a


def forward(buf: MoELayerBuffers, x, w_gate, bias, w1, w3, w2, stream=None) -> torch.Tensor:
    """route -> dispatch layout -> permute -> expert FFN (up, down) -> unpermute + combine, as one call of
    the library's executor (one micro-batch, one stream); without buf.x_perm the permute happens inside
    the up-projection's row loads. Router logits land in buf.logits if it has them."""
    L.moe_layer_forward(buf.d, _layer_args(buf, x, w_gate, bias, w1, w3, w2), 1, stream)
    return buf.y


class LayerExecutor:
    """Buffers, streams and events for ``moe_layer_forward`` (micro-batches, optional side stream and
    shared expert). Allocates once with torch; every call only enqueues the library's kernels."""

    def __init__(self, d: L.moe_dims, n_chunks: int = 1, two_streams: bool = False, shared_F: int = 0,
                 device="cuda", gather: bool = False, split_k: bool = True):
        """gather=True: no x_perm buffer; each micro-batch's up-projection reads its rows from x.
        split_k=False: no split-K workspace, so the down-projection never splits and any number of
        micro-batches gives the whole batch's bits."""
        if d.T % n_chunks != 0:
            raise ValueError("T must split evenly into the micro-batches")
        self.d, self.n_chunks = d, n_chunks
        dt = torch.bfloat16 if d.dtype == L.MOE_BF16 else torch.float32
        P, E, ep = d.T * d.top_k, d.E, d.ep_size
        i32 = dict(dtype=torch.int32, device=device)
        self.topk_idx = torch.empty(P, **i32)
        self.topk_gate = torch.empty(P, dtype=torch.float32, device=device)
        self.pair_to_row = torch.empty(P, **i32)
        self.row_to_pair = torch.empty(P, **i32)
        self.x_perm = None if gather else torch.empty((P, d.D), dtype=dt, device=device)
        self.h = torch.empty((P, d.F), dtype=dt, device=device)
        self.y_perm = torch.empty((P, d.D), dtype=dt, device=device)
        self.y = torch.empty((d.T, d.D), dtype=dt, device=device)
        self.expert_counts = torch.empty((n_chunks, E), **i32)
        self.expert_offsets = torch.empty((n_chunks, E + 1), **i32)
        self.rank_counts = torch.empty((n_chunks, ep), **i32)
        self.rank_offsets = torch.empty((n_chunks, ep + 1), **i32)
        dc = L.moe_dims.from_buffer_copy(d)
        dc.T = d.T // n_chunks
        ws = (L.moe_workspace_size(dc, L.MOE_STAGE_LAYOUT) + 255) // 256 * 256
        self.layout_ws = torch.empty(max(1, ws * n_chunks), dtype=torch.uint8, device=device)
        # split-K scratch of the micro-batches' down-projections (they run one after another on one stream)
        n = L.moe_workspace_size(dc, L.MOE_STAGE_FFN_DOWN) if split_k else 0
        self.down_ws = torch.empty(n, dtype=torch.uint8, device=device) if n > 0 else None
        self.shared_F = shared_F
        if shared_F > 0:
            self.shared_h = torch.empty((d.T, shared_F), dtype=dt, device=device)
            self.shared_y = torch.empty((d.T, d.D), dtype=dt, device=device)
            self.shared_offsets = torch.tensor([0, d.T // n_chunks], **i32)
        self.side = torch.cuda.Stream(device=device) if two_streams else None
        self.events = [L.moe_event_create() for _ in range(2 * n_chunks)] if two_streams else None

    def __del__(self):
        for e in (self.events or []):
            try:
                L.moe_event_destroy(e)
            except Exception:
                pass
        self.events = None

    def forward(self, x, w_gate, bias, w1, w3, w2, shared=None, stream=None) -> torch.Tensor:
        """shared: (shared_w1, shared_w3, shared_w2) or None."""
        p = lambda t: None if t is None else t.data_ptr()
        a = L.moe_layer_args()
        a.x, a.w_gate, a.bias, a.w1, a.w3, a.w2, a.y = p(x), p(w_gate), p(bias), p(w1), p(w3), p(w2), p(self.y)
        for n in ("topk_idx", "topk_gate", "pair_to_row", "row_to_pair", "x_perm", "h", "y_perm", "expert_counts",
                  "expert_offsets", "rank_counts", "rank_offsets", "layout_ws"):
            setattr(a, n, p(getattr(self, n)))
        a.layout_ws_bytes = self.layout_ws.numel()
        if self.down_ws is not None:
            a.down_ws, a.down_ws_bytes = self.down_ws.data_ptr(), self.down_ws.numel()
        if shared is not None:
            if self.shared_F <= 0:
                raise ValueError("executor built without a shared expert")
            a.shared_w1, a.shared_w3, a.shared_w2 = p(shared[0]), p(shared[1]), p(shared[2])
            a.shared_F = self.shared_F
            a.shared_h, a.shared_y, a.shared_offsets = p(self.shared_h), p(self.shared_y), p(self.shared_offsets)
        L.moe_layer_forward(self.d, a, self.n_chunks, stream, self.side, self.events)
        return self.y


class GraphLayer:
    """The layer forward captured once in a HIP graph and replayed: one graph launch per step instead
    of the eight to ten kernel launches, which is most of the time of a small layer. Every replay
    reads the tensors given here (write new inputs into them in place) and writes ``self.buf.y``.
    The library allocates, synchronises and clears nothing inside the step, so the whole step
    captures; the first (eager) call, made before capture, also raises the router's LDS limit."""

    def __init__(self, d: L.moe_dims, x, w_gate, bias, w1, w3, w2, device="cuda", gather: bool = True):
        self.buf = MoELayerBuffers(d, device=device, x_perm=not gather)
        self.args = (x, w_gate, bias, w1, w3, w2)
        side = torch.cuda.Stream(device=device)
        side.wait_stream(torch.cuda.current_stream(device))
        with torch.cuda.stream(side):
            forward(self.buf, *self.args)
        torch.cuda.current_stream(device).wait_stream(side)
        torch.cuda.synchronize(device)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            forward(self.buf, *self.args)

    def replay(self) -> torch.Tensor:
        self.graph.replay()
        return self.buf.y


class BackwardBuffers:
    """Buffers of one training step's backward for dims d (bf16): saved pre-activations, the backward's
    activations, transposed wgrad operands and float32 gradients. transposed=True also keeps transposed
    copies of the weights (w13t, w2t) for the data-gradient GEMMs; by default they read the weights as
    stored."""

    def __init__(self, d: L.moe_dims, device="cuda", transposed: bool = False):
        self.d = d
        dt = torch.bfloat16
        P, E, D, F = d.T * d.top_k, d.E, d.D, d.F
        nm = 2 if d.act == L.MOE_ACT_SWIGLU else 1
        f32 = dict(dtype=torch.float32, device=device)
        self.pre = torch.empty((P, nm * F), dtype=dt, device=device)
        self.w13t = torch.empty((E, D, nm * F), dtype=dt, device=device) if transposed else None
        self.w2t = torch.empty((E, F, D), dtype=dt, device=device) if transposed else None
        self.dy_perm = torch.empty((P, D), dtype=dt, device=device)
        self.dgate = torch.empty(P, **f32)
        self.da = torch.empty((P, nm * F), dtype=dt, device=device)
        self.dx_perm = torch.empty((P, D), dtype=dt, device=device)
        self.dl = torch.empty((d.T, E), **f32)
        self.dw_gate = torch.empty((E, D), **f32)
        self.dbias = torch.empty(E, **f32)
        self.router_ws = torch.empty(max(1, L.moe_workspace_size(d, L.MOE_STAGE_ROUTER_BWD)), dtype=torch.uint8,
                                     device=device)
        self.dx = torch.empty((d.T, D), dtype=dt, device=device)
        ld = L.moe_wgrad_ld(d)
        self.koff = torch.empty(E + 1, dtype=torch.int32, device=device)
        self.dyp_t = torch.empty((D, ld), dtype=dt, device=device)
        self.h_t = torch.empty((F, ld), dtype=dt, device=device)
        self.da_t = torch.empty((nm * F, ld), dtype=dt, device=device)
        self.xp_t = torch.empty((D, ld), dtype=dt, device=device)
        self.dw1 = torch.empty((E, F, D), **f32)
        self.dw3 = torch.empty((E, F, D), **f32) if nm == 2 else None
        self.dw2 = torch.empty((E, D, F), **f32)


def forward_train(buf: MoELayerBuffers, bw: "BackwardBuffers", x, w_gate, bias, w1, w3, w2, stream=None):
    """The forward with what the backward needs saved: logits (buf must hold them) and pre-activations."""
    if buf.logits is None:
        raise ValueError("forward_train needs MoELayerBuffers(..., logits=True)")
    L.moe_layer_forward(buf.d, _layer_args(buf, x, w_gate, bias, w1, w3, w2, pre=bw.pre), 1, stream)
    return buf.y


def backward(buf: MoELayerBuffers, bw: "BackwardBuffers", x, w_gate, dy, stream=None, transpose_weights=None):
    """The backward as one call of the library's executor. ``transpose_weights``: the forward's (w1, w3,
    w2); the data-gradient GEMMs read them directly, or, with BackwardBuffers(transposed=True), they are
    transposed into bw.w13t / bw.w2t first (as after a weight update; None reuses the copies). Gradients
    land in bw.dx, bw.dw_gate, bw.dbias, bw.dw1, bw.dw3, bw.dw2."""
    a = L.moe_backward_args()
    a.x, a.w_gate, a.dy = _ptr(x), _ptr(w_gate), _ptr(dy)
    if bw.w13t is None and transpose_weights is None:
        raise ValueError("backward without transposed weight copies needs the weights (w1, w3, w2)")
    if transpose_weights is not None:
        a.w1, a.w3, a.w2 = (_ptr(t) for t in transpose_weights)
        a.refresh_weights = 1 if bw.w13t is not None else 0
    for n in ("logits", "topk_idx", "topk_gate", "expert_offsets", "pair_to_row", "row_to_pair", "x_perm", "h",
              "y_perm"):
        setattr(a, n, _ptr(getattr(buf, n)))
    for n in ("pre", "w13t", "w2t", "dy_perm", "dgate", "da", "dx_perm", "dl", "router_ws", "koff", "dx", "dw_gate",
              "dbias", "dw1", "dw3", "dw2"):
        setattr(a, n, _ptr(getattr(bw, n)))
    a.router_ws_bytes = bw.router_ws.numel()
    a.dy_perm_t, a.h_t, a.da_t, a.x_perm_t = _ptr(bw.dyp_t), _ptr(bw.h_t), _ptr(bw.da_t), _ptr(bw.xp_t)
    a.ld = bw.dyp_t.shape[1]
    L.moe_layer_backward(buf.d, a, stream)
    return bw.dx
