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
    def __init__(self, d: L.moe_dims, device="cuda", logits: bool = False):
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
        self.layout_ws = torch.empty(max(1, L.moe_workspace_size(d, L.MOE_STAGE_LAYOUT)), dtype=torch.uint8,
                                     device=device)
        self.x_perm = torch.empty((P, d.D), dtype=dt, device=device)
        self.h = torch.empty((P, d.F), dtype=dt, device=device)
        self.y_perm = torch.empty((P, d.D), dtype=dt, device=device)
        self.y = torch.empty((d.T, d.D), dtype=dt, device=device)

    def as_dict(self) -> Dict[str, Optional[torch.Tensor]]:
        return {k: v for k, v in self.__dict__.items() if isinstance(v, torch.Tensor) or v is None}


def forward(buf: MoELayerBuffers, x, w_gate, bias, w1, w3, w2, stream=None) -> torch.Tensor:
    """route -> dispatch layout -> permute -> expert FFN (up, down) -> unpermute + combine."""
    d = buf.d
    L.moe_route(d, x, w_gate, bias, buf.topk_idx, buf.topk_gate, buf.logits, stream)
    L.moe_dispatch_layout(d, buf.topk_idx, buf.expert_counts, buf.expert_offsets, buf.rank_counts,
                          buf.rank_offsets, buf.pair_to_row, buf.row_to_pair, buf.layout_ws, stream)
    L.moe_permute(d, x, buf.pair_to_row, buf.x_perm, stream)
    L.moe_expert_ffn_up(d, buf.x_perm, buf.expert_offsets, w1, w3, buf.h, stream)
    L.moe_expert_ffn_down(d, buf.h, buf.expert_offsets, w2, buf.y_perm, stream)
    L.moe_unpermute_combine(d, buf.y_perm, buf.pair_to_row, buf.topk_gate, buf.y, stream)
    return buf.y
