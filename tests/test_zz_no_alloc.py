"""moe_dispatch_layout_noalloc (scratch in the library's static per-GPU array) against
moe_dispatch_layout (caller workspace): the same six outputs, bit for bit, on two calls in a row,
the second with a smaller input, through the C ABI. Integer outputs, so the bar is bit-exact."""
import numpy as np
import pytest
import torch

import combine_experts_amd as M
import oracle as O
import workloads as W
from tests import _parity as P

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")

OUTS = ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets", "pair_to_row", "row_to_pair")


def _both(cfg):
    inp = W.make_inputs(cfg, "cuda")
    d = M.dims_from_config(cfg)
    buf = M.MoELayerBuffers(d, device="cuda")
    M.moe_route(d, inp["x"], inp["w_gate"], inp["bias"], buf.topk_idx, buf.topk_gate)
    M.moe_dispatch_layout(d, buf.topk_idx, *(getattr(buf, n) for n in OUTS), buf.layout_ws)
    # the outputs of the allocation-free call start from a fill the layout must overwrite
    got = {n: torch.full_like(getattr(buf, n), -7) for n in OUTS}
    M.moe_dispatch_layout_noalloc(d, buf.topk_idx, *(got[n] for n in OUTS))
    torch.cuda.synchronize()
    return buf, got


@needs_gpu
def test_noalloc_layout_equals_the_workspace_layout_twice():
    # first the DeepSeek-V3-shaped routing at full size (256 chunks x 256 experts = 256 KiB of the
    # 1 MiB array), then a smaller problem with a capacity cut and fewer experts: the second call sees
    # the first call's histograms still in the array and must not depend on them
    big = W.get_config("dsv3", D=512, F=64)
    small = W.MoEConfig(name="small_cap", T=1000, D=128, E=6, top_k=2, F=64, ep_size=2, capacity_factor=0.8,
                        seed=71)
    for cfg in (big, small):
        print(f"[noalloc] {cfg.name} T={cfg.T} E={cfg.E} k={cfg.top_k}", flush=True)
        buf, got = _both(cfg)
        for n in OUTS:
            assert torch.equal(got[n], getattr(buf, n)), f"{cfg.name}: {n} differs"
        # and the oracle's layout of the same selection
        lay = O.dispatch_layout(P.i64(buf.topk_idx).reshape(cfg.T, cfg.top_k), cfg.E, cfg.ep_size,
                                O.capacity(cfg.capacity_factor, cfg.T, cfg.top_k, cfg.E))
        assert np.array_equal(P.i64(got["pair_to_row"]), lay["pair_to_row"])
        assert np.array_equal(P.i64(got["row_to_pair"]), lay["row_to_pair"])
        assert np.array_equal(P.i64(got["expert_offsets"]), lay["expert_offsets"])


@needs_gpu
def test_noalloc_layout_rejects_problems_beyond_its_array():
    # ceil(T*k/512) * E * 4 bytes must fit 1 MiB: 131072 pairs over 2048 experts need 2 MiB
    d = M.make_dims(16384, 64, 1024, 8, 64, ep_size=8)
    P_ = d.T * d.top_k
    idx = torch.zeros(P_, dtype=torch.int32, device="cuda")
    outs = [torch.empty(n, dtype=torch.int32, device="cuda") for n in (1024, 1025, 8, 9, P_, P_)]
    M.moe_dispatch_layout_noalloc(d, idx, *outs)          # exactly 1 MiB: accepted
    d2 = M.make_dims(16384 + 64, 64, 1024, 8, 64, ep_size=8)
    idx2 = torch.zeros(d2.T * 8, dtype=torch.int32, device="cuda")
    outs2 = [torch.empty(n, dtype=torch.int32, device="cuda") for n in (1024, 1025, 8, 9, d2.T * 8, d2.T * 8)]
    with pytest.raises(M.MoEError) as ei:
        M.moe_dispatch_layout_noalloc(d2, idx2, *outs2)   # one chunk more: refused, nothing enqueued
    assert ei.value.status == M.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert outs[0].sum().item() == P_                      # the accepted call ran: every pair on expert 0
