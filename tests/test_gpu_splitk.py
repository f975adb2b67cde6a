"""GPU parity of the split-K down-projection (moe_expert_ffn_down_splitk), taken when the layer has too
few down-projection tiles to fill the GPU: every kept row of y_perm against the oracle's down-projection
of the GPU's own h rows (bf16: 2e-2 per row), and bit for bit the same on a rerun (the S float32 partials
are added in split order, whatever order the blocks finish in)."""
import numpy as np
import pytest
import torch

import combine_experts_amd as M
import oracle as O
import workloads as W
from tests import _parity as P

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")

CASES = {
    # Switch-style capacity layer at full size: 64 tiles, 4 splits
    "switch_cap": W.get_config("switch_cap"),
    # small dropless GELU layer: 4 experts x 4 row tiles x 2 column tiles, F = 2048, 2 splits
    "small_gelu": W.MoEConfig(name="small_gelu", T=1024, D=512, E=4, top_k=1, F=2048, act=W.ACT_GELU, ep_size=1,
                              seed=81),
    # SwiGLU with top-2 and a capacity cut that leaves some experts nearly empty
    "cap_swiglu": W.MoEConfig(name="cap_swiglu", T=1024, D=256, E=8, top_k=2, F=2048, capacity_factor=0.6,
                              bias="normal0.5", ep_size=2, seed=82),
}


@needs_gpu
@pytest.mark.parametrize("name", list(CASES))
def test_split_k_down_projection(name):
    cfg = CASES[name]
    d = M.dims_from_config(cfg)
    n_ws = M.moe_workspace_size(d, M.MOE_STAGE_FFN_DOWN)
    assert n_ws > 0, "these dims are expected to take the split-K path"
    print(f"[splitk] {name}: {cfg} workspace {n_ws / 2**20:.1f} MiB", flush=True)
    inp = W.make_inputs(cfg, "cuda")
    d, buf = P.run_gpu(cfg, inp, split_k=False)   # the layer with the unsplit down-projection fills h, y_perm
    ws = torch.empty(n_ws, dtype=torch.uint8, device="cuda")
    y1 = torch.zeros_like(buf.y_perm)
    y2 = torch.zeros_like(buf.y_perm)
    M.moe_expert_ffn_down_splitk(d, buf.h, buf.expert_offsets, inp["w2"], y1, ws)
    ws.fill_(0xFF)                         # the second call must not depend on the scratch's contents
    M.moe_expert_ffn_down_splitk(d, buf.h, buf.expert_offsets, inp["w2"], y2, ws)
    torch.cuda.synchronize()
    N = int(buf.expert_offsets[-1])
    assert torch.equal(y1[:N], y2[:N]), "split-K result differs between runs"
    # every kept row against the oracle's down-projection of the GPU's h rows
    off = P.i64(buf.expert_offsets)
    hh = P.f64(buf.h[:N])
    ref = np.zeros((N, cfg.D))
    for e in range(cfg.E):
        lo, hi = off[e], off[e + 1]
        if hi > lo:
            ref[lo:hi] = hh[lo:hi] @ O.as_f64(inp["w2"][e].cpu()).T
    err = P.rel_err_rows(P.f64(y1[:N]), ref)
    assert err.max() <= P.TOL_Y[cfg.dtype], f"split-K rows: max rel err {err.max():.3e}"
    # and close to the unsplit down-projection (the same sums, added in another order)
    err_u = P.rel_err_rows(P.f64(y1[:N]), P.f64(buf.y_perm[:N]))
    assert err_u.max() <= 1e-2
    print(f"[splitk] {name}: N={N} max rel err vs oracle {err.max():.2e}, vs unsplit {err_u.max():.2e}", flush=True)


@needs_gpu
def test_split_k_layer_end_to_end():
    """The step as bench.py runs it (route, layout, gathered up-projection, split-K down-projection,
    combine) against the oracle's float64 layer, staged: FFN rows and the combined output."""
    cfg = CASES["small_gelu"]
    inp = W.make_inputs(cfg, "cuda")
    host = P.to_host(inp)
    d = M.dims_from_config(cfg)
    buf = M.MoELayerBuffers(d, device="cuda", logits=True)
    assert buf.down_ws is not None
    M.moe_route(d, inp["x"], inp["w_gate"], inp["bias"], buf.topk_idx, buf.topk_gate, buf.logits)
    M.moe_dispatch_layout(d, buf.topk_idx, buf.expert_counts, buf.expert_offsets, buf.rank_counts, buf.rank_offsets,
                          buf.pair_to_row, buf.row_to_pair, buf.layout_ws)
    M.moe_permute(d, inp["x"], buf.pair_to_row, buf.x_perm)
    M.moe_expert_ffn_up_gather(d, inp["x"], buf.row_to_pair, buf.expert_offsets, inp["w1"], inp["w3"], buf.h)
    M.moe_expert_ffn_down_splitk(d, buf.h, buf.expert_offsets, inp["w2"], buf.y_perm, buf.down_ws)
    M.moe_unpermute_combine(d, buf.y_perm, buf.pair_to_row, buf.topk_gate, buf.y)
    torch.cuda.synchronize()
    r, dec = P.check_route(cfg, host, buf)
    lay = P.check_layout(cfg, buf)
    P.check_ffn_rows(cfg, host, buf, np.arange(lay["n_kept"]), lay)
    P.check_combine_tokens(cfg, buf, np.arange(cfg.T))
    ref = O.layer_forward(host, cfg)
    s = dec["set"]
    err = P.rel_err_rows(P.f64(buf.y)[s], ref["y"][s])
    assert err.max() <= P.TOL_Y[cfg.dtype], f"end to end: {err.max():.3e}"


@needs_gpu
def test_layer_forward_splits_with_a_workspace():
    """moe_layer_forward handed the split-K workspace: the staged entry points' bits with
    moe_expert_ffn_down_splitk, through forward() and a one-micro-batch executor on two streams; without
    the workspace, the unsplit down-projection's bits."""
    cfg = CASES["switch_cap"]
    inp = W.make_inputs(cfg, "cuda")
    args = (inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"])
    d = M.dims_from_config(cfg)
    buf = M.MoELayerBuffers(d, device="cuda")
    assert buf.down_ws is not None
    M.forward(buf, *args)
    st = M.MoELayerBuffers(d, device="cuda")
    M.moe_route(d, inp["x"], inp["w_gate"], inp["bias"], st.topk_idx, st.topk_gate, None)
    M.moe_dispatch_layout(d, st.topk_idx, st.expert_counts, st.expert_offsets, st.rank_counts, st.rank_offsets,
                          st.pair_to_row, st.row_to_pair, st.layout_ws)
    M.moe_permute(d, inp["x"], st.pair_to_row, st.x_perm)
    M.moe_expert_ffn_up(d, st.x_perm, st.expert_offsets, inp["w1"], inp["w3"], st.h)
    M.moe_expert_ffn_down_splitk(d, st.h, st.expert_offsets, inp["w2"], st.y_perm, st.down_ws)
    M.moe_unpermute_combine(d, st.y_perm, st.pair_to_row, st.topk_gate, st.y)
    ex = M.LayerExecutor(d, n_chunks=1, two_streams=True)
    assert ex.down_ws is not None
    y_ex = ex.forward(*args).clone()
    torch.cuda.synchronize()
    assert torch.equal(buf.y, st.y), "forward() differs from the staged split-K path"
    assert torch.equal(y_ex, st.y), "executor differs from the staged split-K path"
    # without the workspace the executor runs the unsplit down-projection
    ex.down_ws = None
    y0 = ex.forward(*args).clone()
    M.moe_expert_ffn_down(d, st.h, st.expert_offsets, inp["w2"], st.y_perm)
    M.moe_unpermute_combine(d, st.y_perm, st.pair_to_row, st.topk_gate, st.y)
    torch.cuda.synchronize()
    assert torch.equal(y0, st.y), "executor without the workspace differs from the unsplit path"
    assert not torch.equal(y0, y_ex), "the split and unsplit sums are expected to round differently somewhere"


@needs_gpu
def test_micro_batches_share_one_split_k_workspace():
    """Four micro-batches on two streams whose down-projections split (each at its own T) and reuse
    one workspace in turn: each micro-batch's rows are the bits of the layer run on that micro-batch
    alone."""
    cfg = W.get_config("switch_cap", T=1024, capacity_factor=0.0)
    n_chunks, tc = 4, 256
    inp = W.make_inputs(cfg, "cuda")
    args = (inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"])
    ex = M.LayerExecutor(M.dims_from_config(cfg), n_chunks=n_chunks, two_streams=True)
    assert ex.down_ws is not None, "a 256-token micro-batch of these dims is expected to split"
    y = ex.forward(inp["x"], *args).clone()
    dc = M.dims_from_config(cfg.replace(T=tc))
    for ci in range(n_chunks):
        one = M.MoELayerBuffers(dc, device="cuda")
        M.forward(one, inp["x"][ci * tc:(ci + 1) * tc].contiguous(), *args)
        torch.cuda.synchronize()
        assert torch.equal(y[ci * tc:(ci + 1) * tc], one.y), f"micro-batch {ci}"
