"""Edge cases of the newer paths on the GPU: an empty batch through the executor, the cluster view,
the padded layout and the backward (every gradient exactly zero); experts that receive no rows in
the backward; a micro-batch count equal to the token count; a layer at the largest top-k (32)."""
import numpy as np
import pytest
import torch

import combine_experts_amd as M
import workloads as W
from tests import _parity as P

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


@needs_gpu
def test_empty_batch_everywhere():
    cfg = W.MoEConfig(name="empty", T=0, D=128, E=8, top_k=2, F=128, ep_size=4, capacity_factor=1.25, seed=71)
    inp = W.make_inputs(cfg, "cuda")
    d = M.dims_from_config(cfg)
    buf = M.MoELayerBuffers(d, device="cuda", logits=True)
    # forward through the executor (one and two streams)
    M.forward(buf, inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"])
    ex = M.LayerExecutor(d, n_chunks=1, two_streams=True)
    ex.forward(inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"])
    # cluster view: a zero matrix, an empty receive layout
    matrix = torch.full((4, 4), 7, dtype=torch.int32, device="cuda")
    M.moe_dispatch_matrix(d, buf.topk_idx, 4, matrix)
    src_off = torch.zeros((4, cfg.E + 1), dtype=torch.int32, device="cuda")
    rc = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    eo = torch.full((cfg.E // 4 + 1,), 7, dtype=torch.int32, device="cuda")
    g2s = torch.full((16,), 7, dtype=torch.int32, device="cuda")
    M.moe_recv_layout(d, 4, 1, 0, src_off, rc, eo, g2s)
    # padded layout: C = 0, no slots
    poff = torch.full((cfg.E + 1,), 7, dtype=torch.int32, device="cuda")
    s2p = torch.empty(0, dtype=torch.int32, device="cuda")
    M.moe_dispatch_layout(d, buf.topk_idx, buf.expert_counts, buf.expert_offsets, buf.rank_counts, buf.rank_offsets,
                          buf.pair_to_row, buf.row_to_pair, buf.layout_ws)
    M.moe_padded_layout(d, buf.topk_idx, buf.expert_offsets, buf.pair_to_row, buf.row_to_pair, buf.pair_to_row, s2p,
                        poff)
    assert M.moe_capacity(d) == 0
    none = torch.empty((0, cfg.D), dtype=torch.bfloat16, device="cuda")
    M.moe_permute_padded(d, inp["x"], s2p, none)
    M.moe_expert_ffn_padded_up(d, none, poff, inp["w1"], inp["w3"], none)
    M.moe_expert_ffn_padded_down(d, none, poff, inp["w2"], none)
    # backward: every gradient exactly zero
    bw = M.BackwardBuffers(d, device="cuda")
    for t in (bw.dw_gate, bw.dbias, bw.dw1, bw.dw3, bw.dw2):
        t.fill_(7.0)
    dy = torch.empty((0, cfg.D), dtype=torch.bfloat16, device="cuda")
    M.forward_train(buf, bw, inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"])
    M.backward(buf, bw, inp["x"], inp["w_gate"], dy, transpose_weights=(inp["w1"], inp["w3"], inp["w2"]))
    torch.cuda.synchronize()
    assert bool((matrix == 0).all())
    assert bool((rc == 0).all()) and bool((eo == 0).all()) and bool((g2s == -1).all())
    assert bool((poff == 0).all())
    for n, t in (("dw_gate", bw.dw_gate), ("dbias", bw.dbias), ("dw1", bw.dw1), ("dw3", bw.dw3), ("dw2", bw.dw2)):
        assert bool((t == 0).all()), f"{n} of an empty batch"


@needs_gpu
def test_backward_experts_without_rows():
    # 64 experts, 40 tokens, k = 1: most experts get no row; their weight gradients are exact zeros
    cfg = W.MoEConfig(name="sparse", T=40, D=128, E=64, top_k=1, F=128, seed=72)
    inp = W.make_inputs(cfg, "cuda")
    d = M.dims_from_config(cfg)
    buf = M.MoELayerBuffers(d, device="cuda", logits=True)
    bw = M.BackwardBuffers(d, device="cuda")
    M.forward_train(buf, bw, inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"])
    dy = torch.randn((cfg.T, cfg.D), device="cuda").to(torch.bfloat16)
    M.backward(buf, bw, inp["x"], inp["w_gate"], dy, transpose_weights=(inp["w1"], inp["w3"], inp["w2"]))
    torch.cuda.synchronize()
    counts = P.i64(buf.expert_counts)
    empty = np.nonzero(counts == 0)[0]
    assert len(empty) > 20
    for e in empty:
        assert bool((bw.dw1[e] == 0).all()) and bool((bw.dw3[e] == 0).all()) and bool((bw.dw2[e] == 0).all())
    # the experts with rows: dW2[e] = dy_perm[rows of e]^T h[rows of e], in float64 from the GPU's own operands
    off = P.i64(buf.expert_offsets)
    dyp, h = P.f64(bw.dy_perm), P.f64(buf.h)
    for e in np.nonzero(counts > 0)[0]:
        r = slice(off[e], off[e + 1])
        ref = dyp[r].T @ h[r]
        err = np.abs(P.f64(bw.dw2[e]) - ref).max() / max(np.abs(ref).max(), 1e-30)
        assert err <= 1e-3, f"dW2 expert {e}: {err:.3e}"


@needs_gpu
def test_one_token_per_micro_batch():
    cfg = W.get_config("mixtral", T=8, D=512, F=448)
    inp = W.make_inputs(cfg, "cuda")
    _, buf = P.run_gpu(cfg, inp, logits=False)
    ex = M.LayerExecutor(M.dims_from_config(cfg), n_chunks=8, two_streams=True)
    y = ex.forward(inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"])
    torch.cuda.synchronize()
    assert torch.equal(y, buf.y)


@needs_gpu
@pytest.mark.parametrize("cf", [0.0, 0.75])
def test_layer_with_the_largest_top_k(cf):
    # k = 32, the router's largest: the general selection, combine and layout paths, every stage
    # against the oracle (with a capacity cut too)
    cfg = W.MoEConfig(name=f"k32_cf{cf}", T=100, D=64, E=48, top_k=32, F=64, ep_size=4, capacity_factor=cf,
                      seed=72)
    print(f"[edge] {cfg.name}", flush=True)
    inp = W.make_inputs(cfg, "cuda")
    host = P.to_host(inp)
    d, buf = P.run_gpu(cfg, inp)
    r, dec = P.check_route(cfg, host, buf, decisive_min_frac=0.5)
    lay = P.check_layout(cfg, buf)
    N = lay["n_kept"]
    P.check_permute_rows(cfg, host, buf, np.arange(N))
    P.check_ffn_rows(cfg, host, buf, np.arange(N), lay)
    P.check_combine_tokens(cfg, buf, np.arange(cfg.T))
    P.check_identity_experts(cfg, buf, inp["x"])
