"""GPU parity of the layer executor: micro-batches on two streams and the shared expert.

Micro-batching changes only which rows share an expert group and when each step runs; every
token's route, every row's FFN and every token's combine meet the same kernels with the same
operands, so the overlapped executor must equal the plain layer bit for bit. (A split-K
down-projection splits by the micro-batch's own tile count, so these comparisons run without the
split-K workspace; its own tests cover it.) The shared expert is
checked against the oracle's float64 layer (routed sum + shared expert) on decisive tokens.
"""
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
    "tiny_fp32": W.get_config("tiny_fp32"),
    "mixtral_small": W.get_config("mixtral", T=1024, D=512, F=1856),
    "dsv3_small": W.get_config("dsv3", T=640, D=512, F=320),
    "skew_small": W.get_config("skew", T=2048, D=256, F=448),
    "switch_dropless": W.get_config("switch_cap", T=1024, capacity_factor=0.0),
}


def _shared(inp):
    return (inp["shared_w1"], inp["shared_w3"], inp["shared_w2"]) if "shared_w1" in inp else None


@needs_gpu
@pytest.mark.parametrize("name", list(CASES))
def test_micro_batches_on_two_streams_equal_the_plain_layer(name):
    cfg = CASES[name]
    print(f"[overlap] {name}: {cfg}", flush=True)
    inp = W.make_inputs(cfg, "cuda")
    _, buf = P.run_gpu(cfg, inp, logits=False, split_k=False)
    d = M.dims_from_config(cfg)
    for n_chunks, two in ((1, False), (2, False), (2, True), (4, True)):
        ex = M.LayerExecutor(d, n_chunks=n_chunks, two_streams=two, split_k=False)
        y = ex.forward(inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"])
        torch.cuda.synchronize()
        assert torch.equal(y, buf.y), f"{n_chunks} micro-batches, two streams={two}"
        # a second call reuses buffers and events
        y2 = ex.forward(inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"]).clone()
        torch.cuda.synchronize()
        assert torch.equal(y2, buf.y)


SHARED = {
    "dsv3_small_shared": W.get_config("dsv3", T=640, D=512, F=320, shared_F=320),
    "mixtral_small_shared": W.get_config("mixtral", T=512, D=512, F=1856, shared_F=1024),
    "gelu_shared": W.MoEConfig(name="gelu_shared", T=384, D=256, E=16, top_k=1, F=512, act=W.ACT_GELU, ep_size=4,
                               bias="normal0.5", seed=51, shared_F=256),
    "f32_shared": W.MoEConfig(name="f32_shared", T=128, D=64, E=8, top_k=2, F=96, dtype=W.DT_F32, seed=52,
                              shared_F=80),
}


@needs_gpu
@pytest.mark.parametrize("name", list(SHARED))
def test_shared_expert_layer(name):
    cfg = SHARED[name]
    print(f"[overlap] {name}: {cfg}", flush=True)
    inp = W.make_inputs(cfg, "cuda")
    host = P.to_host(inp)
    d = M.dims_from_config(cfg)
    ex1 = M.LayerExecutor(d, n_chunks=1, shared_F=cfg.shared_F, split_k=False)
    y1 = ex1.forward(inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"], shared=_shared(inp)).clone()
    torch.cuda.synchronize()
    # against the oracle's float64 layer (routed + shared) on decisive tokens
    ref = O.layer_forward(host, cfg)
    dec = O.decisive_tokens(ref["logits"], cfg.top_k, 1e-3, cfg.n_groups, cfg.topk_groups, cfg.gate)["set"]
    assert dec.mean() > 0.5
    err = P.rel_err_rows(P.f64(y1)[dec], ref["y"][dec])
    assert err.max() <= P.TOL_Y[cfg.dtype], f"shared-expert layer: max rel err {err.max():.3e}"
    # the shared part alone: the executor's scratch holds the shared expert's output
    sh_ref = O.shared_expert_ffn(host["x"], host["shared_w1"], host["shared_w3"], host["shared_w2"], cfg.act)
    err_s = P.rel_err_rows(P.f64(ex1.shared_y), sh_ref)
    assert err_s.max() <= P.TOL_Y[cfg.dtype], f"shared expert: max rel err {err_s.max():.3e}"
    # micro-batches on two streams: bit for bit the same
    for n_chunks in (2, 4):
        ex = M.LayerExecutor(d, n_chunks=n_chunks, two_streams=True, shared_F=cfg.shared_F, split_k=False)
        y = ex.forward(inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"], shared=_shared(inp))
        torch.cuda.synchronize()
        assert torch.equal(y, y1), f"{n_chunks} micro-batches with the shared expert"


@needs_gpu
def test_combine_with_addend():
    cfg = W.get_config("mixtral", T=300, D=512, F=1856)
    inp = W.make_inputs(cfg, "cuda")
    _, buf = P.run_gpu(cfg, inp, logits=False)
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    add = torch.randn((cfg.T, cfg.D), generator=g, device="cuda").to(torch.bfloat16)
    y = torch.empty_like(buf.y)
    M.moe_unpermute_combine_add(buf.d, buf.y_perm, buf.pair_to_row, buf.topk_gate, add, y)
    y0 = torch.empty_like(buf.y)
    M.moe_unpermute_combine_add(buf.d, buf.y_perm, buf.pair_to_row, buf.topk_gate, None, y0)
    torch.cuda.synchronize()
    assert torch.equal(y0, buf.y), "no addend = moe_unpermute_combine"
    N = int(buf.expert_offsets[-1])
    ref = O.combine(P.f64(buf.y_perm[:N]), P.i64(buf.pair_to_row), P.f64(buf.topk_gate), cfg.T, cfg.top_k) + P.f64(add)
    err = P.rel_err_rows(P.f64(y), ref)
    assert err.max() <= P.TOL_COMBINE[cfg.dtype], f"combine with addend: max rel err {err.max():.3e}"


@needs_gpu
def test_overlapped_full_dsv3_with_shared_expert():
    cfg = W.get_config("dsv3", shared_F=2048)
    print(f"[overlap] full dsv3 + shared expert", flush=True)
    inp = W.make_inputs(cfg, "cuda")
    d = M.dims_from_config(cfg)
    ex1 = M.LayerExecutor(d, n_chunks=1, shared_F=cfg.shared_F, split_k=False)
    y1 = ex1.forward(inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"], shared=_shared(inp)).clone()
    del ex1
    ex2 = M.LayerExecutor(d, n_chunks=2, two_streams=True, shared_F=cfg.shared_F, split_k=False)
    y2 = ex2.forward(inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"], shared=_shared(inp))
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    # sampled tokens against the oracle (routed part through the GPU's own routing and rows)
    host_x = inp["x"][:8].cpu()
    sh = O.shared_expert_ffn(host_x, inp["shared_w1"].cpu(), inp["shared_w3"].cpu(), inp["shared_w2"].cpu(), cfg.act)
    err = P.rel_err_rows(P.f64(ex2.shared_y[:8]), sh)
    assert err.max() <= P.TOL_Y[cfg.dtype]
