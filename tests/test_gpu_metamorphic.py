"""Properties of the whole layer on the GPU that need no oracle values.

The layer equation makes a token's output depend only on that token and on which experts (not
which expert numbers) it reaches. Every kernel on the path computes a token's logits, an expert
row's FFN and a token's combine from that token's data alone, in an order that does not depend on
where the row sits in a tile, so the GPU must reproduce these properties bit for bit:
- renaming the experts (router rows, bias and weights moved together) renames the chosen experts
  and leaves the gates, the drops and y unchanged;
- permuting the tokens permutes the routing and y (dropless: with a capacity, token order decides
  the drops);
- a zero down-projection gives y = 0;
- identical experts with gates summing to 1 give every token the same FFN output in each of its k
  rows, and y equal to that row (the float32 gate sum is within a few 2^-24 of 1, far inside the
  half-spacing of bfloat16, so the single rounding returns it);
- in the backward, renaming the experts leaves dx unchanged and moves every per-expert gradient
  (dW_g and bias rows, dW1, dW3, dW2) with its expert."""
import numpy as np
import pytest
import torch

import combine_experts_amd as M
import workloads as W

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")

CASES = [
    # (name, config, expert renaming)
    ("softmax_bias", dict(T=1000, D=256, E=16, top_k=4, F=384, bias="normal0.5"), "shuffle"),
    ("grouped_sigmoid", dict(T=700, D=192, E=64, top_k=8, F=128, gate=W.GATE_SIGMOID_TOPK, n_groups=8,
                             topk_groups=4), "groups"),
    ("gelu_capacity", dict(T=900, D=128, E=8, top_k=1, F=256, act=W.ACT_GELU, capacity_factor=1.25,
                           bias="normal0.5"), "shuffle"),
]


def _run(cfg, inp):
    d = M.dims_from_config(cfg)
    buf = M.MoELayerBuffers(d, device="cuda", x_perm=False)
    M.forward(buf, inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"])
    torch.cuda.synchronize()
    T, k = cfg.T, cfg.top_k
    return {n: getattr(buf, n).clone() for n in ("topk_idx", "topk_gate", "pair_to_row", "expert_counts", "y",
                                                 "y_perm")} | {"idx2": buf.topk_idx.view(T, k).long()}


def _renaming(cfg, kind):
    rng = np.random.default_rng(cfg.seed + 7)
    if kind == "shuffle":
        return rng.permutation(cfg.E)
    # the group limit needs groups kept whole: move whole groups and shuffle inside each
    G = cfg.E // cfg.n_groups
    gperm = rng.permutation(cfg.n_groups)
    return np.concatenate([gperm[g] * G + rng.permutation(G) for g in range(cfg.n_groups)])


@needs_gpu
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_renamed_experts(case):
    name, kw, kind = case
    print(f"[metamorphic] renamed experts {name}", flush=True)
    cfg = W.MoEConfig(name=name, seed=301, **kw)
    inp = W.make_inputs(cfg, "cuda")
    pi = _renaming(cfg, kind)
    pi_t = torch.as_tensor(pi, dtype=torch.long, device="cuda")
    moved = dict(inp)
    for key in ("w_gate", "bias", "w1", "w3", "w2"):
        if inp[key] is not None:
            moved[key] = torch.empty_like(inp[key]).index_copy_(0, pi_t, inp[key])
    a, b = _run(cfg, inp), _run(cfg, moved)
    assert torch.equal(b["idx2"], pi_t[a["idx2"]])
    assert torch.equal(b["topk_gate"], a["topk_gate"])
    assert torch.equal(b["expert_counts"][pi_t], a["expert_counts"])
    assert torch.equal(b["pair_to_row"] >= 0, a["pair_to_row"] >= 0)
    assert torch.equal(b["y"], a["y"])


@needs_gpu
@pytest.mark.parametrize("case", CASES[:2], ids=[c[0] for c in CASES[:2]])
def test_permuted_tokens(case):
    name, kw, _ = case
    print(f"[metamorphic] permuted tokens {name}", flush=True)
    cfg = W.MoEConfig(name=name, seed=302, **kw)
    inp = W.make_inputs(cfg, "cuda")
    g = torch.Generator().manual_seed(303)
    sigma = torch.randperm(cfg.T, generator=g).cuda()
    a, b = _run(cfg, inp), _run(cfg, dict(inp, x=inp["x"][sigma].contiguous()))
    assert torch.equal(b["idx2"], a["idx2"][sigma])
    assert torch.equal(b["y"], a["y"][sigma])


@needs_gpu
def test_zero_down_projection():
    print("[metamorphic] zero W2", flush=True)
    cfg = W.MoEConfig(name="zero_w2", T=500, D=192, E=8, top_k=2, F=256, seed=304)
    inp = W.make_inputs(cfg, "cuda")
    r = _run(cfg, dict(inp, w2=torch.zeros_like(inp["w2"])))
    assert bool((r["y"] == 0).all())


@needs_gpu
@pytest.mark.parametrize("act", [W.ACT_SWIGLU, W.ACT_GELU])
def test_identical_experts(act):
    print(f"[metamorphic] identical experts act={act}", flush=True)
    cfg = W.MoEConfig(name="same_experts", T=600, D=256, E=12, top_k=3, F=192, act=act, seed=305)
    inp = W.make_inputs(cfg, "cuda")
    same = dict(inp)
    for key in ("w1", "w3", "w2"):
        if inp[key] is not None:
            same[key] = inp[key][:1].expand_as(inp[key]).contiguous()
    r = _run(cfg, same)
    rows = r["pair_to_row"].view(cfg.T, cfg.top_k).long()
    assert bool((rows >= 0).all())
    yp = r["y_perm"][rows]                                  # [T, k, D]: a token's k expert rows
    assert torch.equal(yp, yp[:, :1].expand_as(yp))         # the same bits in every slot
    assert torch.equal(r["y"], yp[:, 0])


def _train_step(cfg, inp, dy):
    d = M.dims_from_config(cfg)
    buf = M.MoELayerBuffers(d, device="cuda", logits=True, x_perm=False)
    bw = M.BackwardBuffers(d, device="cuda")
    M.forward_train(buf, bw, inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"])
    M.backward(buf, bw, inp["x"], inp["w_gate"], dy, transpose_weights=(inp["w1"], inp["w3"], inp["w2"]))
    torch.cuda.synchronize()
    out = {n: getattr(bw, n).clone() for n in ("dx", "dw_gate", "dbias", "dw1", "dw2")}
    out["dw3"] = None if bw.dw3 is None else bw.dw3.clone()
    return out


@needs_gpu
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_renamed_experts_backward(case):
    # the backward sums an expert's rows in pair-id order and a token's slots in slot order, neither
    # of which depends on the experts' numbers: dx is unchanged and every per-expert gradient moves
    # with its expert, bit for bit
    name, kw, kind = case
    print(f"[metamorphic] renamed experts, backward {name}", flush=True)
    cfg = W.MoEConfig(name=name, seed=306, **kw)
    inp = W.make_inputs(cfg, "cuda")
    if inp["bias"] is None:
        inp["bias"] = (torch.randn(cfg.E, generator=torch.Generator().manual_seed(307)) * 0.1).cuda()
    pi = _renaming(cfg, kind)
    pi_t = torch.as_tensor(pi, dtype=torch.long, device="cuda")
    moved = dict(inp)
    for key in ("w_gate", "bias", "w1", "w3", "w2"):
        if inp[key] is not None:
            moved[key] = torch.empty_like(inp[key]).index_copy_(0, pi_t, inp[key])
    dy = torch.randn((cfg.T, cfg.D), generator=torch.Generator().manual_seed(308)).to(torch.bfloat16).cuda()
    a, b = _train_step(cfg, inp, dy), _train_step(cfg, moved, dy)
    assert torch.equal(b["dx"], a["dx"])
    for n in ("dw_gate", "dbias", "dw1", "dw3", "dw2"):
        if a[n] is not None:
            assert torch.equal(b[n][pi_t], a[n]), n
