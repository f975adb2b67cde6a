"""Grouped expert GEMMs on hand-picked per-expert row counts.

The bf16 grouped GEMM covers an expert's rows with 320-row tiles (the last one partial), so the
counts here hit every case: an empty expert, one row, a 32-row edge, exactly one full tile, one row
past it, partial second and third tiles, and an expert with more than ten tiles. Up- and down-projection (plain, gathered rows from x, and the K-major weight
read of the backward data gradient) are compared row by row with the oracle's expert FFN on the same
rows; the gathered up-projection equals the one on permuted rows bit for bit. A second set has more
experts than a GEMM block has threads, which takes the tile map's multi-pass scan; and a reduction long
enough (F = 8192) for the down-projection's earlier ring refill."""
import numpy as np
import pytest
import torch

import combine_experts_amd as M
import oracle as O
import workloads as W
from tests._parity import TOL_Y, f64, rel_err_rows

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")

COUNTS = [0, 1, 32, 33, 320, 321, 352, 641, 700, 961, 3201, 17]


def _setup(act):
    E = len(COUNTS)
    N = sum(COUNTS)
    cfg = W.MoEConfig(name="row_tiles", T=N, D=192, E=E, top_k=1, F=128, act=act, seed=91)
    inp = W.make_inputs(cfg, "cuda")
    d = M.dims_from_config(cfg)
    offsets = torch.tensor(np.concatenate([[0], np.cumsum(COUNTS)]), dtype=torch.int32, device="cuda")
    # rows of x in a fixed shuffled order: x_perm[r] = x[row_to_pair[r]] (top-1, so pair = token)
    g = torch.Generator().manual_seed(92)
    row_to_pair = torch.randperm(N, generator=g).to(torch.int32).cuda()
    x_perm = inp["x"][row_to_pair.long()].contiguous()
    return cfg, inp, d, offsets, row_to_pair, x_perm


def _experts_of_rows():
    return np.repeat(np.arange(len(COUNTS)), COUNTS)


@needs_gpu
@pytest.mark.parametrize("act", [W.ACT_SWIGLU, W.ACT_GELU])
def test_forward_on_every_row_split(act):
    print(f"[row_tiles] forward act={act}", flush=True)
    cfg, inp, d, offsets, row_to_pair, x_perm = _setup(act)
    N = cfg.T
    h = torch.full((N, cfg.F), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.moe_expert_ffn_up(d, x_perm, offsets, inp["w1"], inp["w3"], h)
    hg = torch.full_like(h, float("nan"))
    M.moe_expert_ffn_up_gather(d, inp["x"], row_to_pair, offsets, inp["w1"], inp["w3"], hg)
    y = torch.full((N, cfg.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.moe_expert_ffn_down(d, h, offsets, inp["w2"], y)
    torch.cuda.synchronize()
    assert torch.equal(hg, h)
    ref = O.expert_ffn_rows(x_perm.cpu(), _experts_of_rows(), inp["w1"].cpu(),
                            None if inp["w3"] is None else inp["w3"].cpu(), inp["w2"].cpu(), act)
    err = rel_err_rows(f64(y), ref)
    assert err.max() <= TOL_Y[cfg.dtype], f"max rel err {err.max():.3e} at row {int(err.argmax())}"


@needs_gpu
def test_data_gradients_on_every_row_split():
    # da = (dy_perm · W2[e]) * GELU'(pre) and dx_perm = da · W1[e], the weights read as stored
    print("[row_tiles] data gradients", flush=True)
    cfg, inp, d, offsets, _, _ = _setup(W.ACT_GELU)
    N = cfg.T
    g = torch.Generator(device="cuda").manual_seed(93)
    dy = torch.randn((N, cfg.D), device="cuda", generator=g).to(torch.bfloat16)
    pre = torch.randn((N, cfg.F), device="cuda", generator=g).to(torch.bfloat16)
    da = torch.full((N, cfg.F), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.moe_expert_ffn_down_backward_w(d, dy, offsets, inp["w2"], pre, da)
    dx = torch.full((N, cfg.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.moe_expert_ffn_up_backward_w(d, da, offsets, inp["w1"], None, dx)
    torch.cuda.synchronize()
    w1, w2, dyh, dah = f64(inp["w1"]), f64(inp["w2"]), f64(dy), f64(da)
    ref_da = np.empty((N, cfg.F))
    ref_dx = np.empty((N, cfg.D))
    o = 0
    for e, c in enumerate(COUNTS):
        ref_da[o:o + c] = dyh[o:o + c] @ w2[e]
        ref_dx[o:o + c] = dah[o:o + c] @ w1[e]  # on the GPU's own da: each GEMM checked alone
        o += c
    ref_da *= O.gelu_grad(f64(pre))
    for name, got, ref in (("da", da, ref_da), ("dx_perm", dx, ref_dx)):
        err = rel_err_rows(f64(got), ref)
        assert err.max() <= TOL_Y[cfg.dtype], f"{name}: max rel err {err.max():.3e} at row {int(err.argmax())}"


@needs_gpu
def test_more_experts_than_block_threads():
    # 600 experts (the tile map scans the per-expert tile counts in several block-wide passes)
    print("[row_tiles] 600 experts", flush=True)
    rng = np.random.default_rng(94)
    counts = rng.integers(0, 40, size=600)
    counts[::7] = 0
    counts[5] = 700  # one expert with three row tiles
    E, N = len(counts), int(counts.sum())
    cfg = W.MoEConfig(name="many_experts", T=N, D=64, E=E, top_k=1, F=64, seed=95)
    inp = W.make_inputs(cfg, "cuda")
    d = M.dims_from_config(cfg)
    offsets = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device="cuda")
    x_perm = inp["x"]
    h = torch.full((N, cfg.F), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = torch.full((N, cfg.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.moe_expert_ffn_up(d, x_perm, offsets, inp["w1"], inp["w3"], h)
    M.moe_expert_ffn_down(d, h, offsets, inp["w2"], y)
    torch.cuda.synchronize()
    experts = np.repeat(np.arange(E), counts)
    ref = O.expert_ffn_rows(x_perm.cpu(), experts, inp["w1"].cpu(), inp["w3"].cpu(), inp["w2"].cpu(), cfg.act)
    err = rel_err_rows(f64(y), ref)
    assert err.max() <= TOL_Y[cfg.dtype], f"max rel err {err.max():.3e} at row {int(err.argmax())}"


@needs_gpu
def test_down_projection_with_a_long_reduction():
    # F = 8192: the plain down-projection takes the ring that loads every other stage one k-step
    # earlier (reductions this long); every row of ragged tiles against the oracle's expert FFN rows
    counts = [0, 1, 33, 320, 321, 700]
    E, N, F, D = len(counts), sum(counts), 8192, 128
    cfg = W.MoEConfig(name="long_k", T=N, D=D, E=E, top_k=1, F=F, act=W.ACT_GELU, seed=93)
    print(f"[row_tiles] long reduction F={F}", flush=True)
    inp = W.make_inputs(cfg, "cuda")
    d = M.dims_from_config(cfg)
    offsets = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device="cuda")
    h = torch.full((N, F), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.moe_expert_ffn_up(d, inp["x"], offsets, inp["w1"], None, h)
    y = torch.full((N, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.moe_expert_ffn_down(d, h, offsets, inp["w2"], y)
    torch.cuda.synchronize()
    experts = np.repeat(np.arange(E), counts)
    ref = O.expert_ffn_rows(inp["x"].cpu(), experts, inp["w1"].cpu(), None, inp["w2"].cpu(), W.ACT_GELU)
    err = rel_err_rows(f64(y), ref)
    assert err.max() <= TOL_Y[cfg.dtype], f"max rel err {err.max():.3e} at row {int(err.argmax())}"
    # the down-projection alone on the GPU's own h, against a float64 product of the same operands
    hh, w2 = f64(h), inp["w2"].double().cpu().numpy()
    ref2 = np.concatenate([hh[o:o + c] @ w2[e].T for e, (o, c) in
                           enumerate(zip(np.concatenate([[0], np.cumsum(counts)])[:-1], counts))])
    err2 = rel_err_rows(f64(y), ref2)
    assert err2.max() <= 8e-3, f"down-projection on the GPU's h: max rel err {err2.max():.3e}"
