"""GPU parity on seeded random layer shapes: every stage against the oracle (the staged protocol of
tests/_parity.py), on dims drawn across what the entry points accept -- bf16 and float32, 1 to 256
experts, top-1 to top-8, the three gate forms, group limits, capacity cuts, selection biases, odd token
counts -- so that combinations no hand-picked case names are covered too."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests import _parity as P

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")

N_CASES = 64


def _divisors(n, lo=1, hi=None):
    hi = n if hi is None else hi
    return [v for v in range(lo, min(n, hi) + 1) if n % v == 0]


def random_config(i):
    """Layer dims number i: a seeded draw within the library's documented limits (router: E <= 256,
    bf16 D a multiple of 64; grouped GEMMs: bf16 D, F multiples of 64, float32 of 16)."""
    rng = np.random.default_rng(1000 + i)
    E = int(rng.choice([1, 2, 3, 5, 8, 12, 16, 24, 32, 64, 96, 128, 256]))
    k = int(rng.integers(1, min(E, 8) + 1))
    gate = int(rng.choice([W.GATE_SOFTMAX_TOPK, W.GATE_SIGMOID_TOPK, W.GATE_SOFTMAX_FULL]))
    n_groups = topk_groups = 0
    if E >= 4 and rng.random() < 0.35:
        opts = [g for g in _divisors(E, 2, 64) if g < E]
        if opts:
            n_groups = int(rng.choice(opts))
            gsize = E // n_groups
            lo = max(1, -(-k // gsize))   # enough kept groups to hold k experts
            topk_groups = int(rng.integers(lo, n_groups + 1))
    bf16 = rng.random() < 0.7
    if bf16:
        D, F = 64 * int(rng.integers(1, 5)), 64 * int(rng.integers(1, 6))
    else:
        D, F = 16 * int(rng.integers(1, 17)), 16 * int(rng.integers(1, 21))
    T = int(rng.choice([1, 2, 7, 33, 64, 65, 127, 200, 333, 400, 1000, 2049]))
    return W.MoEConfig(
        name=f"random{i}", T=T, D=D, E=E, top_k=k, F=F,
        act=int(rng.choice([W.ACT_SWIGLU, W.ACT_GELU])),
        dtype=W.DT_BF16 if bf16 else W.DT_F32, gate=gate,
        capacity_factor=float(rng.choice([0.0, 0.0, 0.5, 1.0, 1.25, 2.0])),
        ep_size=int(rng.choice(_divisors(E))), n_groups=n_groups, topk_groups=topk_groups,
        bias=str(rng.choice(["none", "normal0.5"])), seed=2000 + i)


def test_random_configs_are_valid():
    # (host only) the draws stay inside the documented limits and cover each option at least once
    cfgs = [random_config(i) for i in range(N_CASES)]
    for c in cfgs:
        assert 1 <= c.top_k <= min(c.E, 8) and c.E % c.ep_size == 0
        if c.n_groups:
            assert c.E % c.n_groups == 0 and c.topk_groups * (c.E // c.n_groups) >= c.top_k
        assert (c.D % 64 == 0 and c.F % 64 == 0) if c.dtype == W.DT_BF16 else (c.D % 16 == 0 and c.F % 16 == 0)
    assert {c.dtype for c in cfgs} == {W.DT_BF16, W.DT_F32}
    assert {c.gate for c in cfgs} == {W.GATE_SOFTMAX_TOPK, W.GATE_SIGMOID_TOPK, W.GATE_SOFTMAX_FULL}
    assert any(c.n_groups for c in cfgs) and any(c.capacity_factor > 0 for c in cfgs)
    assert any(c.bias != "none" for c in cfgs) and any(c.act == W.ACT_GELU for c in cfgs)


@needs_gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_all_stages(i):
    cfg = random_config(i)
    print(f"[random] {cfg}", flush=True)
    inp = W.make_inputs(cfg, "cuda")
    host = P.to_host(inp)
    d, buf = P.run_gpu(cfg, inp)
    r, dec = P.check_route(cfg, host, buf, decisive_min_frac=0.0)
    lay = P.check_layout(cfg, buf)
    N = lay["n_kept"]
    assert int(buf.expert_offsets[-1]) == N
    P.check_permute_rows(cfg, host, buf, np.arange(N))
    if N:
        P.check_ffn_rows(cfg, host, buf, np.arange(N), lay)
    P.check_combine_tokens(cfg, buf, np.arange(cfg.T))
    P.check_identity_experts(cfg, buf, inp["x"])
    if cfg.capacity_factor <= 0 and dec["set"].any():
        ref = O.layer_forward(host, cfg)
        s = dec["set"]
        err = P.rel_err_rows(P.f64(buf.y)[s], ref["y"][s])
        assert err.max() <= P.TOL_Y[cfg.dtype], f"end-to-end max rel err {err.max():.3e}"
