"""GPU parity of the load-balancing pieces: the router's selection-only bias and probability sums
(moe_route_ex) and the statistics / bias step (moe_load_balance), against the oracle.

Selection under a bias is compared like plain routing: bit for bit against the oracle's
selection applied to the GPU's own float32 logits (tokens whose biased scores tie within 1e-5
excepted, since the GPU's float32 sigmoid may differ from the correctly rounded one by an ulp),
and bit for bit against the oracle's float64 routing on decisive tokens (biased-score margin
> 1e-3). Probability sums and the auxiliary loss: float32 sums against float64, relative 1e-5.
The bias step is bit-exact (its sign is decided in integers, the add is one float32 rounding).
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
    "mixtral_small": W.get_config("mixtral", T=1000, D=512, F=1856),
    "dsv3_small": W.get_config("dsv3", T=600, D=512, F=320),
    "skew_small": W.get_config("skew", T=3000, D=256, F=448),
    "switch_small": W.get_config("switch_cap", T=700),
    "odd_f32": W.MoEConfig(name="odd_f32", T=50, D=48, E=5, top_k=3, F=80, ep_size=5, dtype=W.DT_F32,
                           gate=W.GATE_SOFTMAX_FULL, seed=8),
    "sigmoid_nogroup": W.MoEConfig(name="sigmoid_nogroup", T=300, D=128, E=32, top_k=4, F=128, ep_size=8,
                                   gate=W.GATE_SIGMOID_TOPK, seed=10),
    "softmax_groups": W.MoEConfig(name="softmax_groups", T=200, D=128, E=64, top_k=6, F=128, ep_size=16,
                                  n_groups=8, topk_groups=3, seed=11),
    "general_e100": W.MoEConfig(name="general_e100", T=130, D=64, E=100, top_k=5, F=64, ep_size=4,
                                gate=W.GATE_SIGMOID_TOPK, n_groups=10, topk_groups=4, seed=12),
}

TOL_P = 1e-5


def _route_ex(cfg, inp, sb, want_partials=True):
    d = M.dims_from_config(cfg)
    dev = inp["x"].device
    idx = torch.empty(cfg.T * cfg.top_k, dtype=torch.int32, device=dev)
    gate = torch.empty(cfg.T * cfg.top_k, dtype=torch.float32, device=dev)
    logits = torch.empty(cfg.T * cfg.E, dtype=torch.float32, device=dev)
    n_part = (cfg.T + 63) // 64
    part = torch.full((max(1, n_part) * cfg.E,), float("nan"), dtype=torch.float32, device=dev) \
        if want_partials else None
    M.moe_route_ex(d, inp["x"], inp["w_gate"], inp["bias"], sb, idx, gate, logits, part)
    torch.cuda.synchronize()
    return d, idx, gate, logits, part


def _check_biased_route(cfg, host, sb_host, idx, gate, logits):
    T, E, k = cfg.T, cfg.E, cfg.top_k
    l_gpu = P.f64(logits).reshape(T, E)
    idx_gpu = P.i64(idx).reshape(T, k)
    g_gpu = P.f64(gate).reshape(T, k)
    # (1) the oracle's biased selection on the GPU's own logits
    key = O.selection_key(l_gpu, cfg.gate, sb_host)
    if cfg.n_groups > 0:
        want, _ = O.select_group_limited(key, k, cfg.n_groups, cfg.topk_groups, key)
    else:
        want = O.select_topk(key, k)
    if cfg.gate == W.GATE_SIGMOID_TOPK or cfg.n_groups > 0:
        # float32 sigmoid and float32 group sums may differ from the oracle's by an ulp
        dm = O.decisive_tokens(key, k, 1e-5, cfg.n_groups, cfg.topk_groups, W.GATE_SOFTMAX_TOPK)["order"]
        assert dm.mean() > 0.9, f"only {dm.mean():.3f} tokens clear of float32 ties"
    else:
        dm = np.ones(T, dtype=bool)  # logit + bias is one float32 rounding on both sides
    assert np.array_equal(want[dm], idx_gpu[dm]), "biased selection on GPU logits"
    # gates always come from the unbiased logits of the chosen experts
    g_want = O.gate_weights(l_gpu, idx_gpu, cfg.gate)
    assert np.abs(g_want - g_gpu).max() <= P.TOL_GATE, "gates on GPU logits"
    # (2) decisive tokens against the oracle's float64 routing with the same bias
    r = O.route(host["x"], host["w_gate"], host["bias"], k, cfg.gate, cfg.n_groups, cfg.topk_groups,
                select_bias=sb_host)
    key64 = O.selection_key(O.round_to_f32(r["logits"]), cfg.gate, sb_host)
    dec = O.decisive_tokens(key64, k, 1e-3, cfg.n_groups, cfg.topk_groups, W.GATE_SOFTMAX_TOPK)
    s, o = dec["set"], dec["order"]
    assert s.mean() >= 0.5
    assert np.array_equal(np.sort(idx_gpu[s], axis=1), np.sort(r["topk_idx"][s], axis=1)), "decisive sets"
    assert np.array_equal(idx_gpu[o], r["topk_idx"][o]), "decisive slot order"
    assert np.abs(g_gpu[o] - r["topk_gate"][o]).max(initial=0.0) <= 1e-5, "decisive gates"
    return r


def _check_partials(cfg, logits, part):
    T, E = cfg.T, cfg.E
    l_gpu = P.f64(logits).reshape(T, E)
    p = O.router_probabilities(l_gpu, cfg.gate)
    n_part = (T + 63) // 64
    got = P.f64(part)[: n_part * E].reshape(n_part, E)
    for b in range(n_part):
        want = p[64 * b: 64 * b + 64].sum(axis=0)
        assert np.abs(got[b] - want).max() <= TOL_P * 64, f"probability partial of block {b}"


@needs_gpu
@pytest.mark.parametrize("name", list(CASES))
def test_route_ex_select_bias_and_partials(name):
    cfg = CASES[name]
    print(f"[balance] {name}: {cfg}", flush=True)
    inp = W.make_inputs(cfg, "cuda", with_experts=False)
    host = P.to_host(inp)
    sb = W.make_select_bias(cfg, "cuda")
    _, idx, gate, logits, part = _route_ex(cfg, inp, sb)
    _check_biased_route(cfg, host, sb.cpu().numpy(), idx, gate, logits)
    _check_partials(cfg, logits, part)


@needs_gpu
@pytest.mark.parametrize("name", ["mixtral_small", "dsv3_small", "general_e100", "tiny_fp32"])
def test_route_ex_without_extras_is_route(name):
    cfg = CASES[name]
    inp = W.make_inputs(cfg, "cuda", with_experts=False)
    d = M.dims_from_config(cfg)
    a = [torch.empty(cfg.T * cfg.top_k, dtype=t, device="cuda") for t in (torch.int32, torch.float32)]
    la = torch.empty(cfg.T * cfg.E, dtype=torch.float32, device="cuda")
    M.moe_route(d, inp["x"], inp["w_gate"], inp["bias"], a[0], a[1], la)
    # partials only: the selection and gates must not move at all
    _, idx, gate, logits, part = _route_ex(cfg, inp, None, want_partials=True)
    assert torch.equal(a[0], idx) and torch.equal(a[1], gate) and torch.equal(la, logits)
    _, idx, gate, logits, _ = _route_ex(cfg, inp, None, want_partials=False)
    assert torch.equal(a[0], idx) and torch.equal(a[1], gate)
    if cfg.gate != W.GATE_SIGMOID_TOPK:
        # a zero bias on logits ranks the logits themselves
        _, idx, gate, _, _ = _route_ex(cfg, inp, torch.zeros(cfg.E, device="cuda"), want_partials=False)
        assert torch.equal(a[0], idx) and torch.equal(a[1], gate)


@needs_gpu
@pytest.mark.parametrize("name", ["dsv3_small", "skew_small", "odd_f32", "general_e100"])
def test_load_balance_stats_and_bias_step(name):
    cfg = CASES[name]
    inp = W.make_inputs(cfg, "cuda", with_experts=False)
    sb = W.make_select_bias(cfg, "cuda")
    d, idx, gate, logits, part = _route_ex(cfg, inp, sb)
    counts = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    buf = M.MoELayerBuffers(d, device="cuda")
    M.moe_dispatch_layout(d, idx, counts, buf.expert_offsets, buf.rank_counts, buf.rank_offsets, buf.pair_to_row,
                          buf.row_to_pair, buf.layout_ws)
    stats = torch.full((2 * cfg.E + 2,), float("nan"), dtype=torch.float32, device="cuda")
    sb_before = sb.cpu().numpy().copy()
    alpha, gamma = 0.01, 1e-3
    M.moe_load_balance(d, counts, part, alpha, stats, gamma, sb)
    torch.cuda.synchronize()
    c = P.i64(counts)
    assert c.sum() == cfg.T * cfg.top_k
    probs = O.router_probabilities(P.f64(logits).reshape(cfg.T, cfg.E), cfg.gate)
    want = O.load_balance_stats(c, probs, cfg.top_k, alpha)
    got = P.f64(stats)
    E = cfg.E
    np.testing.assert_allclose(got[:E], want["f"], rtol=1e-7, atol=0)
    np.testing.assert_allclose(got[E:2 * E], want["P"], rtol=TOL_P, atol=1e-7)
    assert got[2 * E] == pytest.approx(want["aux_loss"], rel=TOL_P)
    assert got[2 * E + 1] == pytest.approx(want["imbalance"], rel=1e-6)
    np.testing.assert_array_equal(sb.cpu().numpy(), O.update_select_bias(sb_before, c, gamma))
    # the same call again gives the same statistics bit for bit (fixed summation order)
    stats2 = torch.empty_like(stats)
    M.moe_load_balance(d, counts, part, alpha, stats2, 0.0, None)
    torch.cuda.synchronize()
    assert torch.equal(stats, stats2)


@needs_gpu
def test_load_balance_empty_batch():
    cfg = W.MoEConfig(name="empty", T=0, D=64, E=8, top_k=2, F=64, ep_size=1)
    d = M.dims_from_config(cfg)
    counts = torch.zeros(cfg.E, dtype=torch.int32, device="cuda")
    stats = torch.full((2 * cfg.E + 2,), float("nan"), dtype=torch.float32, device="cuda")
    sb = torch.linspace(-1, 1, cfg.E, device="cuda")
    sb0 = sb.clone()
    M.moe_load_balance(d, counts, None, 0.01, stats, 0.5, sb)
    torch.cuda.synchronize()
    assert bool((stats == 0).all())
    assert torch.equal(sb, sb0)


@needs_gpu
@pytest.mark.parametrize("gate", [W.GATE_SOFTMAX_TOPK, W.GATE_SIGMOID_TOPK])
def test_closed_loop_bias_balances_skewed_routing(gate):
    """Route -> count -> bias step, repeated on the GPU: every step matches the oracle's step on the
    GPU's counts bit for bit, and the load imbalance falls well below where it started."""
    cfg = W.get_config("skew", T=4096, D=256, F=448, gate=gate, n_groups=0, topk_groups=0)
    inp = W.make_inputs(cfg, "cuda", with_experts=False)
    d = M.dims_from_config(cfg)
    buf = M.MoELayerBuffers(d, device="cuda")
    n_part = (cfg.T + 63) // 64
    part = torch.empty(n_part * cfg.E, dtype=torch.float32, device="cuda")
    stats = torch.empty(2 * cfg.E + 2, dtype=torch.float32, device="cuda")
    sb = torch.zeros(cfg.E, dtype=torch.float32, device="cuda")
    gamma = 0.01 if gate == W.GATE_SIGMOID_TOPK else 0.05
    imb = []
    for _ in range(40):
        M.moe_route_ex(d, inp["x"], inp["w_gate"], inp["bias"], sb, buf.topk_idx, buf.topk_gate, None, part)
        M.moe_dispatch_layout(d, buf.topk_idx, buf.expert_counts, buf.expert_offsets, buf.rank_counts,
                              buf.rank_offsets, buf.pair_to_row, buf.row_to_pair, buf.layout_ws)
        before = sb.cpu().numpy().copy()
        M.moe_load_balance(d, buf.expert_counts, part, 0.01, stats, gamma, sb)
        torch.cuda.synchronize()
        c = P.i64(buf.expert_counts)
        np.testing.assert_array_equal(sb.cpu().numpy(), O.update_select_bias(before, c, gamma))
        imb.append(float(stats[2 * cfg.E + 1]))
        assert imb[-1] == pytest.approx(c.max() / c.mean(), rel=1e-6)
    print(f"[balance] imbalance {imb[0]:.3f} -> {imb[-1]:.3f}", flush=True)
    assert imb[0] > 2.5
    assert max(imb[-5:]) < 0.6 * imb[0]


@needs_gpu
def test_route_ex_full_dsv3_shape():
    """The DeepSeek-V3-shaped router at its full size (T=16384, D=7168, E=256, 8 groups) with a bias."""
    cfg = W.get_config("dsv3")
    print(f"[balance] full dsv3 route: {cfg}", flush=True)
    inp = W.make_inputs(cfg, "cuda", with_experts=False)
    host = P.to_host(inp)
    sb = W.make_select_bias(cfg, "cuda")
    _, idx, gate, logits, part = _route_ex(cfg, inp, sb)
    _check_biased_route(cfg, host, sb.cpu().numpy(), idx, gate, logits)
    p = O.router_probabilities(P.f64(logits).reshape(cfg.T, cfg.E), cfg.gate)
    n_part = (cfg.T + 63) // 64
    got = P.f64(part).reshape(n_part, cfg.E).sum(axis=0) / cfg.T
    np.testing.assert_allclose(got, p.mean(axis=0), rtol=TOL_P, atol=1e-8)
