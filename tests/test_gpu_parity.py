"""GPU parity: every stage of the HIP path against the CPU oracle (staged protocol, see _parity.py).

Small variants of each workload shape run the oracle on everything (element by element); they
span several row and column tiles and leave ragged tails. The full workload shapes (the launch
configuration bench.py times) are checked on sampled rows/tokens and by properties that hold at
any size.
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

SMALL = {
    "tiny_fp32": W.get_config("tiny_fp32"),
    "switch_cap": W.get_config("switch_cap"),
    "switch_cap_cf1": W.get_config("switch_cap", T=2048, capacity_factor=1.0),
    "mixtral_small": W.get_config("mixtral", T=1000, D=512, F=1856),
    "dsv3_small": W.get_config("dsv3", T=600, D=512, F=320),
    "skew_small": W.get_config("skew", T=3000, D=256, F=448),
    "odd_bf16": W.MoEConfig(name="odd_bf16", T=77, D=64, E=3, top_k=2, F=192, ep_size=3, seed=7),
    "odd_f32": W.MoEConfig(name="odd_f32", T=50, D=48, E=5, top_k=3, F=80, ep_size=5, dtype=W.DT_F32,
                           gate=W.GATE_SOFTMAX_FULL, seed=8),
    "cap_k2": W.MoEConfig(name="cap_k2", T=500, D=128, E=6, top_k=2, F=128, ep_size=2, capacity_factor=0.8,
                          bias="normal0.5", seed=9),
    "sigmoid_nogroup": W.MoEConfig(name="sigmoid_nogroup", T=300, D=128, E=32, top_k=4, F=128, ep_size=8,
                                   gate=W.GATE_SIGMOID_TOPK, seed=10),
    "softmax_groups": W.MoEConfig(name="softmax_groups", T=200, D=128, E=64, top_k=6, F=128, ep_size=16,
                                  n_groups=8, topk_groups=3, seed=11),
}


@needs_gpu
@pytest.mark.parametrize("name", list(SMALL))
def test_small_all_stages(name):
    cfg = SMALL[name]
    print(f"[parity] {name}: {cfg}", flush=True)
    inp = W.make_inputs(cfg, "cuda")
    host = P.to_host(inp)
    d, buf = P.run_gpu(cfg, inp)
    r, dec = P.check_route(cfg, host, buf, decisive_min_frac=0.5)
    lay = P.check_layout(cfg, buf)
    N = lay["n_kept"]
    assert int(buf.expert_offsets[-1]) == N
    P.check_permute_rows(cfg, host, buf, np.arange(N))
    P.check_ffn_rows(cfg, host, buf, np.arange(N), lay)
    P.check_combine_tokens(cfg, buf, np.arange(cfg.T))
    P.check_identity_experts(cfg, buf, inp["x"])
    # volume accounting: dispatch writes N rows, combine reads N rows
    assert O.comm_volume_elements(N, cfg.D) == 2 * N * cfg.D
    assert int(buf.rank_counts.sum()) == N == cfg.T * cfg.top_k - lay["n_dropped"]
    # end to end on decisive tokens, against the oracle's own float64 layer (dropless only:
    # with a capacity, one flipped route elsewhere can change who is dropped)
    if cfg.capacity_factor <= 0:
        ref = O.layer_forward(host, cfg)
        s = dec["set"]
        err = P.rel_err_rows(P.f64(buf.y)[s], ref["y"][s])
        assert err.max() <= P.TOL_Y[cfg.dtype], f"end-to-end max rel err {err.max():.3e}"


@needs_gpu
@pytest.mark.parametrize("name", ["tiny_fp32", "switch_cap", "mixtral_small", "dsv3_small", "odd_f32", "cap_k2"])
def test_expert_ffn_single_call(name):
    """moe_expert_ffn (both FFN halves, h in the caller's workspace) against the oracle's expert FFN on
    the GPU's own x_perm and offsets, element by element; the same bits as the two halves in turn."""
    cfg = SMALL[name]
    print(f"[parity] moe_expert_ffn {name}: {cfg}", flush=True)
    inp = W.make_inputs(cfg, "cuda")
    host = P.to_host(inp)
    d, buf = P.run_gpu(cfg, inp)
    ws = torch.empty(M.moe_workspace_size(d, M.MOE_STAGE_FFN), dtype=torch.uint8, device="cuda")
    y_perm = torch.zeros_like(buf.y_perm)
    M.moe_expert_ffn(d, buf.x_perm, buf.expert_offsets, inp["w1"], inp["w3"], inp["w2"], y_perm, ws)
    # the same two halves called one by one (the down-projection split over K where these dims split)
    h2, y2 = torch.empty_like(buf.h), torch.zeros_like(buf.y_perm)
    M.moe_expert_ffn_up(d, buf.x_perm, buf.expert_offsets, inp["w1"], inp["w3"], h2)
    M.moe_expert_ffn_down_splitk(d, h2, buf.expert_offsets, inp["w2"], y2, buf.down_ws)
    torch.cuda.synchronize()
    N = int(buf.expert_offsets[-1])
    assert torch.equal(y_perm[:N], y2[:N]), "moe_expert_ffn differs from up + down"
    assert torch.equal(y_perm[:N], buf.y_perm[:N]), "moe_expert_ffn differs from the layer's FFN"
    off = P.i64(buf.expert_offsets)
    ref = O.expert_ffn(P.f64(buf.x_perm[:N]), off, host["w1"], host["w3"], host["w2"], cfg.act)
    err = P.rel_err_rows(P.f64(y_perm[:N]), ref[:N])
    assert err.max(initial=0.0) <= P.TOL_Y[cfg.dtype], f"moe_expert_ffn: max rel err {err.max():.3e}"


@needs_gpu
@pytest.mark.parametrize("name", ["mixtral_small", "dsv3_small", "cap_k2"])
def test_deterministic_rerun(name):
    cfg = SMALL[name]
    inp = W.make_inputs(cfg, "cuda")
    _, b1 = P.run_gpu(cfg, inp)
    _, b2 = P.run_gpu(cfg, inp)
    for key, t in b1.as_dict().items():
        if t is None or key in ("layout_ws", "down_ws"):   # scratch
            continue
        t2 = getattr(b2, key)
        if key in ("x_perm", "h", "y_perm"):       # rows past N are unspecified
            n = int(b1.expert_offsets[-1])
            t, t2 = t[:n], t2[:n]
        assert torch.equal(t, t2), f"{key} differs between runs"


@needs_gpu
def test_empty_batch():
    cfg = W.MoEConfig(name="empty", T=0, D=64, E=4, top_k=2, F=64, ep_size=2)
    inp = W.make_inputs(cfg.replace(T=1), "cuda")
    inp["x"] = inp["x"][:0]
    d = M.dims_from_config(cfg)
    buf = M.MoELayerBuffers(d, device="cuda", logits=True)
    M.forward(buf, inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"])
    torch.cuda.synchronize()
    assert buf.expert_counts.tolist() == [0, 0, 0, 0]
    assert buf.expert_offsets.tolist() == [0, 0, 0, 0, 0]
    assert buf.rank_counts.tolist() == [0, 0] and buf.rank_offsets.tolist() == [0, 0, 0]


@needs_gpu
def test_all_tokens_to_one_expert_spans_many_tiles():
    cfg = W.MoEConfig(name="hot", T=700, D=128, E=8, top_k=1, F=192, ep_size=4, seed=12)
    inp = W.make_inputs(cfg, "cuda")
    inp["bias"] = torch.tensor([50.0] + [0.0] * 7, device="cuda")
    host = P.to_host(inp)
    d, buf = P.run_gpu(cfg, inp)
    P.check_route(cfg, host, buf)
    lay = P.check_layout(cfg, buf)
    assert lay["expert_counts"].tolist() == [700, 0, 0, 0, 0, 0, 0, 0]
    P.check_permute_rows(cfg, host, buf, np.arange(700))
    P.check_ffn_rows(cfg, host, buf, np.arange(700), lay)
    P.check_combine_tokens(cfg, buf, np.arange(700))


@needs_gpu
def test_k_equals_e():
    cfg = W.MoEConfig(name="k_eq_e", T=130, D=64, E=4, top_k=4, F=64, ep_size=2, seed=13)
    inp = W.make_inputs(cfg, "cuda")
    host = P.to_host(inp)
    d, buf = P.run_gpu(cfg, inp)
    P.check_route(cfg, host, buf, decisive_min_frac=0.9)
    lay = P.check_layout(cfg, buf)
    assert lay["expert_counts"].tolist() == [130] * 4
    P.check_ffn_rows(cfg, host, buf, np.arange(lay["n_kept"]), lay)
    P.check_combine_tokens(cfg, buf, np.arange(cfg.T))
    P.check_identity_experts(cfg, buf, inp["x"])


@needs_gpu
def test_exact_ties_go_to_lowest_index():
    # duplicate router rows give bit-identical logits; the lower expert index must win
    cfg = W.MoEConfig(name="ties", T=256, D=64, E=8, top_k=2, F=64, ep_size=1, seed=14)
    inp = W.make_inputs(cfg, "cuda")
    wg = inp["w_gate"].clone()
    wg[5] = wg[2]
    wg[7] = wg[2]
    inp["w_gate"] = wg
    host = P.to_host(inp)
    d, buf = P.run_gpu(cfg, inp)
    P.check_route(cfg, host, buf, decisive_min_frac=0.0)
    idx = P.i64(buf.topk_idx).reshape(cfg.T, cfg.top_k)
    # experts 5 and 7 carry expert 2's logits: wherever one of them is chosen, 2 was chosen first
    for row in idx:
        if 5 in row or 7 in row:
            assert 2 in row and list(row).index(2) < min(list(row).index(e) for e in (5, 7) if e in row)


# ------------------------------------------------------------------------------------------------
# Full workload shapes: sampled checks and whole-size properties
# ------------------------------------------------------------------------------------------------

FULL = ["switch_cap", "mixtral", "dsv3", "skew"]


def _sample_rows(lay, rng, per_expert=4, n_random=512, max_experts=12):
    off = lay["expert_offsets"]
    E = len(off) - 1
    nonempty = [e for e in range(E) if off[e + 1] > off[e]]
    sizes = {e: off[e + 1] - off[e] for e in nonempty}
    pick = {nonempty[0], nonempty[-1], max(sizes, key=sizes.get), min(sizes, key=sizes.get)}
    rest = [e for e in nonempty if e not in pick]
    pick |= set(rng.choice(rest, size=min(len(rest), max_experts - len(pick)), replace=False).tolist()) if rest else set()
    rows = set()
    for e in pick:
        lo, hi = off[e], off[e + 1]
        rows |= {lo, hi - 1}
        rows |= set(rng.integers(lo, hi, size=min(per_expert, hi - lo)).tolist())
    # random rows restricted to the picked experts keep the weight fetches bounded
    allowed = np.concatenate([np.arange(off[e], off[e + 1]) for e in pick])
    rows |= set(rng.choice(allowed, size=min(n_random, allowed.size), replace=False).tolist())
    return np.array(sorted(rows))


@needs_gpu
@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    cfg = W.get_config(name)
    print(f"[parity-full] {name}: {cfg.desc}", flush=True)
    rng = np.random.default_rng(1234)
    inp = W.make_inputs(cfg, "cuda")
    host = {k: (None if inp[k] is None else inp[k].cpu()) for k in ("x", "w_gate", "bias")}
    d, buf = P.run_gpu(cfg, inp)
    print("[parity-full] route", flush=True)
    r, dec = P.check_route(cfg, host, buf, decisive_min_frac=0.5)
    print("[parity-full] layout", flush=True)
    lay = P.check_layout(cfg, buf)
    N = lay["n_kept"]
    print(f"[parity-full] N={N} drops={lay['n_dropped']} max/mean count="
          f"{lay['expert_counts'].max() / lay['expert_counts'].mean():.2f}", flush=True)
    rows = _sample_rows(lay, rng)
    P.check_permute_rows(cfg, host, buf, rows)
    # full-size permute property: every kept row equals its token's x row (checked on the GPU)
    r2p = buf.row_to_pair[:N].long()
    assert torch.equal(buf.x_perm[:N], inp["x"][r2p // cfg.top_k])
    # the up-projection with the permute fused into its row loads (the form the benchmark times):
    # the same h bit for bit
    print("[parity-full] gather up-projection", flush=True)
    h2 = torch.empty_like(buf.h)
    M.moe_expert_ffn_up_gather(d, inp["x"], buf.row_to_pair, buf.expert_offsets, inp["w1"], inp["w3"], h2)
    torch.cuda.synchronize()
    assert torch.equal(h2[:N], buf.h[:N])
    del h2
    print("[parity-full] ffn rows", len(rows), flush=True)
    wcache = {}

    def getter(key):
        def f(e):
            if (key, e) not in wcache:
                wcache[(key, e)] = inp[key][e].cpu()
            return wcache[(key, e)]
        return None if inp[key] is None else f

    hw = {"w1": getter("w1"), "w3": getter("w3"), "w2": getter("w2")}
    P.check_ffn_rows(cfg, hw, buf, rows, lay)
    if name == "skew":
        off = lay["expert_offsets"]
        hot = int(np.argmax(lay["kept_counts"]))
        P.check_ffn_rows(cfg, hw, buf, np.arange(off[hot], off[hot + 1]), lay)
    print("[parity-full] combine", flush=True)
    toks = rng.choice(cfg.T, size=min(1024, cfg.T), replace=False)
    P.check_combine_tokens(cfg, buf, toks)
    P.check_identity_experts(cfg, buf, inp["x"])
    wcache.clear()
    # end to end against the oracle's float64 layer on E2E_TOKENS random decisive tokens, topped up so
    # that every expert serves at least one of them (dropless workloads: with a capacity a flipped route
    # elsewhere can change who is dropped, so switch_cap is compared staged only)
    if cfg.capacity_factor <= 0:
        toks = _e2e_tokens(r["topk_idx"], dec["set"], cfg.E, rng)
        print(f"[parity-full] end to end on {len(toks)} decisive tokens", flush=True)
        idx_t, g_t = r["topk_idx"][toks], r["topk_gate"][toks]
        xr = O.as_f64(host["x"][torch.as_tensor(toks)])
        ref = np.zeros((len(toks), cfg.D))
        for e in np.unique(idx_t):
            ti, sj = np.nonzero(idx_t == e)
            # one expert's weights at a time, upcast exactly to float64
            we = {key: (None if inp[key] is None else inp[key][e].double().cpu().numpy()) for key in ("w1", "w3", "w2")}
            out = O.expert_ffn_rows(xr[ti], np.full(len(ti), e), lambda _e: we["w1"],
                                    None if we["w3"] is None else (lambda _e: we["w3"]), lambda _e: we["w2"], cfg.act)
            ref[ti] += g_t[ti, sj][:, None] * out
        err = P.rel_err_rows(P.f64(buf.y[torch.as_tensor(toks, device=buf.y.device)]), ref)
        print(f"[parity-full] end to end max rel err {err.max():.3e}", flush=True)
        assert err.max() <= P.TOL_Y[cfg.dtype], f"end to end: max rel err {err.max():.3e}"


E2E_TOKENS = 256


def _e2e_tokens(topk_idx, decisive, E, rng):
    """E2E_TOKENS random decisive tokens plus, for any expert none of them uses, one more decisive token
    routed to it (when one exists)."""
    cand = np.nonzero(decisive)[0]
    toks = set(rng.choice(cand, size=min(E2E_TOKENS, cand.size), replace=False).tolist())
    covered = set(topk_idx[sorted(toks)].reshape(-1).tolist())
    for e in range(E):
        if e in covered:
            continue
        hit = cand[(topk_idx[cand] == e).any(axis=1)]
        if hit.size:
            toks.add(int(hit[0]))
            covered |= set(topk_idx[hit[0]].tolist())
    return np.array(sorted(toks))
