"""Shared helpers of the GPU parity tests: run the HIP path, compare each stage with the oracle.

Staged protocol: every GPU stage is compared with the oracle's version of that stage applied to
the GPU's own input for it (the previous GPU stage's output), so integer stages compare bit for
bit on all tokens. Routing is compared with the oracle's own float64 routing on decisive tokens
(k-th vs (k+1)-th logit margin > 1e-3), and bit for bit on all tokens against the oracle's
selection applied to the GPU's float32 logits. Floating tolerances:
  bf16 layer output: max relative error per token <= 2e-2; fp32: <= 1e-4
  (per-token relative error = max_d |y - y_ref| / max(max_d |y_ref|, 1e-6)).
"""
from __future__ import annotations

import numpy as np
import torch

import combine_experts_amd as M
import oracle as O
import workloads as W

TOL_Y = {W.DT_BF16: 2e-2, W.DT_F32: 1e-4}
# combine alone rounds once: one bf16 rounding is 2^-9 relative of the largest element
TOL_COMBINE = {W.DT_BF16: 8e-3, W.DT_F32: 1e-5}
TOL_GATE = 2e-6          # gates from the same fp32 logits: float32 exp/div vs float64
TOL_LOGIT_REL = 1e-5     # float32 accumulation vs float64, relative to sum |x_d W_d|


def to_host(inp):
    return {k: (None if v is None else v.detach().cpu()) for k, v in inp.items()}


def run_gpu(cfg, inp, logits=True, split_k=True):
    """The layer forward; split_k=False drops the split-K workspace, so the down-projection runs
    unsplit wherever it would split."""
    d = M.dims_from_config(cfg)
    buf = M.MoELayerBuffers(d, device="cuda", logits=logits)
    if not split_k:
        buf.down_ws = None
    M.forward(buf, inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"])
    torch.cuda.synchronize()
    return d, buf


def rel_err_rows(y, ref):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.maximum(np.abs(ref).max(axis=1), 1e-6)
    return np.abs(y - ref).max(axis=1) / scale


def f64(t):
    return t.detach().cpu().double().numpy()


def i64(t):
    return t.detach().cpu().long().numpy()


def check_route(cfg, host, buf, decisive_min_frac=0.5):
    """Logits, selection and gates vs the oracle; returns the oracle route and decisive masks."""
    T, E, k = cfg.T, cfg.E, cfg.top_k
    r = O.route(host["x"], host["w_gate"], host["bias"], k, cfg.gate, cfg.n_groups, cfg.topk_groups)
    l_gpu = f64(buf.logits).reshape(T, E)
    # logits: float32 accumulation error bound relative to sum_d |x_d W_ed| (+ |bias|)
    absdot = np.abs(O.as_f64(host["x"])) @ np.abs(O.as_f64(host["w_gate"])).T
    if host["bias"] is not None:
        absdot = absdot + np.abs(O.as_f64(host["bias"]))[None, :]
    assert np.all(np.abs(l_gpu - r["logits"]) <= TOL_LOGIT_REL * absdot + 1e-30), "router logits"
    idx_gpu = i64(buf.topk_idx).reshape(T, k)
    g_gpu = f64(buf.topk_gate).reshape(T, k)
    # (1) all tokens: the oracle's selection on the GPU's own float32 logits picks the same experts
    if cfg.n_groups > 0:
        score = 1.0 / (1.0 + np.exp(-l_gpu)) if cfg.gate == W.GATE_SIGMOID_TOPK else l_gpu
        idx_on_gpu_l, _ = O.select_group_limited(l_gpu, k, cfg.n_groups, cfg.topk_groups, score)
        # group sums are float32 on the GPU: skip tokens whose group scores tie within 1e-5
        dm = O.decisive_tokens(l_gpu, k, 1e-5, cfg.n_groups, cfg.topk_groups, cfg.gate)["set"]
        assert np.array_equal(idx_on_gpu_l[dm], idx_gpu[dm]), "selection on GPU logits (group-limited)"
        assert dm.mean() > 0.99
    else:
        idx_on_gpu_l = O.select_topk(l_gpu, k)
        assert np.array_equal(idx_on_gpu_l, idx_gpu), "selection on GPU logits"
    g_on_gpu_l = O.gate_weights(l_gpu, idx_gpu, cfg.gate)
    assert np.abs(g_on_gpu_l - g_gpu).max() <= TOL_GATE, "gates on GPU logits"
    # (2) decisive tokens: bit-exact against the oracle's float64 routing
    dec = O.decisive_tokens(r["logits"], k, 1e-3, cfg.n_groups, cfg.topk_groups, cfg.gate)
    s, o = dec["set"], dec["order"]
    assert s.mean() >= decisive_min_frac, f"only {s.mean():.3f} decisive"
    assert np.array_equal(np.sort(idx_gpu[s], axis=1), np.sort(r["topk_idx"][s], axis=1)), "decisive sets"
    assert np.array_equal(idx_gpu[o], r["topk_idx"][o]), "decisive slot order"
    assert np.abs(g_gpu[o] - r["topk_gate"][o]).max(initial=0.0) <= 1e-5, "decisive gates"
    if cfg.n_groups > 0:
        gsize = E // cfg.n_groups
        assert all(len(set((row // gsize).tolist())) <= cfg.topk_groups for row in idx_gpu)
    return r, dec


def check_layout(cfg, buf):
    T, E, k = cfg.T, cfg.E, cfg.top_k
    C = O.capacity(cfg.capacity_factor, T, k, E)
    idx_gpu = i64(buf.topk_idx).reshape(T, k)
    lay = O.dispatch_layout(idx_gpu, E, cfg.ep_size, C)
    assert M.moe_capacity(buf.d) == C
    assert np.array_equal(i64(buf.expert_counts), lay["expert_counts"]), "expert_counts"
    assert np.array_equal(i64(buf.expert_offsets), lay["expert_offsets"]), "expert_offsets"
    assert np.array_equal(i64(buf.rank_counts), lay["rank_counts"]), "rank_counts"
    assert np.array_equal(i64(buf.rank_offsets), lay["rank_offsets"]), "rank_offsets"
    assert np.array_equal(i64(buf.pair_to_row), lay["pair_to_row"]), "pair_to_row"
    assert np.array_equal(i64(buf.row_to_pair), lay["row_to_pair"]), "row_to_pair"
    return lay


def check_permute_rows(cfg, host, buf, rows):
    k = cfg.top_k
    r2p = i64(buf.row_to_pair)
    rows = np.asarray(rows, dtype=np.int64)
    got = f64(buf.x_perm[torch.as_tensor(rows, device=buf.x_perm.device)])
    want = O.as_f64(host["x"])[r2p[rows] // k]
    assert np.array_equal(got, want), "permute (bitwise)"


def check_ffn_rows(cfg, host_w, buf, rows, lay):
    """y_perm on the given rows vs the oracle FFN applied to the GPU's x_perm rows."""
    rows = np.asarray(rows, dtype=np.int64)
    off = lay["expert_offsets"]
    experts = np.searchsorted(off, rows, side="right") - 1
    tr = torch.as_tensor(rows, device=buf.x_perm.device)
    xr = buf.x_perm[tr].cpu()
    ref = O.expert_ffn_rows(xr, experts, host_w["w1"], host_w["w3"], host_w["w2"], cfg.act)
    got = f64(buf.y_perm[tr])
    err = rel_err_rows(got, ref)
    assert err.max() <= TOL_Y[cfg.dtype], f"ffn rows: max rel err {err.max():.3e}"
    return err.max()


def check_combine_tokens(cfg, buf, tokens):
    T, k = cfg.T, cfg.top_k
    tokens = np.asarray(tokens, dtype=np.int64)
    p2r = i64(buf.pair_to_row).reshape(T, k)[tokens]
    g = f64(buf.topk_gate).reshape(T, k)[tokens]
    rows = np.unique(p2r[p2r >= 0])
    yp = np.zeros((max(int(rows.max()) + 1 if rows.size else 1, 1), cfg.D))
    if rows.size:
        yp[rows] = f64(buf.y_perm[torch.as_tensor(rows, device=buf.y_perm.device)])
    ref = O.combine(yp, p2r.reshape(-1), g, len(tokens), k)
    got = f64(buf.y[torch.as_tensor(tokens, device=buf.y.device)])
    err = rel_err_rows(got, ref)
    assert err.max() <= TOL_COMBINE[cfg.dtype], f"combine: max rel err {err.max():.3e}"
    allz = (p2r < 0).all(axis=1)
    assert np.all(got[allz] == 0), "fully dropped tokens must be exactly 0"
    return err.max()


def check_identity_experts(cfg, buf, x):
    """Identity experts: combine(permute(x)) with gates summing to 1 gives x back (0 if dropped)."""
    d = buf.d
    y_id = torch.empty_like(buf.y)
    M.moe_unpermute_combine(d, buf.x_perm, buf.pair_to_row, buf.topk_gate, y_id)
    torch.cuda.synchronize()
    kept = (buf.pair_to_row.view(cfg.T, cfg.top_k) >= 0)
    any_kept = kept.any(dim=1)
    all_kept = kept.all(dim=1)
    if cfg.gate == W.GATE_SOFTMAX_FULL:
        # full-softmax gates do not sum to 1 over the top k: identity experts give x * sum_j g_j
        gsum = buf.topk_gate.view(cfg.T, cfg.top_k).double().sum(dim=1, keepdim=True)
        want = (x.double() * gsum)[all_kept]
        tol = 4e-3 if cfg.dtype == W.DT_BF16 else 1e-6
        torch.testing.assert_close(y_id[all_kept].double(), want, rtol=tol, atol=tol)
    elif cfg.dtype == W.DT_BF16:
        assert torch.equal(y_id[all_kept], x[all_kept]), "identity experts (bitwise bf16)"
    else:
        torch.testing.assert_close(y_id[all_kept], x[all_kept], rtol=4e-7, atol=1e-7)
    assert bool((y_id[~any_kept] == 0).all()), "dropped tokens give 0"
