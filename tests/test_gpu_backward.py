"""GPU parity of the layer backward (bf16), stage by stage against the oracle.

Each GPU step is compared with the oracle's formula for that step applied to the GPU's own inputs
for it (the saved forward tensors and the previous backward step's output), so integer routing
differences never enter: dy_perm and dgate, the activation backward da, dx_perm, the router's dl,
dW_g and dbias, the final dx, the transposes (bit for bit) and the three weight gradients. dx is also
compared end to end with the oracle's float64 layer backward on decisive tokens.
Every gradient is then compared with the oracle's float64 layer backward (O.layer_backward) run on
the GPU's own routing, layout, logits, x_perm and y_perm.
Tolerances: bf16 outputs 2e-2 per row relative to the row's largest reference entry (the bound the
layer output has); float32 outputs (dgate, dl, dW_g, dbias) 1e-3 relative to the largest reference
entry; weight gradients element by element within a first-order bound of the GPU's roundings and
within 2e-2 of the largest entry (TOL_WG_SUM, TOL_WG and _perturbation_scale below).
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

TOL_ROW = 2e-2
TOL_F32 = 1e-3
# weight gradients: each is a sum over an expert's rows of products whose GPU operands carry bf16
# roundings; each rounding moves its value by at most 2^-8 relative (bf16 keeps 8 significant bits,
# round to nearest), and _perturbation_scale adds up, to first order, what every rounding on the way to
# an operand can move it by (in units of 2^-8). TOL_WG_SUM allows twice that (the float32 sums add
# ~1e-6 relative). TOL_WG: the largest error within 2e-2 of the expert's largest entry, the bound of
# the layer's bf16 output
TOL_WG_SUM = 2 * 2.0 ** -8
TOL_WG = 2e-2
SILU2_MAX, GELU2_MAX = 0.5, 0.8   # max |SiLU''| = 0.5 (at 0), max |GELU''| = 2 phi(0) = 0.798


def _perturbation_scale(ob, host, cfg, e, lo, hi):
    """First-order bounds, in units of 2^-8, on how far the GPU's bf16 roundings move the left operands
    of expert e's weight gradients: dy_perm (rounded once) for dW2; da1 and da3 for dW1, dW3.
    da1 = dh * a3 * SiLU'(a1) (GELU: dh * GELU'(a1)) and da3 = dh * SiLU(a1) are formed from dh, a sum
    over dy_perm rows (each rounded: |d dh| <= sum |dy_perm||W2| =: dh_abs), the stored pre-activations
    a1, a3 (rounded: |d a| <= |a|, and f(a1) moves by at most max|f''| |a1| for f = SiLU', or max|f'| for
    f = SiLU), and are rounded once more themselves."""
    dyp = np.abs(ob["dy_perm"][lo:hi])
    dh = ob["dh"][lo:hi]
    a1 = ob["a1"][lo:hi]
    dh_abs = dyp @ np.abs(O.as_f64(host["w2"][e]))
    if cfg.act == W.ACT_SWIGLU:
        a3 = ob["a3"][lo:hi]
        s1 = O.silu_grad(a1)
        m1 = dh_abs * np.abs(a3 * s1) + 2 * np.abs(dh * a3 * s1) + SILU2_MAX * np.abs(dh * a3 * a1)
        m3 = dh_abs * np.abs(O.silu(a1)) + 1.1 * np.abs(dh * a1) + np.abs(dh * O.silu(a1))
    else:
        g1 = O.gelu_grad(a1)
        m1 = dh_abs * np.abs(g1) + GELU2_MAX * np.abs(dh * a1) + np.abs(dh * g1)
        m3 = None
    return 2 * dyp, m1, m3

CASES = {
    "mixtral_small": W.get_config("mixtral", T=512, D=512, F=448),
    "dsv3_small": W.get_config("dsv3", T=320, D=512, F=320),
    "gelu_k1_bias": W.MoEConfig(name="gelu_k1_bias", T=384, D=256, E=16, top_k=1, F=512, act=W.ACT_GELU, ep_size=4,
                                bias="normal0.5", seed=61),
    "full_softmax": W.MoEConfig(name="full_softmax", T=256, D=128, E=8, top_k=3, F=192, gate=W.GATE_SOFTMAX_FULL,
                                bias="normal0.5", seed=62),
    "capacity": W.MoEConfig(name="capacity", T=400, D=128, E=6, top_k=2, F=128, capacity_factor=0.8, seed=63),
    "skew_small": W.get_config("skew", T=1024, D=256, F=192),
    # k > 8: the general combine, backward combine and dx kernels (the others keep k rows in registers)
    "k10_general": W.MoEConfig(name="k10_general", T=200, D=128, E=16, top_k=10, F=128, seed=64),
}


def _random_config(i):
    """bf16 layer dims number i for the backward: a seeded draw over expert counts, top-k, the three
    gate forms, group limits, capacity cuts, selection-free biases and both activations."""
    rng = np.random.default_rng(3000 + i)
    E = int(rng.choice([2, 3, 5, 8, 12, 16, 24, 32, 64, 96, 128, 256]))
    k = int(rng.integers(1, min(E, 8) + 1))
    n_groups = topk_groups = 0
    if E >= 4 and rng.random() < 0.4:
        opts = [g for g in range(2, min(E, 64) + 1) if E % g == 0 and g < E]
        if opts:
            n_groups = int(rng.choice(opts))
            topk_groups = int(rng.integers(max(1, -(-k // (E // n_groups))), n_groups + 1))
    return W.MoEConfig(
        name=f"random{i}", T=int(rng.choice([33, 64, 65, 127, 200, 333])), D=64 * int(rng.integers(1, 5)), E=E,
        top_k=k, F=64 * int(rng.integers(1, 6)), act=int(rng.choice([W.ACT_SWIGLU, W.ACT_GELU])),
        gate=int(rng.choice([W.GATE_SOFTMAX_TOPK, W.GATE_SIGMOID_TOPK, W.GATE_SOFTMAX_FULL])),
        capacity_factor=float(rng.choice([0.0, 0.0, 0.5, 1.25])), n_groups=n_groups, topk_groups=topk_groups,
        bias=str(rng.choice(["none", "normal0.5"])), seed=4000 + i)


N_RANDOM = 8
for _i in range(N_RANDOM):
    CASES[f"random{_i}"] = _random_config(_i)


def test_random_backward_configs_are_valid():
    # (host only) the draws are valid layer dims and cover every gate form, both activations, group
    # limits and capacity cuts
    cfgs = [_random_config(i) for i in range(N_RANDOM)]
    for c in cfgs:
        assert 1 <= c.top_k <= min(c.E, 8) and c.D % 64 == 0 and c.F % 64 == 0
        if c.n_groups:
            assert c.E % c.n_groups == 0 and c.topk_groups * (c.E // c.n_groups) >= c.top_k
    assert {c.gate for c in cfgs} == {W.GATE_SOFTMAX_TOPK, W.GATE_SIGMOID_TOPK, W.GATE_SOFTMAX_FULL}
    assert {c.act for c in cfgs} == {W.ACT_SWIGLU, W.ACT_GELU}
    assert any(c.n_groups for c in cfgs) and any(c.capacity_factor > 0 for c in cfgs)


def _nm(cfg):
    return 2 if cfg.act == W.ACT_SWIGLU else 1


def _rel(got, ref):
    return P.rel_err_rows(np.asarray(got, dtype=np.float64).reshape(len(ref), -1), np.asarray(ref).reshape(len(ref), -1))


def _scaled(got, ref):
    ref = np.asarray(ref, dtype=np.float64)
    return np.abs(np.asarray(got, dtype=np.float64) - ref).max() / max(np.abs(ref).max(), 1e-30)


def _train_forward(cfg, inp):
    d = M.dims_from_config(cfg)
    buf = M.MoELayerBuffers(d, device="cuda", logits=True)
    P_ = cfg.T * cfg.top_k
    pre = torch.empty((P_, _nm(cfg) * cfg.F), dtype=torch.bfloat16, device="cuda")
    M.moe_route(d, inp["x"], inp["w_gate"], inp["bias"], buf.topk_idx, buf.topk_gate, buf.logits)
    M.moe_dispatch_layout(d, buf.topk_idx, buf.expert_counts, buf.expert_offsets, buf.rank_counts, buf.rank_offsets,
                          buf.pair_to_row, buf.row_to_pair, buf.layout_ws)
    M.moe_permute(d, inp["x"], buf.pair_to_row, buf.x_perm)
    M.moe_expert_ffn_up_train(d, buf.x_perm, buf.expert_offsets, inp["w1"], inp["w3"], buf.h, pre)
    M.moe_expert_ffn_down(d, buf.h, buf.expert_offsets, inp["w2"], buf.y_perm)
    M.moe_unpermute_combine(d, buf.y_perm, buf.pair_to_row, buf.topk_gate, buf.y)
    return d, buf, pre


@needs_gpu
@pytest.mark.parametrize("name", list(CASES))
def test_backward_stages(name):
    cfg = CASES[name]
    print(f"[backward] {name}: {cfg}", flush=True)
    T, D, E, k, F = cfg.T, cfg.D, cfg.E, cfg.top_k, cfg.F
    nm = _nm(cfg)
    inp = W.make_inputs(cfg, "cuda")
    host = P.to_host(inp)
    d, buf, pre = _train_forward(cfg, inp)
    torch.cuda.synchronize()
    # the training forward's h equals the plain forward's, and pre holds the GEMM pre-activations
    h_plain = torch.empty_like(buf.h)
    M.moe_expert_ffn_up(d, buf.x_perm, buf.expert_offsets, inp["w1"], inp["w3"], h_plain)
    torch.cuda.synchronize()
    N = int(buf.expert_offsets[-1])
    assert torch.equal(h_plain[:N], buf.h[:N]), "h of the training forward"
    off = P.i64(buf.expert_offsets)
    xp = P.f64(buf.x_perm[:N])
    experts = np.searchsorted(off, np.arange(N), side="right") - 1
    a1_ref = np.zeros((N, F))
    a3_ref = np.zeros((N, F))
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        if hi > lo:
            a1_ref[lo:hi] = xp[lo:hi] @ O.as_f64(host["w1"][e]).T
            if nm == 2:
                a3_ref[lo:hi] = xp[lo:hi] @ O.as_f64(host["w3"][e]).T
    pre_h = P.f64(pre[:N])
    assert _rel(pre_h[:, :F], a1_ref).max() <= TOL_ROW, "pre-activation W1 x"
    if nm == 2:
        assert _rel(pre_h[:, F:], a3_ref).max() <= TOL_ROW, "pre-activation W3 x"

    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    dy = torch.randn((T, D), generator=g, device="cuda").to(torch.bfloat16)
    dyh = P.f64(dy)
    Pn = T * k
    dy_perm = torch.empty((Pn, D), dtype=torch.bfloat16, device="cuda")
    dgate = torch.empty(Pn, dtype=torch.float32, device="cuda")
    M.moe_backward_combine(d, dy, buf.pair_to_row, buf.topk_gate, buf.y_perm, dy_perm, dgate)
    w13t = torch.empty((E, D, nm * F), dtype=torch.bfloat16, device="cuda")
    w2t = torch.empty((E, F, D), dtype=torch.bfloat16, device="cuda")
    M.moe_transpose_weights(d, inp["w1"], inp["w3"], inp["w2"], w13t, w2t)
    da = torch.empty((Pn, nm * F), dtype=torch.bfloat16, device="cuda")
    M.moe_expert_ffn_down_backward(d, dy_perm, buf.expert_offsets, w2t, pre, da)
    dx_perm = torch.empty((Pn, D), dtype=torch.bfloat16, device="cuda")
    M.moe_expert_ffn_up_backward(d, da, buf.expert_offsets, w13t, dx_perm)
    dl = torch.empty((T, E), dtype=torch.float32, device="cuda")
    dwg = torch.empty((E, D), dtype=torch.float32, device="cuda")
    dbias = torch.empty(E, dtype=torch.float32, device="cuda")
    ws = torch.empty(M.moe_workspace_size(d, M.MOE_STAGE_ROUTER_BWD), dtype=torch.uint8, device="cuda")
    M.moe_router_backward(d, inp["x"], buf.logits, buf.topk_idx, buf.topk_gate, dgate, dl, dwg, dbias, ws)
    # the expert-grouped dW_g, on a dropless layout of the same selection (the forward's own when dropless)
    if cfg.capacity_factor > 0:
        dd = M.dims_from_config(cfg.replace(capacity_factor=0.0))
        lb = M.MoELayerBuffers(dd, device="cuda")
        M.moe_dispatch_layout(dd, buf.topk_idx, lb.expert_counts, lb.expert_offsets, lb.rank_counts, lb.rank_offsets,
                              lb.pair_to_row, lb.row_to_pair, lb.layout_ws)
        all_off, all_r2p = lb.expert_offsets, lb.row_to_pair
    else:
        all_off, all_r2p = buf.expert_offsets, buf.row_to_pair
    dl2 = torch.empty_like(dl)
    dwg2 = torch.empty_like(dwg)
    M.moe_router_backward(d, inp["x"], buf.logits, buf.topk_idx, buf.topk_gate, dgate, dl2, dwg2, None, None,
                          all_expert_offsets=all_off, all_row_to_pair=all_r2p)
    dx = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")
    M.moe_backward_dx(d, dx_perm, buf.pair_to_row, buf.topk_idx, dl, inp["w_gate"], dx)
    torch.cuda.synchronize()

    # weight transposes: bit for bit
    assert torch.equal(w2t, inp["w2"].transpose(1, 2))
    assert torch.equal(w13t[:, :, :F], inp["w1"].transpose(1, 2))
    if nm == 2:
        assert torch.equal(w13t[:, :, F:], inp["w3"].transpose(1, 2))

    # dy_perm, dgate on the GPU's saved tensors
    p2r = P.i64(buf.pair_to_row)
    r2p = P.i64(buf.row_to_pair)[:N]
    gates = P.f64(buf.topk_gate)
    tok = r2p // k
    dyp_ref = gates[r2p][:, None] * dyh[tok]
    assert _rel(P.f64(dy_perm[:N]), dyp_ref).max() <= TOL_ROW, "dy_perm"
    yp = P.f64(buf.y_perm[:N])
    dgate_ref = np.zeros(Pn)
    dgate_ref[r2p] = (dyh[tok] * yp).sum(axis=1)
    scale = (np.abs(dyh[tok]) * np.abs(yp)).sum(axis=1)
    dg = P.f64(dgate)
    assert np.all(np.abs(dg[r2p] - dgate_ref[r2p]) <= 1e-5 * scale + 1e-30), "dgate"
    assert np.all(dg[p2r < 0] == 0), "dgate of dropped pairs"

    # da from the GPU's dy_perm and pre
    dyp_h = P.f64(dy_perm[:N])
    dh = np.zeros((N, F))
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        if hi > lo:
            dh[lo:hi] = dyp_h[lo:hi] @ O.as_f64(host["w2"][e])
    a1 = pre_h[:, :F]
    if nm == 2:
        a3 = pre_h[:, F:]
        da_ref = np.concatenate([dh * a3 * O.silu_grad(a1), dh * O.silu(a1)], axis=1)
    else:
        da_ref = dh * O.gelu_grad(a1)
    assert _rel(P.f64(da[:N]), da_ref).max() <= TOL_ROW, "da (activation backward)"

    # dx_perm from the GPU's da
    da_h = P.f64(da[:N])
    dxp_ref = np.zeros((N, D))
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        if hi > lo:
            dxp_ref[lo:hi] = da_h[lo:hi, :F] @ O.as_f64(host["w1"][e])
            if nm == 2:
                dxp_ref[lo:hi] += da_h[lo:hi, F:] @ O.as_f64(host["w3"][e])
    assert _rel(P.f64(dx_perm[:N]), dxp_ref).max() <= TOL_ROW, "dx_perm"

    # router: dl from the GPU's logits, selection, gates... and dgate
    l_gpu = P.f64(buf.logits).reshape(T, E)
    idx = P.i64(buf.topk_idx).reshape(T, k)
    dl_ref = O.gate_weights_backward(l_gpu, idx, cfg.gate, dg.reshape(T, k))
    assert _scaled(P.f64(dl), dl_ref) <= TOL_F32, "dl"
    dl_h = P.f64(dl)
    xh = O.as_f64(host["x"])
    assert _scaled(P.f64(dwg), dl_h.T @ xh) <= TOL_F32, "dW_g"
    assert torch.equal(dl2, dl), "dl does not depend on the dW_g form"
    assert _scaled(P.f64(dwg2), dl_h.T @ xh) <= TOL_F32, "dW_g grouped by expert"
    assert _scaled(P.f64(dbias), dl_h.sum(axis=0)) <= TOL_F32, "dbias"

    # dx from the GPU's dx_perm and dl
    dxp_h = P.f64(dx_perm[:N])
    dx_ref = np.zeros((T, D))
    np.add.at(dx_ref, tok, dxp_h)
    dx_ref += dl_h @ O.as_f64(host["w_gate"])
    assert _rel(P.f64(dx), dx_ref).max() <= TOL_ROW, "dx"

    # transposes of the wgrad operands: bit for bit against torch, zero padding between groups
    ld = M.moe_wgrad_ld(d)
    koff = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    tr = {}
    for key, src, C in (("dyp", dy_perm, D), ("h", buf.h, F), ("da", da, nm * F), ("xp", buf.x_perm, D)):
        dst = torch.full((C, ld), 7.0, dtype=torch.bfloat16, device="cuda")
        M.moe_group_transpose(d, src, C, buf.expert_offsets, koff, dst)
        tr[key] = dst
    torch.cuda.synchronize()
    kh = P.i64(koff)
    assert kh[0] == 0 and np.all(np.diff(kh) == (np.diff(off) + 63) // 64 * 64)
    for key, src, C in (("dyp", dy_perm, D), ("h", buf.h, F), ("da", da, nm * F), ("xp", buf.x_perm, D)):
        for e in range(E):
            lo, hi = int(off[e]), int(off[e + 1])
            got = tr[key][:, kh[e]:kh[e + 1]]
            assert torch.equal(got[:, :hi - lo], src[lo:hi].t()), f"transpose {key} expert {e}"
            assert bool((got[:, hi - lo:] == 0).all()), f"padding {key} expert {e}"

    # weight gradients
    dw2 = torch.empty((E, D, F), dtype=torch.float32, device="cuda")
    M.moe_expert_wgrad(d, tr["dyp"], tr["h"], koff, D, F, dw2)
    dw1 = torch.empty((E, F, D), dtype=torch.float32, device="cuda")
    dw3 = torch.empty((E, F, D), dtype=torch.float32, device="cuda") if nm == 2 else None
    M.moe_expert_wgrad(d, tr["da"], tr["xp"], koff, nm * F, D, dw1, dw3, split=F)
    torch.cuda.synchronize()
    h_h = P.f64(buf.h[:N])
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        ref2 = dyp_h[lo:hi].T @ h_h[lo:hi]
        ref1 = da_h[lo:hi, :F].T @ xp[lo:hi]
        if hi == lo:
            assert bool((dw2[e] == 0).all()) and bool((dw1[e] == 0).all()), f"expert {e} without rows"
            continue
        assert _scaled(P.f64(dw2[e]), ref2) <= TOL_F32, f"dW2 expert {e}"
        assert _scaled(P.f64(dw1[e]), ref1) <= TOL_F32, f"dW1 expert {e}"
        if nm == 2:
            assert _scaled(P.f64(dw3[e]), da_h[lo:hi, F:].T @ xp[lo:hi]) <= TOL_F32, f"dW3 expert {e}"

    # The pinned oracle as the checker: O.layer_backward on a forward record that holds the GPU's own
    # routing, layout, logits, x_perm and y_perm (staged), so every token compares, drops included.
    fwd_g = {"pair_to_row": p2r, "row_to_pair": P.i64(buf.row_to_pair), "expert_offsets": off,
             "topk_gate": gates.reshape(T, k), "topk_idx": idx, "logits": l_gpu,
             "y_perm": P.f64(buf.y_perm), "x_perm": P.f64(buf.x_perm)}
    ob = O.layer_backward(host, cfg, fwd_g, dyh)
    errs = {"dy_perm": _rel(dyp_h, ob["dy_perm"]).max(),
            "da1": _rel(da_h[:, :F], ob["da1"]).max(),
            "dx_perm": _rel(dxp_h, ob["dx_perm"]).max(),
            "dx": _rel(P.f64(dx), ob["dx"]).max(),
            "dgate": _scaled(dg.reshape(T, k)[p2r.reshape(T, k) >= 0], ob["dgate"][p2r.reshape(T, k) >= 0]),
            "dl": _scaled(dl_h, ob["dl"]), "dw_gate": _scaled(P.f64(dwg), ob["dw_gate"]),
            "dbias": _scaled(P.f64(dbias), ob["dbias"])}
    if nm == 2:
        errs["da3"] = _rel(da_h[:, F:], ob["da3"]).max()
    for key in ("dy_perm", "da1", "da3", "dx_perm", "dx"):
        if key in errs:
            assert errs[key] <= TOL_ROW, f"{key} vs the oracle's backward: {errs[key]:.3e}"
    for key in ("dgate", "dl", "dw_gate", "dbias"):
        assert errs[key] <= TOL_F32, f"{key} vs the oracle's backward: {errs[key]:.3e}"
    # weight gradients element by element: |got - ref| <= TOL_WG_SUM * (M^T |B|), M the first-order
    # magnitude of the GPU's rounding perturbations of the left operand (_perturbation_scale), B the
    # right operand (h for dW2, x_perm for dW1/dW3); and within TOL_WG of the expert's largest entry
    wg_err = 0.0
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        m2, m1, m3 = _perturbation_scale(ob, host, cfg, e, lo, hi)
        pairs = [("dw2", dw2[e], ob["dw2"][e], m2, ob["h"][lo:hi]),
                 ("dw1", dw1[e], ob["dw1"][e], m1, xp[lo:hi])]
        if nm == 2:
            pairs.append(("dw3", dw3[e], ob["dw3"][e], m3, xp[lo:hi]))
        for key, got, ref, A, B in pairs:
            got = P.f64(got)
            bound = TOL_WG_SUM * (A.T @ np.abs(B))
            assert np.all(np.abs(got - ref) <= bound + 1e-30), f"{key} expert {e} vs the oracle: elementwise bound"
            sc = _scaled(got, ref)
            assert sc <= TOL_WG, f"{key} expert {e} vs the oracle's backward: {sc:.3e}"
            wg_err = max(wg_err, sc)
    print(f"[backward] {name}: vs O.layer_backward " + ", ".join(f"{k_} {v:.1e}" for k_, v in errs.items())
          + f", weight gradients {wg_err:.1e}", flush=True)

    # end to end: dx against the oracle's own float64 forward + backward on decisive tokens (dropless)
    if cfg.capacity_factor <= 0:
        fwd = O.layer_forward(host, cfg)
        bwd = O.layer_backward(host, cfg, fwd, dyh)
        dec = O.decisive_tokens(fwd["logits"], k, 1e-3, cfg.n_groups, cfg.topk_groups, cfg.gate)["order"]
        same = (fwd["topk_idx"] == idx).all(axis=1) & dec
        assert same.mean() > 0.5
        err = P.rel_err_rows(P.f64(dx)[same], bwd["dx"][same])
        assert err.max() <= TOL_ROW, f"dx end to end: max rel err {err.max():.3e}"
        print(f"[backward] {name}: dx end-to-end max rel err {err.max():.2e} on {same.sum()} tokens", flush=True)


@needs_gpu
@pytest.mark.parametrize("name", ["dsv3_small", "gelu_k1_bias", "capacity"])
def test_native_backward_equals_the_steps(name):
    """moe_layer_backward (one call) gives the same bits as the step entry points called in order."""
    cfg = CASES[name]
    inp = W.make_inputs(cfg, "cuda")
    d = M.dims_from_config(cfg)
    buf = M.MoELayerBuffers(d, device="cuda", logits=True)
    bw = M.BackwardBuffers(d, device="cuda", transposed=True)
    M.forward_train(buf, bw, inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"])
    g = torch.Generator(device="cuda")
    g.manual_seed(9)
    dy = torch.randn((cfg.T, cfg.D), generator=g, device="cuda").to(torch.bfloat16)
    M.backward(buf, bw, inp["x"], inp["w_gate"], dy, transpose_weights=(inp["w1"], inp["w3"], inp["w2"]))
    torch.cuda.synchronize()
    native = {n: getattr(bw, n).clone() for n in ("dx", "dw_gate", "dbias", "dw1", "dw2", "dl", "dgate")}
    if bw.dw3 is not None:
        native["dw3"] = bw.dw3.clone()
    # the same steps, one entry point at a time
    nm = 2 if cfg.act == W.ACT_SWIGLU else 1
    M.moe_backward_combine(d, dy, buf.pair_to_row, buf.topk_gate, buf.y_perm, bw.dy_perm, bw.dgate)
    M.moe_expert_ffn_down_backward(d, bw.dy_perm, buf.expert_offsets, bw.w2t, bw.pre, bw.da)
    M.moe_expert_ffn_up_backward(d, bw.da, buf.expert_offsets, bw.w13t, bw.dx_perm)
    grouped = dict(all_expert_offsets=buf.expert_offsets, all_row_to_pair=buf.row_to_pair) \
        if cfg.capacity_factor <= 0 else {}
    M.moe_router_backward(d, inp["x"], buf.logits, buf.topk_idx, buf.topk_gate, bw.dgate, bw.dl, bw.dw_gate, bw.dbias,
                          bw.router_ws, **grouped)
    M.moe_backward_dx(d, bw.dx_perm, buf.pair_to_row, buf.topk_idx, bw.dl, inp["w_gate"], bw.dx)
    M.moe_group_transpose(d, bw.dy_perm, cfg.D, buf.expert_offsets, bw.koff, bw.dyp_t)
    M.moe_group_transpose(d, buf.h, cfg.F, buf.expert_offsets, bw.koff, bw.h_t)
    M.moe_expert_wgrad(d, bw.dyp_t, bw.h_t, bw.koff, cfg.D, cfg.F, bw.dw2)
    M.moe_group_transpose(d, bw.da, nm * cfg.F, buf.expert_offsets, bw.koff, bw.da_t)
    M.moe_group_transpose(d, buf.x_perm, cfg.D, buf.expert_offsets, bw.koff, bw.xp_t)
    M.moe_expert_wgrad(d, bw.da_t, bw.xp_t, bw.koff, nm * cfg.F, cfg.D, bw.dw1, bw.dw3, split=cfg.F)
    torch.cuda.synchronize()
    for n, v in native.items():
        assert torch.equal(getattr(bw, n), v), f"{n}: native executor differs from the steps"
