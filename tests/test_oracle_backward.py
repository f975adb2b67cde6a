"""Pins for the oracle's layer backward: central finite differences of the float64 forward.

L = sum(y * dy) for a fixed random dy; every gradient entry is compared with
(L(theta + eps) - L(theta - eps)) / (2 eps), the routing decision (which the backward holds fixed)
checked unchanged under each perturbation. Covers all three gate modes, both activations, a group
limit, a capacity with drops and a router bias; plus closed forms (k = 1 softmax gates carry no
router gradient; the dense one-expert case).
"""
import numpy as np
import pytest

import oracle as O
import workloads as W

EPS = 1e-6


def _inputs(cfg, seed):
    rng = np.random.default_rng(seed)
    inp = {
        "x": rng.standard_normal((cfg.T, cfg.D)),
        "w_gate": rng.standard_normal((cfg.E, cfg.D)) * 0.7,
        "bias": rng.standard_normal(cfg.E) * 0.3 if cfg.bias != "none" else None,
        "w1": rng.standard_normal((cfg.E, cfg.F, cfg.D)) * 0.5,
        "w3": rng.standard_normal((cfg.E, cfg.F, cfg.D)) * 0.5 if cfg.act == W.ACT_SWIGLU else None,
        "w2": rng.standard_normal((cfg.E, cfg.D, cfg.F)) * 0.5,
    }
    dy = rng.standard_normal((cfg.T, cfg.D))
    return inp, dy


def _loss(inp, cfg, dy):
    f = O.layer_forward(inp, cfg)
    return float((f["y"] * dy).sum()), f["topk_idx"].copy(), f["pair_to_row"].copy()


CFGS = {
    "softmax_swiglu": W.MoEConfig(name="a", T=6, D=5, E=4, top_k=2, F=3, dtype=W.DT_F32),
    "sigmoid_groups": W.MoEConfig(name="b", T=5, D=4, E=6, top_k=2, F=3, dtype=W.DT_F32, gate=W.GATE_SIGMOID_TOPK,
                                  n_groups=3, topk_groups=2),
    "full_softmax_gelu": W.MoEConfig(name="c", T=5, D=4, E=5, top_k=3, F=2, dtype=W.DT_F32, act=W.ACT_GELU,
                                     gate=W.GATE_SOFTMAX_FULL, bias="normal0.5"),
    "capacity_drops": W.MoEConfig(name="d", T=8, D=3, E=3, top_k=2, F=2, dtype=W.DT_F32, capacity_factor=0.5,
                                  bias="normal0.5"),
}
PARAMS = ["x", "w_gate", "bias", "w1", "w3", "w2"]
GRAD = {"x": "dx", "w_gate": "dw_gate", "bias": "dbias", "w1": "dw1", "w3": "dw3", "w2": "dw2"}


@pytest.mark.parametrize("name", list(CFGS))
def test_backward_matches_central_differences(name):
    cfg = CFGS[name]
    inp, dy = _inputs(cfg, seed=len(name))
    fwd = O.layer_forward(inp, cfg)
    if cfg.capacity_factor > 0:
        assert (fwd["pair_to_row"] < 0).any(), "the capacity case must drop something"
    g = O.layer_backward(inp, cfg, fwd, dy)
    for pname in PARAMS:
        if inp[pname] is None:
            continue
        base = inp[pname]
        num = np.zeros_like(base)
        for i in np.ndindex(base.shape):
            hi = dict(inp)
            lo = dict(inp)
            hi[pname] = base.copy()
            lo[pname] = base.copy()
            hi[pname][i] += EPS
            lo[pname][i] -= EPS
            lp, idx_p, p2r_p = _loss(hi, cfg, dy)
            lm, idx_m, p2r_m = _loss(lo, cfg, dy)
            assert np.array_equal(idx_p, fwd["topk_idx"]) and np.array_equal(idx_m, fwd["topk_idx"])
            assert np.array_equal(p2r_p, fwd["pair_to_row"]) and np.array_equal(p2r_m, fwd["pair_to_row"])
            num[i] = (lp - lm) / (2 * EPS)
        np.testing.assert_allclose(g[GRAD[pname]], num, rtol=2e-6, atol=2e-7, err_msg=pname)


def test_k1_softmax_gates_carry_no_router_gradient():
    cfg = W.MoEConfig(name="e", T=7, D=4, E=5, top_k=1, F=3, dtype=W.DT_F32, act=W.ACT_GELU)
    inp, dy = _inputs(cfg, seed=3)
    fwd = O.layer_forward(inp, cfg)
    g = O.layer_backward(inp, cfg, fwd, dy)
    assert np.all(g["dl"] == 0) and np.all(g["dw_gate"] == 0)      # g = softmax of one logit = 1


def test_dense_one_expert_closed_form():
    # E = 1, k = 1: y = W2 GELU(W1 x); dW2 = dy^T h, dW1 = (dy W2 * GELU'(a))^T x, dx = (dy W2 * GELU'(a)) W1
    cfg = W.MoEConfig(name="f", T=9, D=4, E=1, top_k=1, F=3, dtype=W.DT_F32, act=W.ACT_GELU)
    inp, dy = _inputs(cfg, seed=4)
    fwd = O.layer_forward(inp, cfg)
    g = O.layer_backward(inp, cfg, fwd, dy)
    x, w1, w2 = inp["x"], inp["w1"][0], inp["w2"][0]
    a = x @ w1.T
    h = O.gelu(a)
    da = (dy @ w2) * O.gelu_grad(a)
    np.testing.assert_allclose(g["dw2"][0], dy.T @ h, rtol=1e-13)
    np.testing.assert_allclose(g["dw1"][0], da.T @ x, rtol=1e-13)
    np.testing.assert_allclose(g["dx"], da @ w1, rtol=1e-12, atol=1e-14)


def test_activation_derivatives_against_differences():
    a = np.linspace(-6, 6, 97)
    for f, df in ((O.silu, O.silu_grad), (O.gelu, O.gelu_grad)):
        num = (f(a + 1e-6) - f(a - 1e-6)) / 2e-6
        np.testing.assert_allclose(df(a), num, rtol=1e-7, atol=1e-9)


@pytest.mark.parametrize("mode", [W.GATE_SOFTMAX_TOPK, W.GATE_SIGMOID_TOPK, W.GATE_SOFTMAX_FULL])
def test_gate_weights_backward_against_differences(mode):
    # dl[t, e] = sum_j dgate[t, j] * d g[t, j] / d l[t, e] with the selection held fixed, each
    # derivative by a central difference of gate_weights itself (no layer around it)
    rng = np.random.default_rng(11 + mode)
    T, E, k = 5, 7, 3
    l = rng.normal(0.0, 1.5, (T, E))
    idx = np.argsort(-l, axis=1)[:, :k]
    dg = rng.normal(0.0, 1.0, (T, k))
    got = O.gate_weights_backward(l, idx, mode, dg)
    eps = 1e-6
    want = np.zeros((T, E))
    for e in range(E):
        lp, lm = l.copy(), l.copy()
        lp[:, e] += eps
        lm[:, e] -= eps
        want[:, e] = ((O.gate_weights(lp, idx, mode) - O.gate_weights(lm, idx, mode)) * dg).sum(axis=1) / (2 * eps)
    np.testing.assert_allclose(got, want, rtol=1e-7, atol=1e-9)
    if mode != W.GATE_SOFTMAX_FULL:
        # only the selected logits move renormalised top-k gates
        unsel = np.ones((T, E), dtype=bool)
        np.put_along_axis(unsel, idx, False, axis=1)
        assert np.all(got[unsel] == 0)
