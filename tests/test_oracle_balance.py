"""Pins for the oracle's load-balancing pieces: router probabilities, the auxiliary loss, the
selection-only bias and its update rule.

Checked against hand-worked values, closed forms (balanced and collapsed routing), a library
softmax, and a behavioural property the pages state: repeated bias updates even out the load.
"""
import numpy as np
import pytest
from scipy.special import softmax as scipy_softmax

import oracle as O


def test_router_probabilities_softmax_is_library_softmax():
    rng = np.random.default_rng(3)
    l = rng.standard_normal((9, 13)) * 3
    for gate in (O.GATE_SOFTMAX_TOPK, O.GATE_SOFTMAX_FULL):
        np.testing.assert_allclose(O.router_probabilities(l, gate), scipy_softmax(l, axis=1), rtol=1e-13, atol=0)


def test_router_probabilities_sigmoid_hand_example():
    # sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4 -> normalised [0.4, 0.6]
    p = O.router_probabilities(np.array([[0.0, np.log(3.0)]]), O.GATE_SIGMOID_TOPK)
    np.testing.assert_allclose(p, [[0.4, 0.6]], rtol=1e-15)


def test_aux_loss_hand_example():
    # E=2, T=2, k=2: counts [3,1] -> f = [3/4, 1/4]; P = [0.7, 0.3]
    # L = 0.01 * 2 * (0.75*0.7 + 0.25*0.3) = 0.012; imbalance = 3 / 2
    probs = np.array([[0.9, 0.1], [0.5, 0.5]])
    st = O.load_balance_stats(np.array([3, 1]), probs, k=2, alpha=0.01)
    np.testing.assert_allclose(st["f"], [0.75, 0.25])
    np.testing.assert_allclose(st["P"], [0.7, 0.3])
    assert st["aux_loss"] == pytest.approx(0.012, rel=1e-14)
    assert st["imbalance"] == pytest.approx(1.5)


@pytest.mark.parametrize("E,k", [(8, 2), (64, 8), (5, 1)])
def test_aux_loss_closed_forms_balanced_and_collapsed(E, k):
    T = 10 * E
    alpha = 0.37
    # perfectly even routing and uniform probabilities: f_i = P_i = 1/E, so L = alpha
    st = O.load_balance_stats(np.full(E, T * k // E), np.full((T, E), 1.0 / E), k, alpha)
    assert st["aux_loss"] == pytest.approx(alpha, rel=1e-12)
    assert st["imbalance"] == pytest.approx(1.0)
    # every pair to expert 0 with all probability on it: f_0 = P_0 = 1, so L = alpha * E
    c = np.zeros(E, dtype=np.int64)
    c[0] = T * k
    p = np.zeros((T, E))
    p[:, 0] = 1.0
    st = O.load_balance_stats(c, p, k, alpha)
    assert st["aux_loss"] == pytest.approx(alpha * E, rel=1e-12)
    assert st["imbalance"] == pytest.approx(E)


def test_fractions_sum_to_one_on_a_routed_batch():
    rng = np.random.default_rng(5)
    T, D, E, k = 200, 16, 12, 3
    x, wg = rng.standard_normal((T, D)), rng.standard_normal((E, D))
    r = O.route(x, wg, None, k, O.GATE_SOFTMAX_TOPK)
    lay = O.dispatch_layout(r["topk_idx"], E, 1)
    st = O.load_balance_stats(lay["expert_counts"], O.router_probabilities(r["logits"], O.GATE_SOFTMAX_TOPK), k, 1.0)
    assert st["f"].sum() == pytest.approx(1.0, rel=1e-14)
    assert st["P"].sum() == pytest.approx(1.0, rel=1e-14)


def test_bias_update_hand_example():
    # loads [5,3,4]: mean 4 -> over, under, exact -> bias moves by [-g, +g, 0]
    b = O.update_select_bias(np.array([0.0, 0.25, -1.0], dtype=np.float32), np.array([5, 3, 4]), 0.125)
    assert b.dtype == np.float32
    assert b.tolist() == [-0.125, 0.375, -1.0]


def test_zero_select_bias_changes_nothing():
    rng = np.random.default_rng(6)
    T, D, E, k = 50, 8, 16, 4
    x, wg = rng.standard_normal((T, D)), rng.standard_normal((E, D))
    for gate in (O.GATE_SOFTMAX_TOPK, O.GATE_SIGMOID_TOPK):
        for ng, tg in ((0, 0), (4, 2)):
            a = O.route(x, wg, None, k, gate, ng, tg)
            b = O.route(x, wg, None, k, gate, ng, tg, select_bias=np.zeros(E, dtype=np.float32))
            np.testing.assert_array_equal(a["topk_idx"], b["topk_idx"])
            np.testing.assert_array_equal(a["topk_gate"], b["topk_gate"])


def test_select_bias_moves_selection_not_gates():
    rng = np.random.default_rng(7)
    T, D, E = 40, 8, 6
    x, wg = rng.standard_normal((T, D)), rng.standard_normal((E, D))
    sb = np.zeros(E, dtype=np.float32)
    sb[4] = 100.0
    # a huge bias puts expert 4 in slot 0 of every token
    r = O.route(x, wg, None, 2, O.GATE_SOFTMAX_TOPK, select_bias=sb)
    assert (r["topk_idx"][:, 0] == 4).all()
    # with k = E every expert is kept, only the slot order moves: each expert's gate is unchanged
    a = O.route(x, wg, None, E, O.GATE_SOFTMAX_TOPK)
    b = O.route(x, wg, None, E, O.GATE_SOFTMAX_TOPK, select_bias=sb)
    ga = np.zeros((T, E))
    gb = np.zeros((T, E))
    np.put_along_axis(ga, a["topk_idx"], a["topk_gate"], axis=1)
    np.put_along_axis(gb, b["topk_idx"], b["topk_gate"], axis=1)
    np.testing.assert_allclose(ga, gb, rtol=1e-14, atol=0)


def test_sigmoid_select_bias_adds_to_the_score_not_the_logit():
    # logits [2, 0]: scores sigmoid = [0.8808, 0.5]. Bias [0, 0.4] on the score gives keys
    # [0.8808, 0.9] -> expert 1 first; the same bias on the logit would keep expert 0 first.
    x = np.array([[1.0]])
    wg = np.array([[2.0], [0.0]])
    sb = np.array([0.0, 0.4], dtype=np.float32)
    r = O.route(x, wg, None, 1, O.GATE_SIGMOID_TOPK, select_bias=sb)
    assert r["topk_idx"].tolist() == [[1]]
    r2 = O.route(x, wg, None, 2, O.GATE_SIGMOID_TOPK, select_bias=sb)
    s0, s1 = 1 / (1 + np.exp(-2.0)), 0.5
    assert r2["topk_idx"].tolist() == [[1, 0]]
    np.testing.assert_allclose(r2["topk_gate"], [[s1 / (s0 + s1), s0 / (s0 + s1)]], rtol=1e-15)


@pytest.mark.parametrize("gate", [O.GATE_SOFTMAX_TOPK, O.GATE_SIGMOID_TOPK])
def test_repeated_bias_updates_even_out_the_load(gate):
    # Router skew: a logit tilt makes expert 0 take several times its share. Updating the
    # selection bias by the sign rule pulls the load back towards even; a wrong sign would
    # make it worse.
    rng = np.random.default_rng(11)
    T, D, E, k = 2048, 16, 16, 2
    x = rng.standard_normal((T, D))
    wg = rng.standard_normal((E, D)) * 0.3
    tilt = -0.6 * np.log(np.arange(E) + 1.0)
    sb = np.zeros(E, dtype=np.float32)
    gamma = 0.02 if gate == O.GATE_SIGMOID_TOPK else 0.05
    imb = []
    for _ in range(60):
        r = O.route(x, wg, tilt, k, gate, select_bias=sb)
        c = O.dispatch_layout(r["topk_idx"], E, 1)["expert_counts"]
        imb.append(c.max() / c.mean())
        sb = O.update_select_bias(sb, c, gamma)
    assert imb[0] > 2.5
    assert max(imb[-10:]) < 1.35
