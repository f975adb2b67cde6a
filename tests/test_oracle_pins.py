"""Pins for the CPU oracle: page-printed examples, closed forms, invariants, brute force.

Each test checks the oracle against something other than itself: a value a
page prints (fixtures under tests/golden/), a closed form worked by hand, an
independent formulation (rank counting, Python ``sorted``), or an invariant
the pages state. Chosen so that a dropped term, a wrong sign or index, or a
transposed operand in the oracle fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------------------------------------
# Router logits
# ------------------------------------------------------------------------------------------------

def test_logits_hand_example():
    # x=[1,2], W_g rows [3,4] and [5,6], bias [0.5,-1]: l = [1*3+2*4+0.5, 1*5+2*6-1] = [11.5, 16]
    l = O.route_logits(np.array([[1.0, 2.0]]), np.array([[3.0, 4.0], [5.0, 6.0]]), np.array([0.5, -1.0]))
    assert l.tolist() == [[11.5, 16.0]]


def test_logits_one_hot_rows_pick_router_columns():
    rng = np.random.default_rng(0)
    D, E = 7, 5
    wg = rng.standard_normal((E, D))
    x = np.eye(D)
    l = O.route_logits(x, wg)
    np.testing.assert_array_equal(l, wg.T)     # token d sees column d of W_g, exactly


def test_logits_linear_in_tokens():
    rng = np.random.default_rng(1)
    x1, x2 = rng.standard_normal((3, 6)), rng.standard_normal((3, 6))
    wg = rng.standard_normal((4, 6))
    np.testing.assert_allclose(O.route_logits(x1 + x2, wg), O.route_logits(x1, wg) + O.route_logits(x2, wg),
                               rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------------------------------------
# Selection
# ------------------------------------------------------------------------------------------------

def _topk_by_rank_counting(row, k, eligible=None):
    """Independent formulation: expert e sits in slot r iff exactly r eligible experts beat it,
    where e' beats e when l[e'] > l[e], or l[e'] == l[e] and e' < e."""
    E = len(row)
    elig = [True] * E if eligible is None else list(eligible)
    slots = [None] * k
    for e in range(E):
        if not elig[e]:
            continue
        r = sum(1 for f in range(E) if elig[f] and (row[f] > row[e] or (row[f] == row[e] and f < e)))
        if r < k:
            slots[r] = e
    return slots


def test_topk_hand_example_with_tie():
    l = np.array([[0.1, 0.5, 0.5, -1.0]])
    assert O.select_topk(l, 2).tolist() == [[1, 2]]      # exact tie -> lower index first
    assert O.select_topk(l, 3).tolist() == [[1, 2, 0]]


@settings(max_examples=60, deadline=None)
@given(T=st.integers(1, 6), E=st.integers(1, 9), data=st.data())
def test_topk_matches_rank_counting(T, E, data):
    k = data.draw(st.integers(1, E))
    # small integer logits force many exact ties
    vals = data.draw(st.lists(st.integers(-3, 3), min_size=T * E, max_size=T * E))
    l = np.array(vals, dtype=np.float64).reshape(T, E)
    got = O.select_topk(l, k)
    for t in range(T):
        assert got[t].tolist() == _topk_by_rank_counting(l[t].tolist(), k)


def test_group_limit_hand_example():
    # 8 experts in 4 groups of 2, k=2, one group kept, group score = sum of its top-2 scores:
    # groups 0..3 score 1.0, 1.2, 0.95, 0.6 -> keep group 1 = experts {2,3} (tie -> 2 first).
    s = np.array([[0.9, 0.1, 0.6, 0.6, 0.95, 0.0, 0.3, 0.3]])
    idx, groups = O.select_group_limited(s, 2, 4, 1, s)
    assert groups.tolist() == [[1]]
    assert idx.tolist() == [[2, 3]]
    assert O.select_topk(s, 2).tolist() == [[4, 0]]      # without the limit the choice differs


@settings(max_examples=40, deadline=None)
@given(T=st.integers(1, 4), data=st.data())
def test_group_limit_matches_bruteforce(T, data):
    n_groups = data.draw(st.sampled_from([2, 4]))
    gsize = data.draw(st.sampled_from([2, 3]))
    E = n_groups * gsize
    topk_groups = data.draw(st.integers(1, n_groups))
    per = data.draw(st.integers(1, gsize))
    k = per * topk_groups
    vals = data.draw(st.lists(st.integers(-4, 4), min_size=T * E, max_size=T * E))
    l = np.array(vals, dtype=np.float64).reshape(T, E) / 4.0
    idx, groups = O.select_group_limited(l, k, n_groups, topk_groups, l)
    for t in range(T):
        row = l[t].tolist()
        # group score by Python sorted(): sum of the `per` largest members
        gscore = [sum(sorted(row[g * gsize:(g + 1) * gsize], reverse=True)[:per]) for g in range(n_groups)]
        gscore32 = [float(np.float32(v)) for v in gscore]
        kept = _topk_by_rank_counting(gscore32, topk_groups)
        assert sorted(groups[t].tolist()) == sorted(kept)
        elig = [(e // gsize) in kept for e in range(E)]
        assert idx[t].tolist() == _topk_by_rank_counting(row, k, elig)
        assert len({e // gsize for e in idx[t]}) <= topk_groups


def test_group_limit_with_all_groups_is_plain_topk():
    rng = np.random.default_rng(3)
    l = rng.standard_normal((50, 32))
    idx, _ = O.select_group_limited(l, 8, 8, 8, l)
    np.testing.assert_array_equal(idx, O.select_topk(l, 8))


# ------------------------------------------------------------------------------------------------
# Gates
# ------------------------------------------------------------------------------------------------

def test_softmax_topk_hand_example():
    # logits [0, ln 3]: the top-2 gates are e^{ln3}/(1+3) = 0.75 and 1/4 = 0.25
    l = np.array([[0.0, math.log(3.0)]])
    idx = O.select_topk(l, 2)
    assert idx.tolist() == [[1, 0]]
    np.testing.assert_allclose(O.gate_weights(l, idx, O.GATE_SOFTMAX_TOPK), [[0.75, 0.25]], rtol=1e-15)


def test_sigmoid_topk_hand_example():
    # sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4, normalised: 0.75 and 0.25
    l = np.array([[math.log(3.0), -math.log(3.0)]])
    idx = O.select_topk(l, 2)
    np.testing.assert_allclose(O.gate_weights(l, idx, O.GATE_SIGMOID_TOPK), [[0.75, 0.25]], rtol=1e-15)


def test_softmax_topk_equals_full_softmax_renormalised():
    rng = np.random.default_rng(4)
    l = rng.standard_normal((40, 16)) * 3
    idx = O.select_topk(l, 4)
    g = O.gate_weights(l, idx, O.GATE_SOFTMAX_TOPK)
    p = np.exp(l) / np.exp(l).sum(axis=1, keepdims=True)          # full softmax, unshifted
    sel = np.take_along_axis(p, idx, axis=1)
    np.testing.assert_allclose(g, sel / sel.sum(axis=1, keepdims=True), rtol=1e-12)
    np.testing.assert_allclose(O.gate_weights(l, idx, O.GATE_SOFTMAX_FULL), sel, rtol=1e-12)
    assert np.all(np.diff(g, axis=1) <= 0)                         # slot order = descending gate
    np.testing.assert_allclose(g.sum(axis=1), 1.0, rtol=1e-14)


def test_gates_k1_are_one():
    rng = np.random.default_rng(5)
    l = rng.standard_normal((20, 6))
    idx = O.select_topk(l, 1)
    for mode in (O.GATE_SOFTMAX_TOPK, O.GATE_SIGMOID_TOPK):
        np.testing.assert_array_equal(O.gate_weights(l, idx, mode), np.ones((20, 1)))


def test_decisive_flags_near_ties():
    l = np.array([[3.0, 1.0, 1.0005, -2.0], [3.0, 2.0, 1.0, 0.0], [1.0, 1.0, 0.0, -1.0]])
    d = O.decisive_tokens(l, 2)
    assert d["set"].tolist() == [False, True, True]
    assert d["order"].tolist() == [False, True, False]


# Group-limited decisive flags. 12 experts in 4 contiguous groups of 3, k = 4, 2 groups kept, so a
# group scores the sum of its 2 best members (k / kept groups). Margins are hand-placed so that
# exactly one comparison falls below 1e-3 in each token.
_G = dict(k=4, margin=1e-3, n_groups=4, topk_groups=2)


def test_decisive_group_margin_alone_decides():
    # softmax gating (group scores on logits): groups score 10, 8, 7.9995, 2 -> kept {0, 1}, and the
    # last kept (8) vs first dropped (7.9995) margin is 5e-4; the expert margin inside the kept groups
    # (4th best 3 vs 5th best 0) is 3. Control token: the third group scores 7.998 (margin 2e-3).
    l = np.array([[6, 4, 0, 5, 3, -1, 4.5, 3.4995, -3, 1, 1, -5],
                  [6, 4, 0, 5, 3, -1, 4.5, 3.498, -3, 1, 1, -5]], dtype=np.float64)
    d = O.decisive_tokens(l, gate=O.GATE_SOFTMAX_TOPK, **_G)
    assert d["set"].tolist() == [False, True]
    assert d["order"].tolist() == [False, True]       # top 4 = 6, 5, 4, 3: adjacent margins all 1


def test_decisive_expert_margin_counts_eligible_experts_only():
    # groups score 10, 8, 2, 1 (kept {0, 1}, margin 6).
    # token 0: inside the kept groups the 4th and 5th best logits are 3.0004 and 3 -> not decisive.
    # token 1: the near-tie partner 3.0004 sits in a dropped group (group 2 scores 3.0004 - 5 < 8),
    #          so among eligible experts the 4th vs 5th margin is 3 - 0 = 3 -> decisive.
    l = np.array([[6, 4, 3.0004, 5, 3, -1, 1, 1, 0, 0.5, 0.5, 0],
                  [6, 4, 0, 5, 3, -1, 3.0004, -5, -5, 0.5, 0.5, 0]], dtype=np.float64)
    d = O.decisive_tokens(l, gate=O.GATE_SOFTMAX_TOPK, **_G)
    assert d["set"].tolist() == [False, True]
    # without the group limit token 1 would tie within 4e-4 (4th 3.0004 vs 5th 3)
    assert O.decisive_tokens(l, 4, 1e-3)["set"].tolist() == [False, False]


def test_decisive_group_scores_use_sigmoid_scores_under_sigmoid_gating():
    # logits per group: [10, 9, 0], [6, 6, 5.9996], [20, 2, -3], [-1, -1, -2]
    # sigmoid group scores (sum of the 2 best sigmoids) 1.99983, 1.99505, 1.88080, 0.53788 -> keep {0, 1};
    #   eligible logits 10, 9, 6, 6, 5.9996 -> 4th vs 5th margin 4e-4 -> not decisive
    # logit group scores 19, 12, 22, -2 -> keep {2, 0}; eligible 20, 10, 9, 2, 0 -> decisive
    l = np.array([[10, 9, 0, 6, 6, 5.9996, 20, 2, -3, -1, -1, -2]], dtype=np.float64)
    sig = 1.0 / (1.0 + np.exp(-l))
    _, kept_sig = O.select_group_limited(l, 4, 4, 2, sig)
    _, kept_log = O.select_group_limited(l, 4, 4, 2, l)
    assert kept_sig.tolist() == [[0, 1]] and kept_log.tolist() == [[2, 0]]
    assert O.decisive_tokens(l, gate=O.GATE_SIGMOID_TOPK, **_G)["set"].tolist() == [False]
    assert O.decisive_tokens(l, gate=O.GATE_SOFTMAX_TOPK, **_G)["set"].tolist() == [True]
    # a sigmoid near-tie between groups that is wide in logit space: [8, 8] vs [7.5, 9.5] score
    # 1.999329 vs 1.999372 as sigmoids (4.3e-5 apart), 16 vs 17 as logits
    l2 = np.array([[10, 9, 0, 8, 8, 0, 7.5, 9.5, 0, -1, -1, -2]], dtype=np.float64)
    assert O.decisive_tokens(l2, gate=O.GATE_SIGMOID_TOPK, **_G)["set"].tolist() == [False]
    assert O.decisive_tokens(l2, gate=O.GATE_SOFTMAX_TOPK, **_G)["set"].tolist() == [True]


@pytest.mark.parametrize("gate", [O.GATE_SOFTMAX_TOPK, O.GATE_SIGMOID_TOPK])
def test_decisive_tokens_keep_their_selection_under_perturbation(gate):
    # Brute force: a token flagged decisive must select the same experts (and, when flagged for order,
    # in the same slots) after any perturbation of its logits by at most margin/8. That moves a
    # difference of two logits by at most margin/4 and a difference of two group scores (each a sum of
    # two members) by at most margin/2; a sigmoid moves by at most a quarter of its argument's change.
    rng = np.random.default_rng(21)
    T, E, k, ng, tg, margin = 300, 12, 4, 4, 2, 1e-3
    # logits on a 5e-4 grid in a narrow range: many comparisons sit at 0, 5e-4 or 1e-3 apart
    l = rng.integers(-6, 7, size=(T, E)) * 5e-4 + rng.integers(-1, 2, size=(T, E)) * 0.01
    d = O.decisive_tokens(l, k, margin, ng, tg, gate)
    assert 0.05 < d["set"].mean() < 0.95                 # both kinds are present

    def sel(v):
        score = 1.0 / (1.0 + np.exp(-v)) if gate == O.GATE_SIGMOID_TOPK else v
        # selection in float64 (no float32 rounding) so that only the perturbation moves it
        gs = O.group_scores(score, ng, k // tg)
        gorder = np.argsort(-gs, axis=1, kind="stable")[:, :tg]
        elig = np.zeros(v.shape, dtype=bool)
        for j in range(tg):
            for m in range(E // ng):
                elig[np.arange(len(v)), gorder[:, j] * (E // ng) + m] = True
        return O.select_topk(v, k, elig)

    base = sel(l)
    delta = margin / 8
    for _ in range(200):
        pert = l + rng.choice([-delta, 0.0, delta], size=l.shape)
        got = sel(pert)
        s, o = d["set"], d["order"]
        assert np.array_equal(np.sort(got[s], axis=1), np.sort(base[s], axis=1))
        assert np.array_equal(got[o], base[o])


# ------------------------------------------------------------------------------------------------
# Dispatch layout
# ------------------------------------------------------------------------------------------------

def test_worked_example_send_counts_from_page():
    g = _load("a2a_demo_dispatch.json")
    idx = np.array(g["expert_indices"])
    assert O.send_counts(idx, g["num_experts"], g["world_size"]).tolist() == g["send_counts"]
    lay = O.dispatch_layout(idx, g["num_experts"], g["world_size"])
    assert lay["rank_counts"].tolist() == g["send_counts"]


def test_worked_example_full_layout_by_hand():
    # pairs p = t*2 + j: 0:(t0,e0) 1:(t0,e2) 2:(t1,e1) 3:(t1,e3) 4:(t2,e0) 5:(t2,e1) 6:(t3,e2) 7:(t3,e3)
    # grouped by (expert, pair id): e0 <- p0,p4 ; e1 <- p2,p5 ; e2 <- p1,p6 ; e3 <- p3,p7
    idx = np.array(_load("a2a_demo_dispatch.json")["expert_indices"])
    lay = O.dispatch_layout(idx, 4, 2)
    assert lay["expert_counts"].tolist() == [2, 2, 2, 2]
    assert lay["expert_offsets"].tolist() == [0, 2, 4, 6, 8]
    assert lay["row_to_pair"].tolist() == [0, 4, 2, 5, 1, 6, 3, 7]
    assert lay["pair_to_row"].tolist() == [0, 4, 2, 6, 1, 3, 5, 7]
    assert lay["rank_offsets"].tolist() == [0, 4, 8]


def _layout_bruteforce(idx, k, E, ep, C):
    T = len(idx)
    pairs = sorted((idx[t][j], t * k + j) for t in range(T) for j in range(k))   # by (expert, pair id)
    seen = {}
    rows = []
    for e, p in pairs:
        r = seen.get(e, 0)
        seen[e] = r + 1
        if r < C:
            rows.append(p)
    p2r = [-1] * (T * k)
    for r, p in enumerate(rows):
        p2r[p] = r
    kept = [min(sum(1 for t in range(T) for j in range(k) if idx[t][j] == e), C) for e in range(E)]
    return rows, p2r, kept


@settings(max_examples=80, deadline=None)
@given(T=st.integers(0, 9), data=st.data())
def test_layout_matches_sorted_bruteforce(T, data):
    E = data.draw(st.sampled_from([1, 2, 3, 4, 6]))
    k = data.draw(st.integers(1, E))
    ep = data.draw(st.sampled_from([d for d in range(1, E + 1) if E % d == 0]))
    C = data.draw(st.integers(0, max(1, T * k)))
    idx = [data.draw(st.permutations(range(E)))[:k] for _ in range(T)]
    arr = np.array(idx, dtype=np.int64).reshape(T, k)
    lay = O.dispatch_layout(arr, E, ep, C)
    rows, p2r, kept = _layout_bruteforce(idx, k, E, ep, C)
    N = len(rows)
    assert lay["n_kept"] == N
    assert lay["row_to_pair"][:N].tolist() == rows
    assert np.all(lay["row_to_pair"][N:] == -1)
    assert lay["pair_to_row"].tolist() == p2r
    assert lay["kept_counts"].tolist() == kept
    assert lay["rank_counts"].tolist() == [sum(kept[r * (E // ep):(r + 1) * (E // ep)]) for r in range(ep)]


def test_layout_invariants_random():
    rng = np.random.default_rng(7)
    T, E, k = 300, 16, 4
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    lay = O.dispatch_layout(idx, E, 4)
    assert lay["expert_counts"].sum() == T * k                       # counts sum to T*k
    r2p, p2r = lay["row_to_pair"], lay["pair_to_row"]
    assert sorted(r2p.tolist()) == list(range(T * k))              # bijection (dropless)
    assert np.all(p2r[r2p] == np.arange(T * k))
    keys = [(idx.reshape(-1)[p], p) for p in r2p]
    assert keys == sorted(keys)                                    # sorted by (expert, pair id)


def test_capacity_closed_forms():
    for c in _load("closed_forms.json")["capacity"]["cases"]:
        assert O.capacity(c["cf"], c["tokens"], c["k"], c["E"]) == c["C"]
    assert O.capacity(0.0, 100, 2, 4) == 200                       # dropless: every pair fits


def test_capacity_drops_latest_tokens():
    # 6 tokens, k=1, all to expert 1 except token 2 -> expert 0; C = 2: expert 1 keeps tokens 0,1
    idx = np.array([[1], [1], [0], [1], [1], [1]])
    lay = O.dispatch_layout(idx, 2, 1, 2)
    assert lay["kept_counts"].tolist() == [1, 2]
    assert lay["pair_to_row"].tolist() == [1, 2, 0, -1, -1, -1]
    assert lay["n_dropped"] == 3


def test_ep_extremes():
    rng = np.random.default_rng(8)
    idx = np.stack([rng.permutation(8)[:2] for _ in range(40)])
    one = O.dispatch_layout(idx, 8, 1)
    assert one["rank_counts"].tolist() == [80] and one["rank_offsets"].tolist() == [0, 80]
    each = O.dispatch_layout(idx, 8, 8)
    assert each["rank_counts"].tolist() == each["kept_counts"].tolist()
    assert each["rank_offsets"].tolist() == each["expert_offsets"].tolist()


def test_simulated_dispatch_matrix_invariants_from_page():
    g = _load("a2a_sim_dispatch_matrix.json")
    printed = np.array(g["matrix"])
    assert printed.sum() == g["total_pairs"]
    assert printed.sum(axis=1).tolist() == [g["pairs_per_source_device"]] * g["num_devices"]
    rng = np.random.default_rng(9)
    n, tpd, E, k = g["num_devices"], g["tokens_per_device"], g["num_experts"], g["top_k"]
    idx = rng.integers(0, E, size=(n, tpd, k))          # the page draws ids with replacement
    m = O.dispatch_matrix(idx, E, n)
    assert m.sum() == g["total_pairs"]
    assert m.sum(axis=1).tolist() == [g["pairs_per_source_device"]] * n
    # same spread as the printed draw: every entry within 6 binomial std of the mean 256
    sd = math.sqrt(tpd * k * (1 / n) * (1 - 1 / n))
    assert np.all(np.abs(printed - tpd * k / n) < 6 * sd) and np.all(np.abs(m - tpd * k / n) < 6 * sd)


def test_remote_fraction_uniform_routing():
    # Communication Overhead Analysis: about (N-1)/N of pairs cross devices under uniform routing
    rng = np.random.default_rng(10)
    T, E, k, N = 20000, 64, 4, 8
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    lay = O.dispatch_layout(idx, E, N)
    remote = lay["n_kept"] - lay["rank_counts"][0]
    assert abs(remote / (T * k) - (N - 1) / N) < 0.01


def test_dispatch_volume_matches_the_page_equation_on_exactly_uniform_routing():
    # Per-GPU dispatch volume B*S*k*H*(EP-1)/EP*sizeof ("Communication Volume and Hardware Topology").
    # B=2, S=4 (T=8 tokens), k=2, E=8 experts on EP=4 devices (2 each), H=16, bf16 (2 bytes).
    # Pair p = t*k + j goes to expert p mod 8, so each device receives exactly T*k/EP = 4 pairs and,
    # seen from any one device, 16 - 4 = 12 pairs leave it: 2*4*2*16*(3/4)*2 = 384 bytes.
    T, k, E, EP, H = 8, 2, 8, 4, 16
    idx = (np.arange(T * k) % E).reshape(T, k)
    lay = O.dispatch_layout(idx, E, EP)
    assert lay["rank_counts"].tolist() == [4, 4, 4, 4]
    for r in range(EP):
        remote = lay["n_kept"] - lay["rank_counts"][r]
        assert O.dispatch_volume_bytes(remote, H, 2) == 384
    # every pair already on device 0: nothing leaves it; every pair on device 3: all 16 pairs leave
    # device 0 (16 * 16 * 2 = 512 bytes) and nothing leaves device 3
    local = O.dispatch_layout(np.zeros((T, k), dtype=np.int64), E, EP)
    assert O.dispatch_volume_bytes(local["n_kept"] - local["rank_counts"][0], H, 2) == 0
    far = O.dispatch_layout(np.full((T, k), 7), E, EP)
    assert O.dispatch_volume_bytes(far["n_kept"] - far["rank_counts"][0], H, 2) == 512
    assert O.dispatch_volume_bytes(far["n_kept"] - far["rank_counts"][3], H, 2) == 0
    # float32 doubles it (sizeof = 4): 768 bytes on the uniform routing
    assert O.dispatch_volume_bytes(lay["n_kept"] - lay["rank_counts"][1], H, 4) == 768


# ------------------------------------------------------------------------------------------------
# Expert FFN
# ------------------------------------------------------------------------------------------------

def test_activation_textbook_values():
    sf = _load("closed_forms.json")["special_functions"]
    for a, v in sf["gelu"]:
        assert abs(O.gelu(np.array(a)) - v) <= 1e-15 * max(1.0, abs(v))
    for a, v in sf["silu"]:
        assert abs(O.silu(np.array(a)) - v) <= 1e-15 * max(1.0, abs(v))


def test_swiglu_scalar_closed_form_pins_parenthesisation():
    # D = F = 1: x=1, W1=1, W3=2, W2=3 -> SiLU(1)*2*3. The other reading, (W1 x)*SiLU(W3 x)*W2,
    # would give 1*SiLU(2)*3 = 5.2848; SiLU of the product would give SiLU(2)*3 as well.
    w1 = np.array([[[1.0]]]); w3 = np.array([[[2.0]]]); w2 = np.array([[[3.0]]])
    y = O.expert_ffn(np.array([[1.0]]), np.array([0, 1]), w1, w3, w2, O.ACT_SWIGLU)
    assert abs(y[0, 0] - 0.7310585786300049 * 6.0) < 1e-14


def test_ffn_nonsquare_hand_example():
    # D=2, F=3. x=[1,-1]; W1 rows [1,0],[0,1],[1,1] -> a=[1,-1,0]; W3 rows [2,0],[0,0],[1,-1] -> b=[2,0,2]
    # h = SiLU(a)*b = [2*SiLU(1), 0, 0]; W2 [[1,0,0],[0,0,5]] -> y = [2*SiLU(1), 0]
    w1 = np.array([[[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]]])
    w3 = np.array([[[2.0, 0.0], [0.0, 0.0], [1.0, -1.0]]])
    w2 = np.array([[[1.0, 0.0, 0.0], [0.0, 0.0, 5.0]]])
    y = O.expert_ffn(np.array([[1.0, -1.0]]), np.array([0, 1]), w1, w3, w2, O.ACT_SWIGLU)
    np.testing.assert_allclose(y, [[2 * 0.7310585786300049, 0.0]], atol=1e-15)
    # GELU expert: h = GELU(a) = [Phi(1), -0.1586..., 0]; y = [Phi(1), 0]
    y2 = O.expert_ffn(np.array([[1.0, -1.0]]), np.array([0, 1]), w1, None, w2, O.ACT_GELU)
    np.testing.assert_allclose(y2, [[0.8413447460685429, 0.0]], atol=1e-15)


def test_ffn_groups_use_their_own_expert():
    rng = np.random.default_rng(11)
    E, D, F = 3, 5, 4
    w1, w3, w2 = rng.standard_normal((E, F, D)), rng.standard_normal((E, F, D)), rng.standard_normal((E, D, F))
    x = rng.standard_normal((6, D))
    off = np.array([0, 2, 2, 6])                 # expert 1 empty
    y = O.expert_ffn(x, off, w1, w3, w2, O.ACT_SWIGLU)
    # relabelling experts 0 and 2 (weights and groups together) permutes the row blocks
    perm = [2, 1, 0]
    x2 = np.concatenate([x[2:6], x[0:2]])
    y2 = O.expert_ffn(x2, np.array([0, 4, 4, 6]), w1[perm], w3[perm], w2[perm], O.ACT_SWIGLU)
    np.testing.assert_allclose(np.concatenate([y2[4:6], y2[0:4]]), y, rtol=1e-13)
    # zero W2 -> zero output; doubling W2 doubles it
    assert np.all(O.expert_ffn(x, off, w1, w3, 0 * w2, O.ACT_SWIGLU) == 0)
    np.testing.assert_allclose(O.expert_ffn(x, off, w1, w3, 2 * w2, O.ACT_SWIGLU), 2 * y, rtol=1e-14)
    # sampled-rows form agrees with the grouped form
    ex = np.array([0, 0, 2, 2, 2, 2])
    np.testing.assert_allclose(O.expert_ffn_rows(x, ex, w1, w3, w2, O.ACT_SWIGLU), y, rtol=1e-14)


# ------------------------------------------------------------------------------------------------
# Combine and the whole layer
# ------------------------------------------------------------------------------------------------

def test_combine_hand_example():
    # T=2, k=2. y_perm rows r0..r3; token 0 -> rows 2 (g .75) and 0 (g .25); token 1 -> row 3, row 1 dropped
    yp = np.array([[4.0, 0.0], [100.0, 100.0], [0.0, 8.0], [1.0, 2.0]])
    p2r = np.array([2, 0, 3, -1])
    g = np.array([[0.75, 0.25], [0.5, 0.5]])
    y = O.combine(yp, p2r, g, 2, 2)
    assert y.tolist() == [[1.0, 6.0], [0.5, 1.0]]


def test_identity_experts_return_x_and_volume():
    rng = np.random.default_rng(12)
    T, D, E, k = 64, 8, 8, 2
    x = rng.standard_normal((T, D))
    r = O.route(x, rng.standard_normal((E, D)), None, k, O.GATE_SOFTMAX_TOPK)
    lay = O.dispatch_layout(r["topk_idx"], E, 4)
    xp = O.permute(x, lay["row_to_pair"], k)
    y = O.combine(xp, lay["pair_to_row"], r["topk_gate"], T, k)   # identity experts: y_perm = x_perm
    np.testing.assert_allclose(y, x, rtol=1e-14, atol=1e-15)
    moved = xp.size + xp.size                                      # dispatch writes + combine reads
    assert moved == O.comm_volume_elements(lay["n_kept"], D) == 2 * T * k * D
    for c in _load("closed_forms.json")["volume"]["cases"]:
        assert O.comm_volume_elements(c["B"] * c["S"] * c["K"], c["D"]) == c["V"]


def test_dropped_tokens_combine_to_zero():
    x = np.arange(12, dtype=np.float64).reshape(6, 2) + 1
    idx = np.array([[1], [1], [0], [1], [1], [1]])
    lay = O.dispatch_layout(idx, 2, 1, 2)
    xp = O.permute(x, lay["row_to_pair"], 1)
    y = O.combine(xp, lay["pair_to_row"], np.ones((6, 1)), 6, 1)
    np.testing.assert_array_equal(y[[0, 1, 2]], x[[0, 1, 2]])
    assert np.all(y[3:] == 0)


def test_dense_special_case_e1_k1():
    # one expert, k=1: gates are 1 and the layer is that expert's FFN on every token
    rng = np.random.default_rng(13)
    T, D, F = 10, 4, 6
    inputs = {"x": rng.standard_normal((T, D)), "w_gate": rng.standard_normal((1, D)), "bias": None,
              "w1": rng.standard_normal((1, F, D)), "w3": rng.standard_normal((1, F, D)),
              "w2": rng.standard_normal((1, D, F))}
    cfg = type("Cfg", (), dict(T=T, D=D, E=1, top_k=1, F=F, gate=O.GATE_SOFTMAX_TOPK, n_groups=0,
                                topk_groups=0, capacity_factor=0.0, ep_size=1, act=O.ACT_SWIGLU))
    out = O.layer_forward(inputs, cfg)
    x = inputs["x"]
    a = np.array([[sum(inputs["w1"][0][f][d] * x[t][d] for d in range(D)) for f in range(F)] for t in range(T)])
    b = np.array([[sum(inputs["w3"][0][f][d] * x[t][d] for d in range(D)) for f in range(F)] for t in range(T)])
    h = a / (1 + np.exp(-a)) * b
    y = np.array([[sum(inputs["w2"][0][d][f] * h[t][f] for f in range(F)) for d in range(D)] for t in range(T)])
    np.testing.assert_allclose(out["y"], y, rtol=1e-12, atol=1e-12)


def test_tiny_layer_end_to_end_invariants():
    import workloads as W
    cfg = W.get_config("tiny_fp32")
    inp = W.make_inputs(cfg, "cpu")
    out = O.layer_forward(inp, cfg)
    assert out["expert_counts"].sum() == cfg.T * cfg.top_k
    assert out["n_kept"] == cfg.T * cfg.top_k
    np.testing.assert_allclose(out["topk_gate"].sum(axis=1), 1.0, rtol=1e-14)
    assert out["y"].shape == (cfg.T, cfg.D) and np.all(np.isfinite(out["y"]))


@pytest.mark.parametrize("k", [1, 3])
def test_k_equals_e_selects_everything(k):
    rng = np.random.default_rng(14)
    l = rng.standard_normal((5, k))
    idx = O.select_topk(l, k)
    assert all(sorted(r) == list(range(k)) for r in idx.tolist())
    assert O.decisive_tokens(l, k)["set"].all()


def test_all_pairs_to_one_expert():
    idx = np.zeros((50, 1), dtype=np.int64)
    lay = O.dispatch_layout(idx, 4, 2)
    assert lay["expert_counts"].tolist() == [50, 0, 0, 0]
    assert lay["expert_offsets"].tolist() == [0, 50, 50, 50, 50]
    assert lay["rank_counts"].tolist() == [50, 0]
    assert lay["row_to_pair"].tolist() == list(range(50))


def test_itertools_sanity():
    # the brute-force helper itself picks the k largest by value (checked on all 3-subsets of 5)
    row = [0.3, -1.0, 2.0, 2.0, 0.0]
    best = max(itertools.combinations(range(5), 3), key=lambda c: (sum(row[i] for i in c), [-i for i in c]))
    assert sorted(_topk_by_rank_counting(row, 3)) == sorted(best)


# ------------------------------------------------------------------------------------------------
# Metamorphic checks on the whole layer: relabelled experts, permuted tokens, zero and identical
# experts. Each follows from the layer equation y = sum over the chosen experts of gate * expert(x)
# without reference to how the oracle computes it.
# ------------------------------------------------------------------------------------------------

def _small_layer(seed, T=24, D=8, E=6, k=2, F=5, capacity_factor=0.0, gate=None, act=None):
    rng = np.random.default_rng(seed)
    inputs = {"x": rng.standard_normal((T, D)), "w_gate": rng.standard_normal((E, D)),
              "bias": rng.standard_normal(E) * 0.3,
              "w1": rng.standard_normal((E, F, D)), "w3": rng.standard_normal((E, F, D)),
              "w2": rng.standard_normal((E, D, F))}
    cfg = type("Cfg", (), dict(T=T, D=D, E=E, top_k=k, F=F, n_groups=0, topk_groups=0,
                                gate=O.GATE_SOFTMAX_TOPK if gate is None else gate,
                                capacity_factor=capacity_factor, ep_size=1,
                                act=O.ACT_SWIGLU if act is None else act))
    return inputs, cfg


@pytest.mark.parametrize("capacity_factor", [0.0, 0.75])
@pytest.mark.parametrize("gate", [O.GATE_SOFTMAX_TOPK, O.GATE_SIGMOID_TOPK])
def test_relabelled_experts_give_the_same_layer(capacity_factor, gate):
    # expert e renamed pi[e] (its router row, bias and weights move with it): every token picks the
    # same experts under their new names, in the same slots, and y does not change; the keep rule
    # ranks an expert's pairs by pair id, so drops follow the expert too
    inputs, cfg = _small_layer(20, capacity_factor=capacity_factor, gate=gate)
    pi = np.array([3, 0, 5, 1, 4, 2])
    moved = dict(inputs)
    for key in ("w_gate", "bias", "w1", "w3", "w2"):
        a = np.empty_like(inputs[key])
        a[pi] = inputs[key]
        moved[key] = a
    ref, got = O.layer_forward(inputs, cfg), O.layer_forward(moved, cfg)
    np.testing.assert_array_equal(got["topk_idx"], pi[ref["topk_idx"]])
    np.testing.assert_array_equal(got["topk_gate"], ref["topk_gate"])
    np.testing.assert_array_equal(got["expert_counts"][pi], ref["expert_counts"])
    np.testing.assert_array_equal(got["pair_to_row"] >= 0, ref["pair_to_row"] >= 0)
    np.testing.assert_allclose(got["y"], ref["y"], rtol=1e-12, atol=1e-12)


def test_permuted_tokens_permute_the_output():
    # dropless: a token's output depends on that token alone
    inputs, cfg = _small_layer(21)
    sigma = np.random.default_rng(22).permutation(cfg.T)
    moved = dict(inputs, x=inputs["x"][sigma])
    ref, got = O.layer_forward(inputs, cfg), O.layer_forward(moved, cfg)
    np.testing.assert_array_equal(got["topk_idx"], ref["topk_idx"][sigma])
    np.testing.assert_allclose(got["y"], ref["y"][sigma], rtol=1e-12, atol=1e-12)


def test_zero_down_projection_gives_zero_output():
    inputs, cfg = _small_layer(23)
    inputs["w2"] = np.zeros_like(inputs["w2"])
    out = O.layer_forward(inputs, cfg)
    assert np.all(out["y"] == 0.0)
    assert np.all(out["y_perm"] == 0.0) and out["n_kept"] == cfg.T * cfg.top_k


@pytest.mark.parametrize("act", [O.ACT_SWIGLU, O.ACT_GELU])
def test_identical_experts_make_a_dense_ffn(act):
    # every expert the same FFN and the gates of a token summing to 1: the routed sum is that FFN of
    # the token, whatever the router picked (closed form computed here with plain loops)
    inputs, cfg = _small_layer(24, T=7, D=4, E=5, k=3, F=3, act=act)
    for key in ("w1", "w3", "w2"):
        inputs[key] = np.repeat(inputs[key][:1], cfg.E, axis=0)
    if act == O.ACT_GELU:
        inputs["w3"] = None
    out = O.layer_forward(inputs, cfg)
    x, w1, w2 = inputs["x"], inputs["w1"][0], inputs["w2"][0]
    for t in range(cfg.T):
        a = [sum(w1[f][d] * x[t][d] for d in range(cfg.D)) for f in range(cfg.F)]
        if act == O.ACT_SWIGLU:
            w3 = inputs["w3"][0]
            b = [sum(w3[f][d] * x[t][d] for d in range(cfg.D)) for f in range(cfg.F)]
            h = [a[f] / (1.0 + math.exp(-a[f])) * b[f] for f in range(cfg.F)]
        else:
            h = [0.5 * a[f] * (1.0 + math.erf(a[f] / math.sqrt(2.0))) for f in range(cfg.F)]
        want = [sum(w2[d][f] * h[f] for f in range(cfg.F)) for d in range(cfg.D)]
        np.testing.assert_allclose(out["y"][t], want, rtol=1e-11, atol=1e-12)


def test_round_to_f32_ties_to_even():
    # 1 + 2^-24 lies halfway between 1 and the next float32 (1 + 2^-23): the even one, 1, wins;
    # 1 + 3*2^-24 lies halfway between 1 + 2^-23 and 1 + 2^-22: again the even mantissa, 1 + 2^-22
    got = O.round_to_f32(np.array([1 + 2.0 ** -24, 1 + 3 * 2.0 ** -24, -(1 + 2.0 ** -24), 0.1]))
    assert got[0] == 1.0 and got[1] == 1 + 2.0 ** -22 and got[2] == -1.0
    assert got[3] == float(np.float32(0.1)) and got[3] != 0.1


def test_selection_key_hand_values():
    # sigmoid gating ranks sigmoid(l) + b, the other gates l + b; each term held in float32
    l = np.array([[0.0, 2.0, -1.0]])
    b = np.array([0.25, -0.5, 1e-9], dtype=np.float32)
    sig = O.selection_key(l, O.GATE_SIGMOID_TOPK, b)
    s2 = float(np.float32(1.0 / (1.0 + np.exp(-2.0))))
    s_1 = float(np.float32(1.0 / (1.0 + np.exp(1.0))))
    assert sig[0, 0] == 0.75
    assert sig[0, 1] == float(np.float32(s2 - 0.5))
    assert sig[0, 2] == float(np.float32(s_1 + float(np.float32(1e-9))))
    soft = O.selection_key(l, O.GATE_SOFTMAX_TOPK, b)
    assert soft[0, 0] == 0.25 and soft[0, 1] == 1.5
    assert soft[0, 2] == -1.0  # 1e-9 is below half an ulp of 1 in float32: the sum rounds back to -1
