"""Pins for the oracle's cluster view (source shards, receive layout, whole-cluster forward) and the
GShard-style padded capacity layout.

Checked against an independent formulation (Python ``sorted`` over (local expert, source, row)
tags), the page's dispatch-matrix invariant (each source sends T/EP*k pairs), closed forms of the
padding waste, and the identity that a cluster of emulated devices computes the same layer as one
device.
"""
import numpy as np
import pytest

import oracle as O
import workloads as W


def _tiny(**kw):
    base = dict(name="tiny_cluster", T=64, D=16, E=8, top_k=2, F=24, ep_size=4, dtype=W.DT_F32, seed=21)
    base.update(kw)
    return W.MoEConfig(**base)


def test_source_shards():
    assert O.source_shards(12, 3) == [(0, 4), (4, 8), (8, 12)]
    with pytest.raises(ValueError):
        O.source_shards(10, 3)


def _recv_bruteforce(src_off, E, n_dst, r, stride):
    epr = E // n_dst
    tags = []
    for s in range(src_off.shape[0]):
        for j in range(int(src_off[s, E])):
            e = int(np.searchsorted(src_off[s], j, side="right") - 1)
            if r * epr <= e < (r + 1) * epr:
                tags.append((e - r * epr, s, s * stride + j))
    return [t[2] for t in sorted(tags)]


@pytest.mark.parametrize("n_ep,E,k", [(4, 8, 2), (2, 6, 3), (8, 8, 1), (1, 4, 2)])
def test_recv_layout_matches_sorted_tags(n_ep, E, k):
    rng = np.random.default_rng(n_ep * 100 + E)
    ts = 9
    stride = ts * k
    src_off = np.zeros((n_ep, E + 1), dtype=np.int64)
    for s in range(n_ep):
        idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(ts)])
        src_off[s] = O.dispatch_layout(idx, E, n_ep)["expert_offsets"]
    total = 0
    for r in range(n_ep):
        rl = O.recv_layout(src_off, E, n_ep, r, stride)
        assert rl["grouped_to_src_row"].tolist() == _recv_bruteforce(src_off, E, n_ep, r, stride)
        assert rl["expert_offsets"][-1] == len(rl["grouped_to_src_row"]) == rl["recv_counts"].sum()
        total += rl["recv_counts"]
    # every row a source sends lands on exactly one destination: T/EP * k per source (dropless)
    assert total.tolist() == [ts * k] * n_ep


@pytest.mark.parametrize("kw", [dict(), dict(act=W.ACT_GELU, top_k=1), dict(E=16, top_k=4, ep_size=8),
                                dict(gate=W.GATE_SIGMOID_TOPK, n_groups=4, topk_groups=2, top_k=2)])
def test_cluster_forward_is_the_one_device_layer(kw):
    cfg = _tiny(**kw)
    inp = W.make_inputs(cfg, "cpu")
    one = O.layer_forward(inp, cfg)
    for n_ep in sorted({1, 2, cfg.ep_size}):
        cl = O.cluster_forward(inp, cfg, n_ep)
        np.testing.assert_allclose(cl["y"], one["y"], rtol=1e-12, atol=1e-14)
        # the [src, dst] matrix: rows sum to T/EP * k; it matches the page's per-device bincount
        ts = cfg.T // n_ep
        assert cl["matrix"].sum(axis=1).tolist() == [ts * cfg.top_k] * n_ep
        per_src = one["topk_idx"].reshape(n_ep, ts, cfg.top_k)
        np.testing.assert_array_equal(cl["matrix"], O.dispatch_matrix(per_src, cfg.E, n_ep))


def test_padded_layout_keeps_what_the_compact_layout_keeps():
    rng = np.random.default_rng(4)
    T, E, k = 300, 6, 2
    idx = np.stack([rng.choice(E, size=k, replace=False, p=[0.3, 0.25, 0.2, 0.1, 0.1, 0.05]) for _ in range(T)])
    for C in (1, 37, 100, 250, T * k):
        comp = O.dispatch_layout(idx, E, 1, C)
        pad = O.padded_layout(idx, E, C)
        kept = comp["pair_to_row"] >= 0
        np.testing.assert_array_equal(pad["pair_to_slot"] >= 0, kept)
        e = idx.reshape(-1)
        np.testing.assert_array_equal(pad["pair_to_slot"][kept] - e[kept] * C,
                                      comp["pair_to_row"][kept] - comp["expert_offsets"][e[kept]])
        assert pad["padding"] == E * C - comp["n_kept"]
        filled = pad["slot_to_pair"] >= 0
        np.testing.assert_array_equal(pad["pair_to_slot"][pad["slot_to_pair"][filled]], np.nonzero(filled)[0])


def test_padding_waste_closed_forms():
    # perfectly even routing: every expert gets exactly T*k/E pairs
    T, E, k = 64, 8, 2
    idx = np.stack([[(2 * t) % E, (2 * t + 1) % E] for t in range(T)])
    per = T * k // E
    C1 = O.capacity(1.0, T, k, E)
    assert C1 == per
    p1 = O.padded_layout(idx, E, C1)
    assert p1["padding"] == 0 and p1["n_kept"] == T * k
    # CF 1.25: 25 % headroom over the even load, so 1/5 of the buffer is padding
    C2 = O.capacity(1.25, T, k, E)
    assert C2 == 20
    p2 = O.padded_layout(idx, E, C2)
    assert p2["n_kept"] == T * k
    assert p2["padding"] == E * (C2 - per) == 32
    assert p2["padding"] / (E * C2) == pytest.approx(0.2)


def test_permute_padded_zero_fills_padding():
    x = np.arange(12.0).reshape(4, 3)
    s2p = np.array([3, -1, 0, 5, -1, -1])
    out = O.permute_padded(x, s2p, k=2)
    np.testing.assert_array_equal(out, [x[1], [0, 0, 0], x[0], x[2], [0, 0, 0], [0, 0, 0]])


@pytest.mark.parametrize("cf", [0.75, 1.0, 1.5])
def test_padded_forward_equals_compact_forward_with_capacity(cf):
    cfg = _tiny(capacity_factor=cf, bias="normal0.5")
    inp = W.make_inputs(cfg, "cpu")
    one = O.layer_forward(inp, cfg)
    C = O.capacity(cf, cfg.T, cfg.top_k, cfg.E)
    pad = O.padded_layout(one["topk_idx"], cfg.E, C)
    xp = O.permute_padded(inp["x"], pad["slot_to_pair"], cfg.top_k)
    yp = O.expert_ffn(xp, pad["padded_offsets"], inp["w1"], inp["w3"], inp["w2"], cfg.act)
    # padding rows are zero in and zero out (SiLU(0)*0 = 0, GELU(0) = 0)
    assert np.all(yp[pad["slot_to_pair"] < 0] == 0)
    y = O.combine(yp, pad["pair_to_slot"], one["topk_gate"], cfg.T, cfg.top_k)
    np.testing.assert_allclose(y, one["y"], rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------------------------------------
# Shared expert and micro-batches
# ------------------------------------------------------------------------------------------------

def test_shared_expert_is_a_dense_one_expert_layer():
    # one expert, top-1, gate 1 (k = 1 softmax) routes every token to it: the dense layer
    cfg = _tiny(E=1, top_k=1, ep_size=1)
    inp = W.make_inputs(cfg, "cpu")
    dense = O.layer_forward(inp, cfg)["y"]
    shared = O.shared_expert_ffn(inp["x"], inp["w1"][0], inp["w3"][0], inp["w2"][0], cfg.act)
    np.testing.assert_allclose(shared, dense, rtol=1e-12, atol=1e-14)


def test_shared_expert_adds_to_the_routed_sum():
    cfg = _tiny(shared_F=40)
    inp = W.make_inputs(cfg, "cpu")
    routed = O.layer_forward({k: v for k, v in inp.items() if not k.startswith("shared")}, cfg)["y"]
    both = O.layer_forward(inp, cfg)["y"]
    sh = O.shared_expert_ffn(inp["x"], inp["shared_w1"], inp["shared_w3"], inp["shared_w2"], cfg.act)
    np.testing.assert_allclose(both, routed + sh, rtol=1e-13, atol=1e-15)
    # a zero shared down-projection contributes nothing
    z = dict(inp)
    z["shared_w2"] = inp["shared_w2"] * 0
    np.testing.assert_array_equal(O.layer_forward(z, cfg)["y"], routed)


@pytest.mark.parametrize("n_chunks", [1, 2, 4, 8])
def test_micro_batches_equal_the_whole_batch(n_chunks):
    cfg = _tiny(shared_F=24, gate=W.GATE_SIGMOID_TOPK, n_groups=4, topk_groups=2)
    inp = W.make_inputs(cfg, "cpu")
    np.testing.assert_allclose(O.layer_forward_chunked(inp, cfg, n_chunks)["y"], O.layer_forward(inp, cfg)["y"],
                               rtol=1e-12, atol=1e-14)
