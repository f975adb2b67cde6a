"""GPU parity of the cluster view (expert parallelism emulated on one GPU) and the padded layout.

The cluster emulation runs the layer the way EP devices would: every source shard lays out its
own tokens, each rank's receive layout drives one gather that performs the exchange and the
per-expert regroup, the rank's experts run the grouped FFN, a scatter sends the outputs back,
and every source combines its own tokens. Each integer stage is compared bit for bit with the
oracle, and the final output must equal the one-GPU layer's output bit for bit (every row meets
the same kernels with the same operands). The padded (fixed-capacity) path must likewise equal
the compact path with the same capacity, bit for bit, with padding rows exactly zero.
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


def _one_gpu(cfg, inp):
    # the emulated ranks and the padded path run the unsplit down-projection; so does this reference
    d, buf = P.run_gpu(cfg, inp, logits=False, split_k=False)
    return d, buf


def _cluster_forward(cfg, inp, buf, n_src, check_oracle=True):
    """Emulated EP forward; returns y [T, D] and the per-rank receive counts."""
    T, D, E, k, ep = cfg.T, cfg.D, cfg.E, cfg.top_k, cfg.ep_size
    assert T % n_src == 0
    ts = T // n_src
    stride = ts * k
    epr = E // ep
    dt = W.torch_dtype(cfg.dtype)
    dev = "cuda"
    i32 = dict(dtype=torch.int32, device=dev)
    d_full = M.dims_from_config(cfg)
    d_src = M.dims_from_config(cfg.replace(T=ts))
    src_off = torch.empty((n_src, E + 1), **i32)
    p2r = torch.empty((n_src, ts * k), **i32)
    r2p = torch.empty((n_src, ts * k), **i32)
    counts = torch.empty(E, **i32)
    rc = torch.empty(ep, **i32)
    ro = torch.empty(ep + 1, **i32)
    ws = torch.empty(max(1, M.moe_workspace_size(d_src, M.MOE_STAGE_LAYOUT)), dtype=torch.uint8, device=dev)
    send = torch.zeros((n_src * stride, D), dtype=dt, device=dev)
    for s in range(n_src):
        idx_s = buf.topk_idx[s * ts * k:(s + 1) * ts * k]
        M.moe_dispatch_layout(d_src, idx_s, counts, src_off[s], rc, ro, p2r[s], r2p[s], ws)
        M.moe_permute(d_src, inp["x"][s * ts:(s + 1) * ts], p2r[s], send[s * stride:(s + 1) * stride])
    matrix = torch.empty((n_src, ep), **i32)
    M.moe_dispatch_matrix(d_full, buf.topk_idx, n_src, matrix)
    torch.cuda.synchronize()
    idx_h = P.i64(buf.topk_idx).reshape(n_src, ts, k)
    want_matrix = O.dispatch_matrix(idx_h, E, ep)
    assert np.array_equal(P.i64(matrix), want_matrix), "dispatch matrix"
    assert (want_matrix.sum(axis=1) == ts * k).all()
    back = torch.zeros_like(send)
    n_max = T * k
    g2s = torch.empty(n_max, **i32)
    recv_counts = torch.empty(n_src, **i32)
    eoff = torch.empty(epr + 1, **i32)
    grouped = torch.empty((n_max, D), dtype=dt, device=dev)
    y_grouped = torch.empty((n_max, D), dtype=dt, device=dev)
    # the rank's grouped FFN: its E/ep experts; rows bounded by T*k (top_k = 1 keeps top_k <= E valid)
    d_rank = M.dims_from_config(cfg.replace(T=T * k, top_k=1, E=epr, ep_size=1, n_groups=0, topk_groups=0))
    h = torch.empty((n_max, cfg.F), dtype=dt, device=dev)
    src_off_h = P.i64(src_off)
    per_rank = []
    for r in range(ep):
        M.moe_recv_layout(d_full, n_src, r, stride, src_off, recv_counts, eoff, g2s)
        if check_oracle:
            torch.cuda.synchronize()
            want = O.recv_layout(src_off_h, E, ep, r, stride)
            n = len(want["grouped_to_src_row"])
            got = P.i64(g2s)
            assert np.array_equal(got[:n], want["grouped_to_src_row"]), f"rank {r}: grouped_to_src_row"
            assert (got[n:] == -1).all()
            assert np.array_equal(P.i64(recv_counts), want["recv_counts"]), f"rank {r}: recv_counts"
            assert np.array_equal(P.i64(recv_counts), want_matrix[:, r])
            assert np.array_equal(P.i64(eoff), want["expert_offsets"]), f"rank {r}: expert offsets"
        M.moe_gather_rows(d_full, g2s, send, grouped)
        w1 = inp["w1"][r * epr:(r + 1) * epr]
        w3 = None if inp["w3"] is None else inp["w3"][r * epr:(r + 1) * epr]
        w2 = inp["w2"][r * epr:(r + 1) * epr]
        M.moe_expert_ffn_up(d_rank, grouped, eoff, w1, w3, h)
        M.moe_expert_ffn_down(d_rank, h, eoff, w2, y_grouped)
        M.moe_scatter_rows(d_full, g2s, y_grouped, back)
        per_rank.append(int(want_matrix[:, r].sum()))
    y = torch.empty((T, D), dtype=dt, device=dev)
    for s in range(n_src):
        M.moe_unpermute_combine(d_src, back[s * stride:(s + 1) * stride], p2r[s], buf.topk_gate[s * ts * k:(s + 1) * ts * k],
                                y[s * ts:(s + 1) * ts])
    torch.cuda.synchronize()
    return y, per_rank


CLUSTER = {
    "tiny_fp32": (W.get_config("tiny_fp32"), 4),
    "mixtral_small": (W.get_config("mixtral", T=1024, D=512, F=1856), 8),
    "dsv3_small": (W.get_config("dsv3", T=640, D=512, F=320), 64),
    "dsv3_small_8src": (W.get_config("dsv3", T=640, D=512, F=320, ep_size=8), 8),
    "gelu_k1": (W.MoEConfig(name="gelu_k1", T=768, D=256, E=16, top_k=1, F=512, act=W.ACT_GELU, ep_size=4,
                            bias="normal0.5", seed=31), 4),
    "skew_small": (W.get_config("skew", T=2048, D=256, F=448), 16),
}


@needs_gpu
@pytest.mark.parametrize("name", list(CLUSTER))
def test_cluster_emulation_equals_one_gpu_layer(name):
    cfg, n_src = CLUSTER[name]
    print(f"[cluster] {name}: {cfg} sources={n_src}", flush=True)
    inp = W.make_inputs(cfg, "cuda")
    _, buf = _one_gpu(cfg, inp)
    y, per_rank = _cluster_forward(cfg, inp, buf, n_src)
    assert sum(per_rank) == cfg.T * cfg.top_k
    assert torch.equal(y, buf.y), "cluster output differs from the one-GPU layer"


@needs_gpu
@pytest.mark.parametrize("name", ["mixtral", "dsv3"])
def test_cluster_emulation_full_size(name):
    cfg = W.get_config(name)
    n_src = cfg.ep_size
    print(f"[cluster] full {name}: sources={n_src}", flush=True)
    inp = W.make_inputs(cfg, "cuda")
    _, buf = _one_gpu(cfg, inp)
    y, per_rank = _cluster_forward(cfg, inp, buf, n_src, check_oracle=(name == "mixtral"))
    assert torch.equal(y, buf.y), "cluster output differs from the one-GPU layer"
    print(f"[cluster] rows per rank: min {min(per_rank)} max {max(per_rank)}", flush=True)


@needs_gpu
def test_gather_scatter_roundtrip():
    cfg = W.MoEConfig(name="rows", T=300, D=136, E=4, top_k=2, F=64, dtype=W.DT_BF16, seed=41)
    d = M.dims_from_config(cfg)
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    src = torch.randn((500, cfg.D), generator=g, device="cuda").to(torch.bfloat16)
    perm = torch.randperm(500, generator=g, device="cuda").to(torch.int32)
    row_map = torch.cat([perm[:450], torch.full((30,), -1, dtype=torch.int32, device="cuda")])
    dst = torch.full((480, cfg.D), 7.0, dtype=torch.bfloat16, device="cuda")
    M.moe_gather_rows(d, row_map, src, dst)
    back = torch.zeros_like(src)
    M.moe_scatter_rows(d, row_map, dst, back)
    torch.cuda.synchronize()
    assert torch.equal(dst[:450], src[perm[:450].long()])
    assert bool((dst[450:] == 7.0).all()), "rows with -1 are untouched"
    assert torch.equal(back[perm[:450].long()], src[perm[:450].long()])
    untouched = torch.ones(500, dtype=torch.bool, device="cuda")
    untouched[perm[:450].long()] = False
    assert bool((back[untouched] == 0).all())


PADDED = {
    "switch_small": W.get_config("switch_cap", T=2048),
    "cap_k2": W.MoEConfig(name="cap_k2", T=500, D=128, E=6, top_k=2, F=128, ep_size=2, capacity_factor=0.8,
                          bias="normal0.5", seed=9),
    "cf2_swiglu": W.MoEConfig(name="cf2_swiglu", T=600, D=256, E=8, top_k=2, F=192, capacity_factor=2.0, seed=33),
    "cap_f32": W.MoEConfig(name="cap_f32", T=200, D=64, E=4, top_k=2, F=96, capacity_factor=1.25, dtype=W.DT_F32,
                           bias="normal0.5", seed=34),
}


def _padded_forward(cfg, inp, buf):
    d = buf.d
    C = M.moe_capacity(d)
    R = cfg.E * C
    dt = W.torch_dtype(cfg.dtype)
    i32 = dict(dtype=torch.int32, device="cuda")
    p2s = torch.empty(cfg.T * cfg.top_k, **i32)
    s2p = torch.empty(R, **i32)
    poff = torch.empty(cfg.E + 1, **i32)
    M.moe_padded_layout(d, buf.topk_idx, buf.expert_offsets, buf.pair_to_row, buf.row_to_pair, p2s, s2p, poff)
    x_pad = torch.empty((R, cfg.D), dtype=dt, device="cuda")
    M.moe_permute_padded(d, inp["x"], s2p, x_pad)
    h_pad = torch.empty((R, cfg.F), dtype=dt, device="cuda")
    y_pad = torch.empty((R, cfg.D), dtype=dt, device="cuda")
    M.moe_expert_ffn_padded_up(d, x_pad, poff, inp["w1"], inp["w3"], h_pad)
    M.moe_expert_ffn_padded_down(d, h_pad, poff, inp["w2"], y_pad)
    y = torch.empty((cfg.T, cfg.D), dtype=dt, device="cuda")
    M.moe_unpermute_combine(d, y_pad, p2s, buf.topk_gate, y, n_rows=R)
    torch.cuda.synchronize()
    return dict(C=C, p2s=p2s, s2p=s2p, poff=poff, x_pad=x_pad, y_pad=y_pad, y=y)


@needs_gpu
@pytest.mark.parametrize("name", list(PADDED))
def test_padded_path_equals_compact_path(name):
    cfg = PADDED[name]
    print(f"[padded] {name}: {cfg}", flush=True)
    inp = W.make_inputs(cfg, "cuda")
    host = P.to_host(inp)
    _, buf = _one_gpu(cfg, inp)
    out = _padded_forward(cfg, inp, buf)
    C = out["C"]
    want = O.padded_layout(P.i64(buf.topk_idx).reshape(cfg.T, cfg.top_k), cfg.E, C)
    assert np.array_equal(P.i64(out["p2s"]), want["pair_to_slot"]), "pair_to_slot"
    assert np.array_equal(P.i64(out["s2p"]), want["slot_to_pair"]), "slot_to_pair"
    assert np.array_equal(P.i64(out["poff"]), want["padded_offsets"]), "padded_offsets"
    assert np.array_equal(P.f64(out["x_pad"]), O.permute_padded(host["x"], want["slot_to_pair"], cfg.top_k)), "x_pad"
    pad = torch.as_tensor(want["slot_to_pair"] < 0, device="cuda")
    assert bool((out["y_pad"][pad] == 0).all()), "padding rows must come out exactly zero"
    assert torch.equal(out["y"], buf.y), "padded path differs from the compact path"
    print(f"[padded] C={C} padding {want['padding']} of {cfg.E * C} slots "
          f"({want['padding'] / (cfg.E * C):.1%}), dropped {cfg.T * cfg.top_k - want['n_kept']}", flush=True)
