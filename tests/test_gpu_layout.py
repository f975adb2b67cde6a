"""GPU parity of the dispatch layout in both of its launch forms: one block with every chunk histogram
in LDS (at most 64 chunks of 512 pairs and 8192 histogram entries), and four kernels with the
histograms in the workspace. Sizes sit on either side of each limit; expert ids are drawn with a
Zipf-shaped skew so that a capacity cut drops pairs; every output is compared with the oracle's
layout bit for bit, through moe_dispatch_layout and moe_dispatch_layout_noalloc."""
import numpy as np
import pytest
import torch

import combine_experts_amd as M
import oracle as O

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")

# name: (T, k, E, ep_size, capacity factor); the comment gives the form the size takes
CASES = {
    "chunks_64": (16384, 2, 8, 8, 0.0),        # 64 chunks: one block
    "chunks_65": (16385, 2, 8, 8, 0.0),        # 65 chunks: four kernels
    "hist_8192": (8192, 4, 128, 16, 1.0),      # 64 x 128 entries: one block, capacity cut
    "hist_8256": (8192, 4, 129, 3, 1.0),       # 64 x 129 entries: four kernels, capacity cut
    "e1024_8chunks": (4096, 1, 1024, 8, 1.25),  # 8 x 1024: one block
    "e1024_9chunks": (4097, 1, 1024, 8, 1.25),  # 9 x 1024: four kernels
    "ragged_small": (77, 3, 5, 5, 0.7),         # one partial chunk
    "ragged_large": (70001, 2, 16, 4, 0.9),     # 274 chunks, the last one partial
}


def _skewed_topk(T, k, E, seed):
    """k distinct experts per token, drawn without replacement with weights proportional to 1/(e+1)."""
    rng = np.random.default_rng(seed)
    w = 1.0 / np.arange(1, E + 1)
    keys = np.log(rng.random((T, E))) / w      # Gumbel-top-k: the k largest keys
    return np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int32)


@needs_gpu
@pytest.mark.parametrize("name", list(CASES))
def test_layout_forms_equal_the_oracle(name):
    T, k, E, ep, cf = CASES[name]
    print(f"[layout] {name}: T={T} k={k} E={E} ep={ep} cf={cf}", flush=True)
    idx = _skewed_topk(T, k, E, seed=11 + list(CASES).index(name))
    d = M.make_dims(T, 64, E, k, 64, ep_size=ep, capacity_factor=cf)
    C = O.capacity(cf, T, k, E)
    assert M.moe_capacity(d) == C
    want = O.dispatch_layout(idx, E, ep, C)
    i32 = dict(dtype=torch.int32, device="cuda")
    topk = torch.as_tensor(idx.reshape(-1), device="cuda")
    ws = torch.empty(max(256, M.moe_workspace_size(d, M.MOE_STAGE_LAYOUT)), dtype=torch.uint8, device="cuda")
    for form in ("workspace", "noalloc"):
        outs = [torch.full((n,), -7, **i32) for n in (E, E + 1, ep, ep + 1, T * k, T * k)]
        if form == "workspace":
            M.moe_dispatch_layout(d, topk, *outs, ws)
        else:
            M.moe_dispatch_layout_noalloc(d, topk, *outs)
        torch.cuda.synchronize()
        got = [o.cpu().long().numpy() for o in outs]
        for g, key in zip(got, ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets", "pair_to_row",
                                "row_to_pair")):
            assert np.array_equal(g, want[key]), f"{form}: {key}"
    if cf > 0:
        assert want["n_dropped"] > 0, "the capacity cut is expected to drop pairs here"
