"""Router on odd shapes, against the oracle (moe_route and moe_route_ex).

The bf16 router pads the experts to a multiple of 16 (one to sixteen 16-expert tiles), takes 64
tokens per block and streams 64-wide slices of D through a ring of LDS stages; these cases cover
every padding of E, a partial last block, fewer tokens than one block, and D with fewer slices than
the ring holds (D = 64 and 128), plus the group-limited, full-softmax and selection-bias paths on
such shapes, and top-k up to 32."""
import numpy as np
import pytest
import torch

import combine_experts_amd as M
import workloads as W
from tests._parity import check_route
from tests import test_gpu_balance as B

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")

CASES = [
    # (name, T, D, E, k, extra)
    ("e3_t1_d64", 1, 64, 3, 2, {}),
    ("e17_t63_d128", 63, 128, 17, 3, {}),
    ("e33_t65_d192", 65, 192, 33, 4, {}),
    ("e100_t130_d256", 130, 256, 100, 6, {}),
    ("e200_t129_d64", 129, 64, 200, 8, {}),
    ("e256_t200_d320_grouped", 200, 320, 256, 8,
     dict(gate=W.GATE_SIGMOID_TOPK, n_groups=8, topk_groups=4)),
    ("e64_t97_d128_grouped", 97, 128, 64, 4, dict(n_groups=4, topk_groups=2)),
    ("e24_t300_d64_softmax_full", 300, 64, 24, 2, dict(gate=W.GATE_SOFTMAX_FULL)),
    # k > 16: the general one-token-per-wave selection (the 4-tokens-per-wave one takes k <= 16), up to
    # the router's k = 32
    ("e64_t70_d128_k20", 70, 128, 64, 20, {}),
    ("e256_t65_d64_k32_grouped", 65, 64, 256, 32, dict(gate=W.GATE_SIGMOID_TOPK, n_groups=8, topk_groups=4)),
    ("e40_t33_d64_k32_softmax_full", 33, 64, 40, 32, dict(gate=W.GATE_SOFTMAX_FULL)),
]


@needs_gpu
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_route_odd_shapes(case):
    name, T, D, E, k, extra = case
    print(f"[route_shapes] {name}", flush=True)
    cfg = W.MoEConfig(name=name, T=T, D=D, E=E, top_k=k, F=64, seed=101 + T + E, **extra)
    inp = W.make_inputs(cfg, "cuda", with_experts=False)
    host = {key: (None if v is None else v.detach().cpu()) for key, v in inp.items()}
    d = M.dims_from_config(cfg)
    buf = M.MoELayerBuffers(d, device="cuda", logits=True)
    M.moe_route(d, inp["x"], inp["w_gate"], inp["bias"], buf.topk_idx, buf.topk_gate, buf.logits)
    torch.cuda.synchronize()
    check_route(cfg, host, buf, decisive_min_frac=0.0 if T < 8 else 0.5)


@needs_gpu
@pytest.mark.parametrize("case", CASES[1:6], ids=[c[0] for c in CASES[1:6]])
def test_route_ex_selection_bias_odd_shapes(case):
    # the load-balancing router entry on the same shapes, checked as the balance tests check it
    name, T, D, E, k, extra = case
    print(f"[route_shapes] ex {name}", flush=True)
    cfg = W.MoEConfig(name=name, T=T, D=D, E=E, top_k=k, F=64, seed=201 + T + E, **extra)
    inp = W.make_inputs(cfg, "cuda", with_experts=False)
    host = {key: (None if v is None else v.detach().cpu()) for key, v in inp.items()}
    sb = W.make_select_bias(cfg, "cuda", std=0.05)
    _, idx, gate, logits, part = B._route_ex(cfg, inp, sb)
    B._check_biased_route(cfg, host, sb.cpu().numpy().astype(np.float64), idx, gate, logits)
    B._check_partials(cfg, logits, part)
