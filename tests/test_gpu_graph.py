"""The layer forward captured in a HIP graph and replayed (GraphLayer) against the eager forward: the
same bits on every replay, with eager work and synchronisations between replays and new inputs
written in place between them."""
import pytest
import torch

import combine_experts_amd as M
import workloads as W

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")

CASES = {
    "tiny_fp32": W.get_config("tiny_fp32"),
    "switch_cap": W.get_config("switch_cap"),
    "mixtral_small": W.get_config("mixtral", T=512, D=512, F=448),
    "dsv3_small": W.get_config("dsv3", T=320, D=512, F=320),
}


@needs_gpu
@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("gather", [True, False])
def test_graph_replays_equal_eager(name, gather):
    cfg = CASES[name]
    print(f"[graph] {name} gather={gather}", flush=True)
    inp = W.make_inputs(cfg, "cuda")
    d = M.dims_from_config(cfg)
    args = (inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"])
    gl = M.GraphLayer(d, *args, gather=gather)
    eager = M.MoELayerBuffers(d, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(31)
    for rep in range(4):
        if rep > 0:  # new tokens, written in place into the captured input
            inp["x"].copy_(torch.randn(inp["x"].shape, generator=g, device="cuda").to(inp["x"].dtype))
        y = gl.replay()
        torch.cuda.synchronize()
        ref = M.forward(eager, *args)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"replay {rep}"
        _ = (ref.float() * 2).sum().item()  # unrelated eager work between replays
