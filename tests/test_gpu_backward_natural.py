"""The data-gradient GEMMs on the weights as stored (moe_expert_ffn_down_backward_w,
moe_expert_ffn_up_backward_w: K-major weight slices transposed in the LDS reads) against the same
GEMMs on transposed weight copies (moe_transpose_weights): bit for bit, since both feed the matrix
cores the same values in the same order. Step entry points on six configurations (SwiGLU and GELU,
output widths that do not fill the last 256-column tile, capacity drops) and the full DeepSeek-V3
shape; the backward executor without transposed copies against the executor with them."""
import pytest
import torch

import combine_experts_amd as M
import workloads as W
from tests.test_gpu_backward import CASES, _train_forward

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def _steps_both_ways(cfg, seed):
    inp = W.make_inputs(cfg, "cuda")
    d, buf, pre = _train_forward(cfg, inp)
    nm = 2 if cfg.act == W.ACT_SWIGLU else 1
    P, D, F, E = cfg.T * cfg.top_k, cfg.D, cfg.F, cfg.E
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    dy = torch.randn((cfg.T, D), generator=g, device="cuda").to(torch.bfloat16)
    dy_perm = torch.empty((P, D), dtype=torch.bfloat16, device="cuda")
    dgate = torch.empty(P, dtype=torch.float32, device="cuda")
    M.moe_backward_combine(d, dy, buf.pair_to_row, buf.topk_gate, buf.y_perm, dy_perm, dgate)
    w13t = torch.empty((E, D, nm * F), dtype=torch.bfloat16, device="cuda")
    w2t = torch.empty((E, F, D), dtype=torch.bfloat16, device="cuda")
    M.moe_transpose_weights(d, inp["w1"], inp["w3"], inp["w2"], w13t, w2t)
    da_t = torch.full((P, nm * F), float("nan"), dtype=torch.bfloat16, device="cuda")
    da_w = torch.full((P, nm * F), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.moe_expert_ffn_down_backward(d, dy_perm, buf.expert_offsets, w2t, pre, da_t)
    M.moe_expert_ffn_down_backward_w(d, dy_perm, buf.expert_offsets, inp["w2"], pre, da_w)
    dx_t = torch.full((P, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    dx_w = torch.full((P, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.moe_expert_ffn_up_backward(d, da_t, buf.expert_offsets, w13t, dx_t)
    M.moe_expert_ffn_up_backward_w(d, da_t, buf.expert_offsets, inp["w1"], inp["w3"], dx_w)
    torch.cuda.synchronize()
    N = int(buf.expert_offsets[-1].item())
    return N, (da_t, da_w), (dx_t, dx_w)


@needs_gpu
@pytest.mark.parametrize("name", list(CASES))
def test_stored_weight_dgrad_equals_transposed(name):
    print(f"[natural] {name}", flush=True)
    N, (da_t, da_w), (dx_t, dx_w) = _steps_both_ways(CASES[name], 21)
    assert N > 0
    assert torch.equal(da_w[:N], da_t[:N]), "down-projection data gradient"
    assert torch.equal(dx_w[:N], dx_t[:N]), "up-projection data gradient"


@needs_gpu
def test_stored_weight_dgrad_full_dsv3():
    cfg = W.get_config("dsv3")
    print(f"[natural] {cfg.desc}", flush=True)
    N, (da_t, da_w), (dx_t, dx_w) = _steps_both_ways(cfg, 22)
    assert torch.equal(da_w[:N], da_t[:N])
    assert torch.equal(dx_w[:N], dx_t[:N])


@needs_gpu
@pytest.mark.parametrize("name", ["dsv3_small", "gelu_k1_bias", "capacity", "skew_small"])
def test_executor_without_transposed_copies(name):
    cfg = CASES[name]
    inp = W.make_inputs(cfg, "cuda")
    d = M.dims_from_config(cfg)
    weights = (inp["w1"], inp["w3"], inp["w2"])
    g = torch.Generator(device="cuda")
    g.manual_seed(23)
    dy = torch.randn((cfg.T, cfg.D), generator=g, device="cuda").to(torch.bfloat16)
    out = []
    for transposed in (True, False):
        buf = M.MoELayerBuffers(d, device="cuda", logits=True)
        bw = M.BackwardBuffers(d, device="cuda", transposed=transposed)
        assert (bw.w13t is None) != transposed
        M.forward_train(buf, bw, inp["x"], inp["w_gate"], inp["bias"], *weights)
        M.backward(buf, bw, inp["x"], inp["w_gate"], dy, transpose_weights=weights)
        torch.cuda.synchronize()
        N = int(buf.expert_offsets[-1].item())  # rows past N of da and dx_perm are left untouched
        out.append({n: (getattr(bw, n)[:N] if n in ("da", "dx_perm") else getattr(bw, n)).clone()
                    for n in ("dx", "dw_gate", "dbias", "dw1", "dw2", "dw3", "da", "dx_perm") if getattr(bw, n) is not None})
    for n, v in out[0].items():
        assert torch.equal(out[1][n], v), f"{n}: stored-weight executor differs"
