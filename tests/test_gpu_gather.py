"""The permute fused into the up-projection (moe_expert_ffn_up_gather, and the executor without an
x_perm buffer) against the two separate steps: h and y bit for bit, since the GEMM reads the same
row values in the same order either way. Covers bf16 and float32, SwiGLU and GELU, capacity drops,
skewed routing, micro-batches on two streams and a shared expert; the full-size case is in
test_gpu_parity. Training without x_perm (the pre-activation up-projection and the transposed x
operand of the weight gradient gathering from x) equals training with it, bit for bit."""
import pytest
import torch

import combine_experts_amd as M
import workloads as W

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")

CASES = {
    "mixtral_small": W.get_config("mixtral", T=512, D=512, F=448),
    "dsv3_small": W.get_config("dsv3", T=320, D=512, F=320),
    "skew_small": W.get_config("skew", T=1024, D=256, F=192),
    "capacity_gelu": W.MoEConfig(name="capacity_gelu", T=400, D=128, E=6, top_k=2, F=128, act=W.ACT_GELU,
                                 capacity_factor=0.8, seed=81),
    "f32_swiglu": W.MoEConfig(name="f32_swiglu", T=96, D=64, E=5, top_k=2, F=48, dtype=W.DT_F32, seed=82),
    "f32_gelu_drops": W.MoEConfig(name="f32_gelu_drops", T=64, D=32, E=4, top_k=3, F=16, dtype=W.DT_F32,
                                  act=W.ACT_GELU, capacity_factor=0.6, seed=83),
}


@needs_gpu
@pytest.mark.parametrize("name", list(CASES))
def test_gather_up_equals_permute_then_up(name):
    cfg = CASES[name]
    print(f"[gather] {name}", flush=True)
    inp = W.make_inputs(cfg, "cuda")
    d = M.dims_from_config(cfg)
    buf = M.MoELayerBuffers(d, device="cuda")
    M.forward(buf, inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"])
    h2 = torch.full_like(buf.h, float("nan"))
    M.moe_expert_ffn_up_gather(d, inp["x"], buf.row_to_pair, buf.expert_offsets, inp["w1"], inp["w3"], h2)
    torch.cuda.synchronize()
    N = int(buf.expert_offsets[-1].item())
    assert N > 0
    assert torch.equal(h2[:N], buf.h[:N])
    # the layer without x_perm: the same output
    fused = M.MoELayerBuffers(d, device="cuda", x_perm=False)
    M.forward(fused, inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"])
    torch.cuda.synchronize()
    assert fused.x_perm is None
    assert torch.equal(fused.y, buf.y)


@needs_gpu
@pytest.mark.parametrize("two_streams", [False, True])
def test_gather_executor_micro_batches_and_shared_expert(two_streams):
    cfg = W.get_config("dsv3", T=640, D=512, F=320)
    inp = W.make_inputs(cfg, "cuda")
    d = M.dims_from_config(cfg)
    Fs = 256
    g = torch.Generator(device="cuda").manual_seed(84)
    sw = [(torch.randn((Fs, cfg.D), device="cuda", generator=g) * 0.05).to(torch.bfloat16),
          (torch.randn((Fs, cfg.D), device="cuda", generator=g) * 0.05).to(torch.bfloat16),
          (torch.randn((cfg.D, Fs), device="cuda", generator=g) * 0.05).to(torch.bfloat16)]
    ref = M.LayerExecutor(d, n_chunks=2, two_streams=two_streams, shared_F=Fs)
    fused = M.LayerExecutor(d, n_chunks=2, two_streams=two_streams, shared_F=Fs, gather=True)
    y_ref = ref.forward(inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"], shared=sw)
    y = fused.forward(inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"], shared=sw)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    assert torch.equal(fused.h, ref.h)


TRAIN_CASES = ["dsv3_small", "mixtral_small", "skew_small", "capacity_gelu"]


@needs_gpu
@pytest.mark.parametrize("name", TRAIN_CASES)
def test_training_without_x_perm(name):
    """Training with no x_perm: the up-projection that saves pre-activations and the transposed x
    operand of the W1/W3 gradient both gather their rows from x. Forward outputs, saved tensors and
    every gradient equal those of the run with x_perm bit for bit."""
    cfg = CASES[name]
    print(f"[gather] training {name}", flush=True)
    inp = W.make_inputs(cfg, "cuda")
    d = M.dims_from_config(cfg)
    g = torch.Generator(device="cuda").manual_seed(85)
    dy = torch.randn((cfg.T, cfg.D), generator=g, device="cuda").to(torch.bfloat16)
    runs = {}
    for with_xp in (True, False):
        buf = M.MoELayerBuffers(d, device="cuda", logits=True, x_perm=with_xp)
        bw = M.BackwardBuffers(d, device="cuda")
        M.forward_train(buf, bw, inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"])
        M.backward(buf, bw, inp["x"], inp["w_gate"], dy, transpose_weights=(inp["w1"], inp["w3"], inp["w2"]))
        torch.cuda.synchronize()
        assert (buf.x_perm is None) != with_xp
        N = int(buf.expert_offsets[-1].item())
        out = {"y": buf.y.clone(), "h": buf.h[:N].clone(), "pre": bw.pre[:N].clone()}
        for n in ("dx", "dw_gate", "dbias", "dw1", "dw3", "dw2"):
            v = getattr(bw, n)
            if v is not None:
                out[n] = v.clone()
        runs[with_xp] = out
    for n, v in runs[True].items():
        assert torch.equal(runs[False][n], v), f"{n} differs without x_perm"


@needs_gpu
def test_gathered_training_steps_equal_permute_then_step():
    cfg = CASES["dsv3_small"]
    inp = W.make_inputs(cfg, "cuda")
    d = M.dims_from_config(cfg)
    buf = M.MoELayerBuffers(d, device="cuda")
    M.forward(buf, inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"])
    bw = M.BackwardBuffers(d, device="cuda")
    h1, h2 = torch.zeros_like(buf.h), torch.zeros_like(buf.h)
    p1, p2 = torch.zeros_like(bw.pre), torch.zeros_like(bw.pre)
    M.moe_expert_ffn_up_train(d, buf.x_perm, buf.expert_offsets, inp["w1"], inp["w3"], h1, p1)
    M.moe_expert_ffn_up_train_gather(d, inp["x"], buf.row_to_pair, buf.expert_offsets, inp["w1"], inp["w3"], h2, p2)
    t1, t2 = torch.zeros_like(bw.xp_t), torch.full_like(bw.xp_t, float("nan"))  # padding must be written
    M.moe_group_transpose(d, buf.x_perm, cfg.D, buf.expert_offsets, bw.koff, t1)
    M.moe_group_transpose_gather(d, inp["x"], cfg.D, buf.expert_offsets, buf.row_to_pair, bw.koff, t2)
    torch.cuda.synchronize()
    N = int(buf.expert_offsets[-1].item())
    assert torch.equal(h1[:N], h2[:N]) and torch.equal(p1[:N], p2[:N])
    kend = int(bw.koff[-1].item())  # columns past koff[E] are not written
    assert torch.equal(t1[:, :kend], t2[:, :kend])
