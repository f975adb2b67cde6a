"""Seeded synthetic workloads for the one-GPU MoE layer.

This module only draws inputs. It holds none of the layer's arithmetic: no
routing, no selection, no layout, no expert math. Both the CPU oracle
(``oracle/``) and the GPU library's callers (tests, ``bench.py``,
``__graft_entry__.smoke``) take their inputs from here, and from nowhere else.

Shapes follow the problem statement of the MoE pages: T tokens (T = B*S
flattened), hidden size D, E experts, top-k, expert hidden size F, an
optional capacity factor and an emulated expert-parallel (EP) size for the
send-buffer layout.

Recipe (every draw is seeded; see ``make_inputs``):

* x ~ N(0, 1), router weight W_g ~ N(0, 0.02), expert weights ~ N(0, 0.02),
  drawn in float32 and rounded to nearest-even into the config's dtype.
* ``switch_cap`` adds a per-expert router-logit bias ~ N(0, 0.5) (std 0.5).
* ``skew`` adds a Zipf-shaped logit bias ``-beta * 1.2 * ln(e + 1)``; beta is
  a stored constant calibrated offline (``skew_beta.json``, written by the
  oracle's calibration script) so that expert 0 receives about 3x its fair
  share of (token, expert) pairs.
* Each tensor (and each expert's W1/W3/W2) has its own seed derived from the
  config seed, so one expert can be drawn without drawing the others.

The same seed gives different values on a CPU generator and on a GPU
generator; every comparison uses one draw, copied to the host when the oracle
needs it.
"""
from __future__ import annotations

import dataclasses
import hashlib
import json
import os
from typing import Dict, Optional

import torch

__all__ = [
    "MoEConfig", "CONFIGS", "get_config", "make_inputs", "make_expert_weights",
    "GATE_SOFTMAX_TOPK", "GATE_SIGMOID_TOPK", "GATE_SOFTMAX_FULL",
    "ACT_SWIGLU", "ACT_GELU", "DT_F32", "DT_BF16", "torch_dtype",
]

# Enumerations shared with the C ABI's numeric codes (values fixed by the ABI).
GATE_SOFTMAX_TOPK = 0
GATE_SIGMOID_TOPK = 1
GATE_SOFTMAX_FULL = 2
ACT_SWIGLU = 0
ACT_GELU = 1
DT_F32 = 0
DT_BF16 = 1


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    D: int
    E: int
    top_k: int
    F: int
    act: int = ACT_SWIGLU
    dtype: int = DT_BF16
    gate: int = GATE_SOFTMAX_TOPK
    capacity_factor: float = 0.0      # <= 0 : dropless
    ep_size: int = 1
    ep_rank: int = 0
    n_groups: int = 0                 # 0 : no group limit
    topk_groups: int = 0
    bias: str = "none"                # "none" | "normal0.5" | "zipf"
    seed: int = 0
    desc: str = ""
    shared_F: int = 0                 # > 0 : one shared expert of this hidden size on every token

    def replace(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)

    @property
    def n_pairs(self) -> int:
        return self.T * self.top_k


CONFIGS: Dict[str, MoEConfig] = {
    "tiny_fp32": MoEConfig(
        name="tiny_fp32", T=256, D=128, E=8, top_k=2, F=256, dtype=DT_F32,
        gate=GATE_SOFTMAX_TOPK, ep_size=4, seed=101,
        desc="tiny fp32 layer: T=256 D=128 E=8 k=2 F=256 SwiGLU, EP 4"),
    "switch_cap": MoEConfig(
        name="switch_cap", T=4096, D=1024, E=16, top_k=1, F=4096, act=ACT_GELU,
        capacity_factor=1.25, ep_size=1, bias="normal0.5", seed=102,
        desc="Switch-style capacity/drop layer bf16: T=4096 D=1024 E=16 k=1 F=4096 GELU, CF 1.25"),
    "mixtral": MoEConfig(
        name="mixtral", T=8192, D=4096, E=8, top_k=2, F=14336, ep_size=8, seed=103,
        desc="Mixtral-8x7B-shaped layer bf16: T=8192 D=4096 E=8 k=2 F=14336 SwiGLU, EP 8"),
    "dsv3": MoEConfig(
        name="dsv3", T=16384, D=7168, E=256, top_k=8, F=2048, gate=GATE_SIGMOID_TOPK,
        ep_size=64, n_groups=8, topk_groups=4, seed=104,
        desc="DeepSeek-V3-shaped layer bf16: T=16384 D=7168 E=256 k=8 F=2048 SwiGLU, "
             "sigmoid gates, 8 groups / top-4 groups, EP 64"),
    "skew": MoEConfig(
        name="skew", T=32768, D=4096, E=64, top_k=4, F=1408, ep_size=16, bias="zipf", seed=105,
        desc="skewed-routing stress bf16: T=32768 D=4096 E=64 k=4 F=1408 SwiGLU, Zipf-shaped bias, EP 16"),
}

CONFIG_ORDER = ["tiny_fp32", "switch_cap", "mixtral", "dsv3", "skew"]

_SKEW_BETA_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "skew_beta.json")


def get_config(name: str, **overrides) -> MoEConfig:
    cfg = CONFIGS[name]
    return cfg.replace(**overrides) if overrides else cfg


def torch_dtype(dt: int) -> torch.dtype:
    return {DT_F32: torch.float32, DT_BF16: torch.bfloat16}[dt]


def _sub_seed(seed: int, *key) -> int:
    """A 63-bit seed for one named tensor, derived from the config seed."""
    h = hashlib.sha256(repr((int(seed),) + tuple(key)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, seed: int, *key) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_sub_seed(seed, *key))
    return g


def _normal(shape, std: float, dtype: torch.dtype, device, seed: int, *key) -> torch.Tensor:
    g = _gen(device, seed, *key)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t if dtype == torch.float32 else t.to(dtype)


def skew_beta(cfg: MoEConfig) -> float:
    """Stored Zipf-bias strength for the skewed-routing workload."""
    with open(_SKEW_BETA_FILE) as f:
        table = json.load(f)
    key = f"{cfg.name}:T{cfg.T}:seed{cfg.seed}"
    if key in table:
        return float(table[key])
    return float(table["default"])


def zipf_bias(E: int, beta: float, s: float = 1.2) -> torch.Tensor:
    """bias[e] = -beta * s * ln(e + 1): the logit of a Zipf(s) popularity profile scaled by beta."""
    e = torch.arange(E, dtype=torch.float64)
    return (-beta * s * torch.log(e + 1.0)).to(torch.float32)


def make_bias(cfg: MoEConfig, device="cpu") -> Optional[torch.Tensor]:
    if cfg.bias == "none":
        return None
    if cfg.bias == "normal0.5":
        return _normal((cfg.E,), 0.5, torch.float32, device, cfg.seed, "bias")
    if cfg.bias == "zipf":
        return zipf_bias(cfg.E, skew_beta(cfg)).to(device)
    raise ValueError(cfg.bias)


def make_select_bias(cfg: MoEConfig, device="cpu", std: Optional[float] = None) -> torch.Tensor:
    """A selection-only per-expert bias [E] float32, N(0, std^2).

    Default std: 0.05 under sigmoid gating (the scores it is added to lie in (0, 1)), 0.5 on
    logits otherwise -- large enough to move many selections, small enough to keep most.
    """
    if std is None:
        std = 0.05 if cfg.gate == GATE_SIGMOID_TOPK else 0.5
    return _normal((cfg.E,), std, torch.float32, device, cfg.seed, "select_bias")


def make_expert_weights(cfg: MoEConfig, e: int, device="cpu"):
    """(W1[e] [F,D], W3[e] [F,D] or None, W2[e] [D,F]) for one expert."""
    dt = torch_dtype(cfg.dtype)
    w1 = _normal((cfg.F, cfg.D), 0.02, dt, device, cfg.seed, "w1", e)
    w3 = _normal((cfg.F, cfg.D), 0.02, dt, device, cfg.seed, "w3", e) if cfg.act == ACT_SWIGLU else None
    w2 = _normal((cfg.D, cfg.F), 0.02, dt, device, cfg.seed, "w2", e)
    return w1, w3, w2


def make_inputs(cfg: MoEConfig, device="cpu", with_experts: bool = True) -> Dict[str, Optional[torch.Tensor]]:
    """All inputs of one layer call: x, w_gate, bias, and the stacked expert weights.

    x [T,D], w_gate [E,D] in the config dtype; bias [E] float32 or None;
    w1, w3 [E,F,D] and w2 [E,D,F] (w3 None for GELU experts). Expert weights
    are drawn one expert at a time into preallocated stacks. With shared_F > 0
    also shared_w1, shared_w3 [shared_F, D] and shared_w2 [D, shared_F].
    """
    dt = torch_dtype(cfg.dtype)
    out: Dict[str, Optional[torch.Tensor]] = {}
    out["x"] = _normal((cfg.T, cfg.D), 1.0, dt, device, cfg.seed, "x")
    out["w_gate"] = _normal((cfg.E, cfg.D), 0.02, dt, device, cfg.seed, "w_gate")
    out["bias"] = make_bias(cfg, device)
    if with_experts:
        w1 = torch.empty((cfg.E, cfg.F, cfg.D), dtype=dt, device=device)
        w3 = torch.empty((cfg.E, cfg.F, cfg.D), dtype=dt, device=device) if cfg.act == ACT_SWIGLU else None
        w2 = torch.empty((cfg.E, cfg.D, cfg.F), dtype=dt, device=device)
        for e in range(cfg.E):
            a, b, c = make_expert_weights(cfg, e, device)
            w1[e].copy_(a)
            if w3 is not None:
                w3[e].copy_(b)
            w2[e].copy_(c)
            del a, b, c
        out["w1"], out["w3"], out["w2"] = w1, w3, w2
    if cfg.shared_F > 0:
        fs = cfg.shared_F
        out["shared_w1"] = _normal((fs, cfg.D), 0.02, dt, device, cfg.seed, "shared_w1")
        out["shared_w3"] = (_normal((fs, cfg.D), 0.02, dt, device, cfg.seed, "shared_w3")
                            if cfg.act == ACT_SWIGLU else None)
        out["shared_w2"] = _normal((cfg.D, fs), 0.02, dt, device, cfg.seed, "shared_w2")
    return out


def fair_share(cfg: MoEConfig) -> float:
    return cfg.T * cfg.top_k / cfg.E


def dtype_bytes(cfg: MoEConfig) -> int:
    return 4 if cfg.dtype == DT_F32 else 2
