"""CPU oracle for the one-GPU MoE layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package. The product path
(``combine_experts_amd``) never imports it, and this package never imports the
product path: the two share no code. Inputs come from ``workloads`` (seeded
generators that hold none of the layer's arithmetic).

Everything here is the plain definition of each step, in float64 (integer
steps exactly), written for a reader to check against the pages by eye. There
is no blocking, fusion or reordering beyond what the definitions state;
library primitives (matmul, stable sort, bincount, erf) serve as steps.

Pages cited (titles as they appear on the pages):
  [EPA2A]  "Expert Parallelism and All-to-All" (praveentn.live)
  [A2AC]   "Expert Parallelism > All-to-All Communication" (mbrenndoerfer.com)
  [CH10]   "Chapter 10: MoE parallelism" (infra-guide)
  [COMM]   "Expert Parallelism > Communication Overhead Analysis" (mbrenndoerfer.com)
  [EPLLM]  "Expert Parallelism in Large Language Models: How All-to-All Token
            Dispatch, Capacity Factors, and Parallel Folding Scale MoE
            Architectures" (llms.blog)

Parity status per function (the tests that pin each one):
  tests/test_oracle_pins.py: route_logits, route, select_topk, group_scores,
    select_group_limited, gate_weights, decisive_tokens, selection_key,
    round_to_f32, capacity, dispatch_layout, send_counts, dispatch_matrix,
    dispatch_volume_bytes, comm_volume_elements, permute, expert_ffn,
    expert_ffn_rows, silu, gelu, combine, layer_forward: pinned.
  tests/test_oracle_backward.py: layer_backward, gate_weights_backward,
    silu_grad, gelu_grad (central differences): pinned.
  tests/test_oracle_balance.py: router_probabilities, load_balance_stats,
    update_select_bias: pinned.
  tests/test_oracle_cluster.py: source_shards, recv_layout, cluster_forward,
    padded_layout, permute_padded, shared_expert_ffn, layer_forward_chunked:
    pinned.
  as_f64 is an exact upcast (no arithmetic).
  The absolute float values of y at the five workload shapes: parity unpinned
  (no page prints a numeric worked example of y; they are pinned only through
  the special cases and invariants in the tests).
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import __all__  # noqa: F401
