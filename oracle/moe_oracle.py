"""Plain float64 CPU definition of the MoE layer, step by step -- test infrastructure only.

Notation: T tokens, hidden D, E experts, top-k, expert hidden F. Pair id
p = t*k + j for token t and slot j (slot 0 = best expert). Arrays are numpy;
floating inputs are upcast exactly to float64 (bf16 and fp32 values are exact
in float64).

Readings taken where the pages are silent, ambiguous or garbled are marked
READING and listed in the design notes.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Tuple

import numpy as np
from scipy.special import erf as _erf

__all__ = [
    "GATE_SOFTMAX_TOPK", "GATE_SIGMOID_TOPK", "GATE_SOFTMAX_FULL", "ACT_SWIGLU", "ACT_GELU",
    "as_f64", "route_logits", "round_to_f32", "select_topk", "select_group_limited",
    "group_scores", "gate_weights", "route", "decisive_tokens", "capacity", "dispatch_layout",
    "send_counts", "dispatch_matrix", "permute", "silu", "gelu", "expert_ffn", "expert_ffn_rows",
    "combine", "comm_volume_elements", "dispatch_volume_bytes", "layer_forward",
    "router_probabilities", "load_balance_stats", "update_select_bias", "selection_key",
    "source_shards", "recv_layout", "cluster_forward", "padded_layout", "permute_padded",
    "shared_expert_ffn", "layer_forward_chunked",
    "silu_grad", "gelu_grad", "gate_weights_backward", "layer_backward",
]

GATE_SOFTMAX_TOPK = 0
GATE_SIGMOID_TOPK = 1
GATE_SOFTMAX_FULL = 2
ACT_SWIGLU = 0
ACT_GELU = 1


def as_f64(a) -> np.ndarray:
    """Exact upcast of a float array (numpy, or a torch tensor of fp32/bf16) to float64."""
    if hasattr(a, "detach"):  # torch tensor (bf16 has no numpy dtype): exact upcast on its side
        a = a.detach().cpu().double().numpy()
    return np.asarray(a, dtype=np.float64)


def round_to_f32(a: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest float32 (ties to even) and return them as float64."""
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------------------------
# Router: logits, selection, gates
# ----------------------------------------------------------------------------------------------

def route_logits(x, w_gate, bias=None) -> np.ndarray:
    """Router logits l[t,e] = sum_d x[t,d] * W_g[e,d] + bias[e].

    [EPLLM] section "The Execution Pipeline", step 1 (Router Gating): the
    router scores each local token against all E experts with W_g x_t.
    [EPLLM] "The Distributed MoE Dilemma": G(x) in R^E per token.
    The optional per-expert bias is added to the logits (it moves both the
    selection and the gate values; READING for the Switch-style workload).
    """
    x = as_f64(x)
    wg = as_f64(w_gate)
    l = x @ wg.T
    if bias is not None:
        l = l + as_f64(bias)[None, :]
    return l


def select_topk(l: np.ndarray, k: int, eligible: Optional[np.ndarray] = None) -> np.ndarray:
    """Top-k expert indices per token, slot order = descending score.

    [EPLLM] "The Execution Pipeline" step 1 and the layer equation of "The
    Distributed MoE Dilemma" (sum over TopK(G(x), k)).
    Ordering key is (-l[t,e], e): exact ties go to the lowest expert index.
    Experts with ``eligible[t,e] == False`` are never chosen.
    """
    l = np.asarray(l, dtype=np.float64)
    T, E = l.shape
    key = l.copy()
    if eligible is not None:
        key = np.where(eligible, key, -np.inf)
    # stable sort of -key keeps equal keys in ascending expert order
    order = np.argsort(-key, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def group_scores(s: np.ndarray, n_groups: int, per_group_top: int) -> np.ndarray:
    """Score of each expert group: the sum of its ``per_group_top`` largest member scores.

    READING of node-limited routing ([EPA2A] "Three ways the system fights
    back": a token may reach at most 4 nodes, chosen before per-expert
    selection). Groups are contiguous blocks of E/n_groups experts, the same
    contiguous map as expert -> device.
    """
    T, E = s.shape
    g = s.reshape(T, n_groups, E // n_groups)
    top = -np.sort(-g, axis=2)[:, :, :per_group_top]
    return top.sum(axis=2)


def select_group_limited(l: np.ndarray, k: int, n_groups: int, topk_groups: int,
                         score: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Group-limited top-k: keep the best ``topk_groups`` groups, then top-k experts inside them.

    Group ranking uses ``group_scores(score, ...)`` with k/topk_groups members
    per group (READING), ordered by (-score_g, g); expert selection inside the
    kept groups orders by (-l, e). Returns (topk_idx [T,k], kept_groups [T,topk_groups]).
    """
    T, E = l.shape
    per_group_top = max(1, k // topk_groups)
    gs = round_to_f32(group_scores(score, n_groups, per_group_top))
    gorder = np.argsort(-gs, axis=1, kind="stable")[:, :topk_groups]
    gsize = E // n_groups
    eligible = np.zeros((T, E), dtype=bool)
    for j in range(topk_groups):
        g = gorder[:, j]
        for m in range(gsize):
            eligible[np.arange(T), g * gsize + m] = True
    return select_topk(l, k, eligible), gorder


def gate_weights(l: np.ndarray, topk_idx: np.ndarray, mode: int) -> np.ndarray:
    """Gate values g[t,j] for the selected experts.

    SOFTMAX_TOPK: g = Softmax(TopK(W_g x_t, k)) -- [EPLLM] "The Execution
      Pipeline" step 1: softmax over the k selected logits only (renormalised).
    SIGMOID_TOPK: g_j = sigmoid(l_j) / sum_i sigmoid(l_i) over the k selected
      (READING for the DeepSeek-V3-shaped workload; the pages name DeepSeek-V3
      routing in [EPA2A] without its gate formula).
    SOFTMAX_FULL: g_j = softmax over all E logits, evaluated at the selected
      experts (no renormalisation) -- the un-renormalised form of the layer
      equation in [EPLLM] "The Distributed MoE Dilemma".
    """
    l = np.asarray(l, dtype=np.float64)
    T = l.shape[0]
    sel = np.take_along_axis(l, topk_idx, axis=1)
    if mode == GATE_SOFTMAX_TOPK:
        m = sel.max(axis=1, keepdims=True)
        w = np.exp(sel - m)
        return w / w.sum(axis=1, keepdims=True)
    if mode == GATE_SIGMOID_TOPK:
        s = 1.0 / (1.0 + np.exp(-sel))
        return s / s.sum(axis=1, keepdims=True)
    if mode == GATE_SOFTMAX_FULL:
        m = l.max(axis=1, keepdims=True)
        w = np.exp(l - m)
        p = w / w.sum(axis=1, keepdims=True)
        return np.take_along_axis(p, topk_idx, axis=1)
    raise ValueError(f"unknown gate mode {mode}")


def selection_key(l32: np.ndarray, gate: int, select_bias) -> np.ndarray:
    """Score that a selection-only bias ranks by: (sigmoid(l) under sigmoid gating, else l) + b.

    READING of the bias-adjusted routing scores ([CH10] section 4; [EPLLM]
    "Modern Dropless Dynamic Dispatch"): each term is rounded to float32 as
    the kernel holds it.
    """
    b = np.asarray(as_f64(select_bias), dtype=np.float64)[None, :]
    if gate == GATE_SIGMOID_TOPK:
        return round_to_f32(round_to_f32(1.0 / (1.0 + np.exp(-np.asarray(l32, dtype=np.float64)))) + b)
    return round_to_f32(np.asarray(l32, dtype=np.float64) + b)


def route(x, w_gate, bias, k: int, gate: int, n_groups: int = 0, topk_groups: int = 0,
          select_bias=None) -> Dict[str, np.ndarray]:
    """Router step end to end: logits, selection, gates.

    Selection decisions are taken on the logits rounded to float32, the
    precision the GPU kernel decides in; exact float32 ties go to the lowest
    expert index. Gate values use the float64 logits.

    ``select_bias`` (optional, [E]): a per-expert bias that moves the selection
    only, never the gate values -- the bias-adjusted routing scores of
    aux-loss-free balancing ([CH10] section 4; [EPLLM] "Modern Dropless
    Dynamic Dispatch"). READING: it is added to the score the selection ranks
    by (the sigmoid score under sigmoid gating, the logit otherwise), in
    float32, and group scores are taken on the biased scores.
    """
    l64 = route_logits(x, w_gate, bias)
    l32 = round_to_f32(l64)
    kept_groups = None
    if select_bias is not None:
        key = selection_key(l32, gate, select_bias)
        if n_groups and n_groups > 0:
            idx, kept_groups = select_group_limited(key, k, n_groups, topk_groups, key)
        else:
            idx = select_topk(key, k)
    elif n_groups and n_groups > 0:
        s = 1.0 / (1.0 + np.exp(-l32)) if gate == GATE_SIGMOID_TOPK else l32
        idx, kept_groups = select_group_limited(l32, k, n_groups, topk_groups, s)
    else:
        idx = select_topk(l32, k)
    g = gate_weights(l64, idx, gate)
    out = {"logits": l64, "topk_idx": idx, "topk_gate": g}
    if kept_groups is not None:
        out["kept_groups"] = kept_groups
    return out


def decisive_tokens(l: np.ndarray, k: int, margin: float = 1e-3, n_groups: int = 0,
                    topk_groups: int = 0, gate: int = GATE_SOFTMAX_TOPK) -> Dict[str, np.ndarray]:
    """Tokens whose selection cannot flip under float32 rounding of the logits.

    ``set``: the k-th vs (k+1)-th logit margin among eligible experts exceeds
    ``margin`` (and, with a group limit, the last kept vs first dropped group
    score margin exceeds it too). ``order``: additionally every adjacent
    margin among the top k exceeds ``margin``, so slot order is unique.
    """
    l = np.asarray(l, dtype=np.float64)
    T, E = l.shape
    ok_set = np.ones(T, dtype=bool)
    eligible = None
    if n_groups and n_groups > 0:
        s = 1.0 / (1.0 + np.exp(-l)) if gate == GATE_SIGMOID_TOPK else l
        gs = group_scores(s, n_groups, max(1, k // topk_groups))
        gsorted = -np.sort(-gs, axis=1)
        if topk_groups < n_groups:
            ok_set &= (gsorted[:, topk_groups - 1] - gsorted[:, topk_groups]) > margin
        gorder = np.argsort(-gs, axis=1, kind="stable")[:, :topk_groups]
        gsize = E // n_groups
        eligible = np.zeros((T, E), dtype=bool)
        for j in range(topk_groups):
            for m in range(gsize):
                eligible[np.arange(T), gorder[:, j] * gsize + m] = True
    key = l if eligible is None else np.where(eligible, l, -np.inf)
    srt = -np.sort(-key, axis=1)
    if k < E:
        nxt = srt[:, k]
        ok_set &= ~np.isfinite(nxt) | ((srt[:, k - 1] - nxt) > margin)
    ok_order = ok_set.copy()
    for j in range(k - 1):
        ok_order &= (srt[:, j] - srt[:, j + 1]) > margin
    return {"set": ok_set, "order": ok_order}


# ----------------------------------------------------------------------------------------------
# Dispatch layout: counts, capacity, stable grouping by expert, per-rank send layout
# ----------------------------------------------------------------------------------------------

def capacity(capacity_factor: float, T: int, k: int, E: int) -> int:
    """Expert capacity C = ceil(CF * k * T / E), T = B*S.

    [EPLLM] "Static Capacity Factors and Token Dropping", capacity equation.
    Evaluated once in IEEE double exactly as written. CF <= 0 means dropless:
    C = T*k (no expert can receive more pairs than exist).
    """
    if capacity_factor is None or capacity_factor <= 0:
        return T * k
    return int(math.ceil(capacity_factor * (k * T) / E))


def dispatch_layout(topk_idx: np.ndarray, E: int, ep_size: int, C: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Group (token, expert) pairs into contiguous per-expert rows; per-rank send counts.

    [EPA2A] "The two exchanges" (dispatch: each device sorts its tokens by
    destination expert into groups); [EPLLM] "The Execution Pipeline" step 1
    (each token is replicated k times, tagged with expert and destination
    rank) and step 2 (local permutation into contiguous per-rank buffers);
    [A2AC] the dispatch example (destination device = expert //
    experts_per_device; send counts = per-device bincount).

    READINGS: rows are ordered by (expert ascending, pair id ascending) --
    stable, which the example's unstable device-only sort is not. With a
    capacity C ([EPLLM] "Static Capacity Factors"), each expert keeps its
    first C pairs in pair-id (token) order and drops the rest; dropped pairs
    get row -1. The layout is compact (no padding slots).
    """
    idx = np.asarray(topk_idx, dtype=np.int64)
    T, k = idx.shape
    P = T * k
    flat = idx.reshape(-1)                          # pair id p = t*k + j
    if C is None:
        C = P
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    order = np.argsort(flat, kind="stable")         # pairs by (expert, pair id)
    first = np.concatenate([[0], np.cumsum(counts)])[:E]
    rank_in_expert = np.empty(P, dtype=np.int64)
    rank_in_expert[order] = np.arange(P) - first[flat[order]]
    kept = rank_in_expert < C
    kept_counts = np.minimum(counts, C)
    offsets = np.concatenate([[0], np.cumsum(kept_counts)]).astype(np.int64)
    N = int(offsets[E])
    pair_to_row = np.where(kept, offsets[flat] + rank_in_expert, -1).astype(np.int64)
    row_to_pair = np.full(P, -1, dtype=np.int64)
    row_to_pair[pair_to_row[kept]] = np.arange(P)[kept]
    epr = E // ep_size                              # experts per rank, contiguous blocks
    rank_counts = kept_counts.reshape(ep_size, epr).sum(axis=1)
    rank_offsets = offsets[::epr].copy()            # o_{r*E/EP}, r = 0..EP
    return {
        "expert_counts": counts, "kept_counts": kept_counts, "expert_offsets": offsets,
        "rank_counts": rank_counts, "rank_offsets": rank_offsets,
        "pair_to_row": pair_to_row, "row_to_pair": row_to_pair, "n_kept": N, "capacity": C,
        "n_dropped": P - N,
    }


def send_counts(topk_idx: np.ndarray, E: int, world_size: int) -> np.ndarray:
    """Pairs bound for each device: bincount(expert // (E / world_size)).

    [A2AC] the dispatch example (destination = expert // experts_per_device,
    send counts by bincount with one bin per device).
    """
    dest = np.asarray(topk_idx, dtype=np.int64).reshape(-1) // (E // world_size)
    return np.bincount(dest, minlength=world_size)


def dispatch_matrix(topk_idx_per_src: np.ndarray, E: int, n_dev: int) -> np.ndarray:
    """[src, dst] counts of (token, expert) pairs for n_dev source shards.

    [A2AC] the routing simulation: each source device's pairs are counted by
    destination device = expert // (E / n_dev).
    """
    out = np.zeros((n_dev, n_dev), dtype=np.int64)
    for src in range(n_dev):
        out[src] = send_counts(topk_idx_per_src[src], E, n_dev)
    return out


def source_shards(T: int, n_src: int):
    """Token ranges of n_src equal source shards: shard s owns tokens [s*T/n_src, (s+1)*T/n_src).

    READING of the routing simulation in [A2AC]: every device routes the same
    number of local tokens; shards are contiguous.
    """
    if n_src < 1 or T % n_src != 0:
        raise ValueError("T must split evenly over the source shards")
    ts = T // n_src
    return [(s * ts, (s + 1) * ts) for s in range(n_src)]


def recv_layout(src_expert_offsets: np.ndarray, E: int, n_dst: int, r: int, src_stride: int) -> Dict[str, np.ndarray]:
    """Receive side of destination rank r: which sent rows it gets and how it regroups them.

    [EPA2A] "The two exchanges": after the dispatch exchange each device holds,
    from every source, a chunk of rows sorted by its local experts; the grouped
    GEMM wants all rows of one local expert together. [A2AC]: rank r owns
    experts [r*E/n_dst, (r+1)*E/n_dst).

    ``src_expert_offsets[s]`` is source s's own compact layout (expert offsets,
    E+1 entries); source s's sent rows live at rows s*src_stride + j of one
    concatenated send buffer. READING: the regrouped order is (local expert,
    source, source row order).

    Returns ``recv_counts[s]`` (rows s sends to r), ``expert_offsets`` [epr+1]
    of the regrouped rows, and ``grouped_to_src_row`` [n]: the send-buffer row
    of each regrouped row.
    """
    off = np.asarray(src_expert_offsets, dtype=np.int64)
    n_src = off.shape[0]
    epr = E // n_dst
    lo, hi = r * epr, (r + 1) * epr
    counts = off[:, lo + 1:hi + 1] - off[:, lo:hi]             # [n_src, epr]
    recv_counts = counts.sum(axis=1)
    exp_off = np.concatenate([[0], np.cumsum(counts.sum(axis=0))]).astype(np.int64)
    rows = []
    for el in range(epr):
        for s in range(n_src):
            start = s * src_stride + off[s, lo + el]
            rows.extend(range(int(start), int(start + counts[s, el])))
    return {"recv_counts": recv_counts, "expert_offsets": exp_off,
            "grouped_to_src_row": np.asarray(rows, dtype=np.int64)}


def cluster_forward(inputs: Dict, cfg, n_ep: int) -> Dict[str, object]:
    """The layer on n_ep emulated devices: shard, route, send layout, exchange, regroup, FFN, return, combine.

    [EPA2A] "The two exchanges" (dispatch then combine all-to-all around the
    expert compute); [EPLLM] "The Execution Pipeline" steps 1-6; [A2AC]
    (contiguous expert -> device map, per-device send counts). Dropless.
    Every device routes its own shard; device r runs its E/n_ep experts on the
    rows it receives, regrouped per local expert; the outputs travel back to
    their source and are combined there. Returns y [T, D] and the [src, dst]
    kept-row matrix.
    """
    T, E, k, D = cfg.T, cfg.E, cfg.top_k, cfg.D
    x = as_f64(inputs["x"])
    shards = source_shards(T, n_ep)
    ts = T // n_ep
    stride = ts * k
    epr = E // n_ep
    w1, w3, w2 = inputs["w1"], inputs.get("w3"), inputs["w2"]
    send = np.zeros((n_ep * stride, D))
    src_off = np.zeros((n_ep, E + 1), dtype=np.int64)
    per_src = []
    for s, (a, b) in enumerate(shards):
        r_s = route(inputs["x"][a:b], inputs["w_gate"], inputs.get("bias"), k, cfg.gate, cfg.n_groups,
                    cfg.topk_groups)
        lay = dispatch_layout(r_s["topk_idx"], E, n_ep, None)
        n = lay["n_kept"]
        send[s * stride: s * stride + n] = permute(x[a:b], lay["row_to_pair"], k, n)
        src_off[s] = lay["expert_offsets"]
        per_src.append((r_s, lay))
    back = np.zeros_like(send)
    matrix = np.zeros((n_ep, n_ep), dtype=np.int64)
    for r in range(n_ep):
        rl = recv_layout(src_off, E, n_ep, r, stride)
        matrix[:, r] = rl["recv_counts"]
        g2s = rl["grouped_to_src_row"]
        grouped = send[g2s]
        w1r = w1[r * epr:(r + 1) * epr]
        w3r = None if w3 is None else w3[r * epr:(r + 1) * epr]
        w2r = w2[r * epr:(r + 1) * epr]
        y_grouped = expert_ffn(grouped, rl["expert_offsets"], w1r, w3r, w2r, cfg.act)
        back[g2s] = y_grouped
    y = np.zeros((T, D))
    for s, (a, b) in enumerate(shards):
        r_s, lay = per_src[s]
        y[a:b] = combine(back[s * stride:(s + 1) * stride], lay["pair_to_row"], r_s["topk_gate"], ts, k)
    return {"y": y, "matrix": matrix, "src_expert_offsets": src_off}


def padded_layout(topk_idx: np.ndarray, E: int, C: int) -> Dict[str, object]:
    """GShard-style fixed-capacity layout: expert e owns slots [e*C, (e+1)*C) of an [E*C] buffer.

    [EPLLM] "Static Capacity Factors and Token Dropping": each expert gets a
    buffer of C = ceil(CF*k*T/E) rows; pairs past C are dropped and unused
    slots are padding. Kept pairs are the same as in the compact layout with
    the same C (first C pairs of each expert in pair-id order); pair p of
    expert e with rank q < C goes to slot e*C + q.
    Returns pair_to_slot [T*k] (-1 dropped), slot_to_pair [E*C] (-1 padding),
    padded_offsets [E+1] = e*C, and the padding (empty slots) count.
    """
    flat = np.asarray(topk_idx, dtype=np.int64).reshape(-1)
    P = flat.shape[0]
    pair_to_slot = np.full(P, -1, dtype=np.int64)
    slot_to_pair = np.full(E * C, -1, dtype=np.int64)
    seen = np.zeros(E, dtype=np.int64)
    for p in range(P):                      # pair-id order: rank within the expert
        e = int(flat[p])
        q = int(seen[e])
        seen[e] += 1
        if q < C:
            pair_to_slot[p] = e * C + q
            slot_to_pair[e * C + q] = p
    return {"pair_to_slot": pair_to_slot, "slot_to_pair": slot_to_pair,
            "padded_offsets": np.arange(E + 1, dtype=np.int64) * C,
            "padding": int((slot_to_pair < 0).sum()), "n_kept": int((pair_to_slot >= 0).sum())}


def permute_padded(x, slot_to_pair: np.ndarray, k: int) -> np.ndarray:
    """x_pad[s] = x[slot_to_pair[s] // k] for filled slots, 0 for padding slots."""
    xa = as_f64(x)
    s2p = np.asarray(slot_to_pair, dtype=np.int64)
    out = np.zeros((s2p.shape[0], xa.shape[1]))
    filled = s2p >= 0
    out[filled] = xa[s2p[filled] // k]
    return out


# ----------------------------------------------------------------------------------------------
# Permute, expert FFN, combine
# ----------------------------------------------------------------------------------------------

def permute(x, row_to_pair: np.ndarray, k: int, n_rows: Optional[int] = None) -> np.ndarray:
    """x_perm[r] = x[row_to_pair[r] // k] for the kept rows r < N.

    [EPLLM] "The Execution Pipeline" step 2 (tokens are physically reordered
    into contiguous buffers). Values are copied unchanged.
    """
    r2p = np.asarray(row_to_pair, dtype=np.int64)
    if n_rows is None:
        n_rows = int((r2p >= 0).sum())
    xa = np.asarray(x) if not hasattr(x, "detach") else as_f64(x)
    return xa[r2p[:n_rows] // k]


def silu(a: np.ndarray) -> np.ndarray:
    """SiLU(a) = a * sigmoid(a)."""
    return a / (1.0 + np.exp(-a))


def gelu(a: np.ndarray) -> np.ndarray:
    """Exact GELU: a * Phi(a) = a/2 * (1 + erf(a / sqrt 2)) (READING: the erf form)."""
    return 0.5 * a * (1.0 + _erf(a / math.sqrt(2.0)))


def _expert_rows(rows: np.ndarray, w1, w3, w2, act: int) -> np.ndarray:
    a = rows @ as_f64(w1).T                    # [n, F]
    if act == ACT_SWIGLU:
        b = rows @ as_f64(w3).T                # [n, F]
        h = silu(a) * b                        # SiLU(W1 x) * (W3 x)
    elif act == ACT_GELU:
        h = gelu(a)
    else:
        raise ValueError(f"unknown activation {act}")
    return h @ as_f64(w2).T                    # [n, D]


def expert_ffn(x_perm, expert_offsets: np.ndarray, w1, w3, w2, act: int) -> np.ndarray:
    """Per-expert FFN over each expert's contiguous rows.

    [EPLLM] "The Execution Pipeline" step 4: all rows bound for one local
    expert go through one batched GEMM; the expert is
    W2 * (SiLU(W1 h) (*) (W3 h)) -- READING of the garbled parenthesisation as
    SwiGLU, SiLU applied to W1 h alone. GELU experts use two matrices:
    W2 * GELU(W1 h) ([COMM]: two matrix multiplications per token).
    Weights: W1, W3 [E,F,D]; W2 [E,D,F].
    """
    xp = as_f64(x_perm)
    off = np.asarray(expert_offsets, dtype=np.int64)
    E = off.shape[0] - 1
    out = np.zeros((int(off[E]), xp.shape[1] if xp.ndim == 2 else 0), dtype=np.float64)
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi <= lo:
            continue
        out[lo:hi] = _expert_rows(xp[lo:hi], w1[e], None if w3 is None else w3[e], w2[e], act)
    return out


def expert_ffn_rows(rows, experts: np.ndarray, w1, w3, w2, act: int) -> np.ndarray:
    """The same expert FFN for an arbitrary set of rows, row i going through expert experts[i].

    Used to check sampled rows at full size; ``w1`` etc. may be callables
    ``e -> matrix`` so one expert's weights are fetched at a time.
    """
    xr = as_f64(rows)
    ex = np.asarray(experts, dtype=np.int64)
    D = xr.shape[1]
    out = np.zeros((xr.shape[0], D), dtype=np.float64)
    get = (lambda w, e: None if w is None else (w(e) if callable(w) else w[e]))
    for e in np.unique(ex):
        sel = np.nonzero(ex == e)[0]
        out[sel] = _expert_rows(xr[sel], get(w1, e), get(w3, e), get(w2, e), act)
    return out


def combine(y_perm, pair_to_row: np.ndarray, topk_gate, T: int, k: int) -> np.ndarray:
    """y[t] = sum over kept slots j of g[t,j] * y_perm[pair_to_row[t*k + j]].

    [EPLLM] "The Execution Pipeline" step 6 (restore order, scale each of the
    k outputs by its gate and sum them; the residual is added outside) and the
    layer equation of "The Distributed MoE Dilemma". A dropped pair adds
    nothing, so a token with every pair dropped comes out as exactly 0
    (READING; gates are not renormalised after drops).
    """
    yp = as_f64(y_perm)
    g = as_f64(topk_gate).reshape(T, k)
    p2r = np.asarray(pair_to_row, dtype=np.int64).reshape(T, k)
    D = yp.shape[1]
    y = np.zeros((T, D), dtype=np.float64)
    for j in range(k):
        rows = p2r[:, j]
        kept = rows >= 0
        y[kept] += g[kept, j][:, None] * yp[rows[kept]]
    return y


def router_probabilities(l: np.ndarray, gate: int) -> np.ndarray:
    """Router probability of every expert for every token (all E, before top-k).

    Softmax over the E logits for softmax gates; the sigmoid scores
    normalised over all E for sigmoid gates (READING: the pages give P_i no
    formula beyond naming it expert i's router probability).
    """
    l = np.asarray(l, dtype=np.float64)
    if gate == GATE_SIGMOID_TOPK:
        s = 1.0 / (1.0 + np.exp(-l))
        return s / s.sum(axis=1, keepdims=True)
    m = l.max(axis=1, keepdims=True)
    w = np.exp(l - m)
    return w / w.sum(axis=1, keepdims=True)


def load_balance_stats(expert_counts: np.ndarray, probs: np.ndarray, k: int, alpha: float) -> Dict[str, object]:
    """Auxiliary load-balancing loss L_aux = alpha * E * sum_i f_i * P_i.

    [EPLLM] "Static Capacity Factors and Token Dropping", auxiliary-loss
    equation. f_i is expert i's share of the routed pairs and P_i its mean
    router probability. READING: f_i = c_i / (T*k) (pairs counted before
    any capacity cut) and P_i = mean over tokens of router_probabilities.
    Also returns the
    imbalance max_i c_i / mean_i c_i ([EPA2A] "When it breaks": one expert
    with several times its share stalls the layer).
    """
    c = np.asarray(expert_counts, dtype=np.float64)
    p = np.asarray(probs, dtype=np.float64)
    T, E = p.shape
    f = c / (T * k)
    P = p.mean(axis=0)
    return {"f": f, "P": P, "aux_loss": float(alpha * E * np.sum(f * P)),
            "imbalance": float(c.max() / c.mean()) if c.mean() > 0 else 0.0}


def update_select_bias(select_bias: np.ndarray, expert_counts: np.ndarray, gamma: float) -> np.ndarray:
    """One aux-loss-free balancing step: b_i <- b_i + gamma * sign(mean load - load_i).

    [CH10] section 4 (aux-loss-free balancing by bias adjustment); [EPLLM]
    "Modern Dropless Dynamic Dispatch" (dynamically adjusted bias terms on
    routing scores). READING: the sign rule with step gamma (the page names
    the mechanism, not the rule), in float32 like the bias itself.
    """
    b = np.asarray(select_bias, dtype=np.float32)
    c = np.asarray(expert_counts, dtype=np.int64)
    E = c.shape[0]
    # sign(mean - c_i) compared in integers: mean*E = sum(c)
    d = np.sign(c.sum() - E * c).astype(np.float32)
    return (b + np.float32(gamma) * d).astype(np.float32)


# ----------------------------------------------------------------------------------------------
# Volume accounting
# ----------------------------------------------------------------------------------------------

def comm_volume_elements(n_kept: int, D: int) -> int:
    """Elements moved by dispatch + combine: 2 * (kept pairs) * D.

    [COMM] the per-layer volume equation V = 2*B*S*K*D; with capacity drops
    the kept-pair count replaces B*S*K (READING).
    """
    return 2 * int(n_kept) * int(D)


def dispatch_volume_bytes(n_remote: int, D: int, elem_bytes: int) -> int:
    """Bytes one device sends in dispatch: its remote pairs * D * sizeof(dtype).

    [EPLLM] "Communication Volume and Hardware Topology", the per-GPU dispatch
    volume equation (B*S*k*H*(EP-1)/EP*sizeof under uniform routing; here the
    exact remote-pair count replaces its expectation).
    """
    return int(n_remote) * int(D) * int(elem_bytes)


# ----------------------------------------------------------------------------------------------
# The whole layer
# ----------------------------------------------------------------------------------------------

def silu_grad(a: np.ndarray) -> np.ndarray:
    """d/da SiLU(a) = s(a) * (1 + a * (1 - s(a))), s the logistic sigmoid."""
    s = 1.0 / (1.0 + np.exp(-a))
    return s * (1.0 + a * (1.0 - s))


def gelu_grad(a: np.ndarray) -> np.ndarray:
    """d/da GELU(a) = Phi(a) + a * phi(a) (exact erf form)."""
    return 0.5 * (1.0 + _erf(a / math.sqrt(2.0))) + a * np.exp(-0.5 * a * a) / math.sqrt(2.0 * math.pi)


def gate_weights_backward(l: np.ndarray, topk_idx: np.ndarray, mode: int, dgate: np.ndarray) -> np.ndarray:
    """Gradient of the gate values with respect to all E logits (the selection held fixed).

    The chain rule through each gate definition of ``gate_weights``:
    SOFTMAX_TOPK  g = softmax(l_sel): dl_sel = g * (dg - sum_j g_j dg_j).
    SIGMOID_TOPK  g_j = s_j / S, s = sigmoid(l_sel), S = sum s:
                  dl_sel_j = s_j (1 - s_j) (dg_j - sum_i g_i dg_i) / S.
    SOFTMAX_FULL  g = p[sel], p = softmax over all E: with dp = dg scattered to
                  the selected experts, dl = p * (dp - sum_e p_e dp_e).
    Unselected logits get 0 except under SOFTMAX_FULL.
    """
    l = np.asarray(l, dtype=np.float64)
    T, E = l.shape
    dg = np.asarray(dgate, dtype=np.float64)
    idx = np.asarray(topk_idx, dtype=np.int64)
    dl = np.zeros((T, E))
    sel = np.take_along_axis(l, idx, axis=1)
    if mode == GATE_SOFTMAX_TOPK:
        m = sel.max(axis=1, keepdims=True)
        w = np.exp(sel - m)
        g = w / w.sum(axis=1, keepdims=True)
        dsel = g * (dg - (g * dg).sum(axis=1, keepdims=True))
        np.put_along_axis(dl, idx, dsel, axis=1)
    elif mode == GATE_SIGMOID_TOPK:
        sg = 1.0 / (1.0 + np.exp(-sel))
        S = sg.sum(axis=1, keepdims=True)
        g = sg / S
        dsel = sg * (1.0 - sg) * (dg - (g * dg).sum(axis=1, keepdims=True)) / S
        np.put_along_axis(dl, idx, dsel, axis=1)
    elif mode == GATE_SOFTMAX_FULL:
        m = l.max(axis=1, keepdims=True)
        w = np.exp(l - m)
        pr = w / w.sum(axis=1, keepdims=True)
        dp = np.zeros((T, E))
        np.put_along_axis(dp, idx, dg, axis=1)
        dl = pr * (dp - (pr * dp).sum(axis=1, keepdims=True))
    else:
        raise ValueError(f"unknown gate mode {mode}")
    return dl


def layer_backward(inputs: Dict, cfg, fwd: Dict, dy) -> Dict[str, np.ndarray]:
    """Gradients of the layer output y (from ``layer_forward``) for an upstream gradient dy [T, D].

    The chain rule through the forward's steps in reverse, the routing decision
    (selection and drops) held fixed: combine -> expert FFN -> permute ->
    router. dy_perm[row] = g * dy[t]; dgate = <dy[t], y_perm[row]>; per
    expert dh = dy_perm W2, dW2 = dy_perm^T h; through the activation
    (SwiGLU: da1 = dh * a3 * SiLU'(a1), da3 = dh * SiLU(a1); GELU: da1 = dh *
    GELU'(a1)); dx_perm = da1 W1 + da3 W3, dW1 = da1^T x_perm, dW3 = da3^T
    x_perm; dx[t] = sum of its kept rows' dx_perm + the router's dl W_g, with
    dl from ``gate_weights_backward``; dW_g = dl^T x; dbias = sum_t dl.
    [EPLLM] "The Execution Pipeline" (the forward steps); the backward is the
    chain rule through them (the pages name backward only as training's other
    half). No shared expert.
    """
    x = as_f64(inputs["x"])
    T, D, E, k = cfg.T, cfg.D, cfg.E, cfg.top_k
    dyv = as_f64(dy)
    p2r = np.asarray(fwd["pair_to_row"], dtype=np.int64).reshape(T, k)
    r2p = np.asarray(fwd["row_to_pair"], dtype=np.int64)
    off = np.asarray(fwd["expert_offsets"], dtype=np.int64)
    N = int(off[E])
    g = np.asarray(fwd["topk_gate"], dtype=np.float64).reshape(T, k)
    yp = np.asarray(fwd["y_perm"], dtype=np.float64)
    xp = np.asarray(fwd["x_perm"], dtype=np.float64)
    tok = r2p[:N] // k
    slot = r2p[:N] % k
    dyp = g[tok, slot][:, None] * dyv[tok]                      # [N, D]
    dgate = np.zeros((T, k))
    dgate[tok, slot] = (dyv[tok] * yp[:N]).sum(axis=1)
    F = cfg.F
    dw1 = np.zeros((E, F, D))
    dw3 = np.zeros((E, F, D)) if cfg.act == ACT_SWIGLU else None
    dw2 = np.zeros((E, D, F))
    dxp = np.zeros((N, D))
    pre1 = np.zeros((N, F))
    pre3 = np.zeros((N, F))
    hh = np.zeros((N, F))
    dh_all = np.zeros((N, F))
    da1_all = np.zeros((N, F))
    da3_all = np.zeros((N, F))
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi <= lo:
            continue
        xr = xp[lo:hi]
        w1 = as_f64(inputs["w1"][e])
        w2 = as_f64(inputs["w2"][e])
        a1 = xr @ w1.T
        if cfg.act == ACT_SWIGLU:
            w3 = as_f64(inputs["w3"][e])
            a3 = xr @ w3.T
            h = silu(a1) * a3
        else:
            a3 = None
            h = gelu(a1)
        dh = dyp[lo:hi] @ w2                                     # [n, F]
        dw2[e] = dyp[lo:hi].T @ h
        if cfg.act == ACT_SWIGLU:
            da1 = dh * a3 * silu_grad(a1)
            da3 = dh * silu(a1)
            dxp[lo:hi] = da1 @ w1 + da3 @ w3
            dw3[e] = da3.T @ xr
            pre3[lo:hi], da3_all[lo:hi] = a3, da3
        else:
            da1 = dh * gelu_grad(a1)
            dxp[lo:hi] = da1 @ w1
        dw1[e] = da1.T @ xr
        pre1[lo:hi], hh[lo:hi], dh_all[lo:hi], da1_all[lo:hi] = a1, h, dh, da1
    dx = np.zeros((T, D))
    np.add.at(dx, tok, dxp)
    dl = gate_weights_backward(fwd["logits"], np.asarray(fwd["topk_idx"]).reshape(T, k), cfg.gate, dgate)
    wg = as_f64(inputs["w_gate"])
    dx = dx + dl @ wg
    return {"dx": dx, "dw_gate": dl.T @ x, "dbias": dl.sum(axis=0), "dw1": dw1, "dw3": dw3, "dw2": dw2,
            "dgate": dgate, "dl": dl, "dy_perm": dyp, "dh": dh_all, "da1": da1_all, "da3": da3_all,
            "dx_perm": dxp, "a1": pre1, "a3": pre3, "h": hh}


def shared_expert_ffn(x, w1, w3, w2, act: int) -> np.ndarray:
    """A shared expert: the same expert FFN applied to every token, with gate 1.

    READING: [EPLLM] "Overlapping All-to-All with Computation" names the shared
    expert computation that the dispatch of the next layer overlaps, without its
    formula; it is read as DeepSeek-V3's shared expert: one always-active
    expert of the routed experts' kind whose output is added to the routed sum.
    """
    return _expert_rows(as_f64(x), w1, w3, w2, act)


def layer_forward_chunked(inputs: Dict, cfg, n_chunks: int) -> Dict[str, np.ndarray]:
    """The layer on n_chunks contiguous micro-batches of T/n_chunks tokens, one after the other.

    [EPA2A] (DeepSeek-V3 splits the work into micro-batches so that the
    exchange of one hides behind the computation of another). Each micro-batch
    is routed, laid out and combined on its own; with no capacity limit the
    result equals the whole-batch layer.
    """
    T = cfg.T
    if n_chunks < 1 or T % n_chunks != 0:
        raise ValueError("T must split evenly into the micro-batches")
    tc = T // n_chunks
    ys = []
    for c in range(n_chunks):
        sub = {k: v for k, v in inputs.items()}
        sub["x"] = inputs["x"][c * tc:(c + 1) * tc]
        ys.append(layer_forward(sub, cfg.replace(T=tc))["y"])
    return {"y": np.concatenate(ys, axis=0)}


def layer_forward(inputs: Dict, cfg) -> Dict[str, np.ndarray]:
    """Router -> layout -> permute -> expert FFN -> combine on one device, all in float64.

    With shared-expert weights in ``inputs`` (shared_w1, shared_w3, shared_w2)
    the shared expert's output is added to the routed sum.
    """
    r = route(inputs["x"], inputs["w_gate"], inputs.get("bias"), cfg.top_k, cfg.gate,
              cfg.n_groups, cfg.topk_groups)
    C = capacity(cfg.capacity_factor, cfg.T, cfg.top_k, cfg.E)
    lay = dispatch_layout(r["topk_idx"], cfg.E, cfg.ep_size, C)
    xp = permute(as_f64(inputs["x"]), lay["row_to_pair"], cfg.top_k, lay["n_kept"])
    yp = expert_ffn(xp, lay["expert_offsets"], inputs["w1"], inputs.get("w3"), inputs["w2"], cfg.act)
    y = combine(yp, lay["pair_to_row"], r["topk_gate"], cfg.T, cfg.top_k)
    if inputs.get("shared_w1") is not None:
        y = y + shared_expert_ffn(inputs["x"], inputs["shared_w1"], inputs.get("shared_w3"), inputs["shared_w2"],
                                  cfg.act)
    out = dict(r)
    out.update(lay)
    out.update({"x_perm": xp, "y_perm": yp, "y": y})
    return out
