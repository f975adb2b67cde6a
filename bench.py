"""Throughput of the one-GPU MoE layer (route -> layout -> permute -> expert FFN -> combine).

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dsv3] [--no-cpu-baseline]

One step = one full layer forward over one batch of seeded synthetic input already resident in
HBM: all five stages, enqueued back to back on one stream with no host synchronisation. The permute
runs inside the up-projection's row loads (moe_expert_ffn_up_gather: the same h bit for bit as
moe_permute + moe_expert_ffn_up); the standalone permute kernel, which the training forward uses, is
timed on its own after the steps and reported as permute_gbps. Prints ONE JSON line on stdout;
diagnostics go to stderr.

value = T / (ms_per_step / 1e3) tokens/s on the one GPU. The roofline object is for the dominant
kernel (the grouped up-projection GEMM with the fused SwiGLU/GELU epilogue), timed with HIP
events around its launch on the stream it runs on, inside the timed region.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s (route+permute+FFN+combine); permute GB/s; GEMM MFMA %"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix-core peak
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 vector peak
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
STAGES = ["route", "layout", "ffn_up", "ffn_down", "combine"]   # ffn_up includes the permute
DOMINANT = "ffn_up"
# what the dominant kernel's machine code is built from: its source, its geometry header and the build
# flags; the committed PMC traffic summary is used only while these are unchanged
DOMINANT_SRC = (os.path.join(ROOT, "combine_experts_amd", "csrc", "ffn.hip"),
                os.path.join(ROOT, "combine_experts_amd", "csrc", "gemm_geometry.h"),
                os.path.join(ROOT, "combine_experts_amd", "build.py"))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(paths) -> str:
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 PMC summary, or None
    if there is none or the kernel's source, geometry header or build flags changed since the counters
    were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_ffn_up_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != source_sha(DOMINANT_SRC):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, inp, n_random_rows: int = 512, seed: int = 0):
    """The CPU oracle, untouched, timed on the host cores: route, dispatch layout, permute and combine on
    all T tokens; the expert FFN on a seeded sample of rows (the first and last row of every non-empty
    expert group, n_random_rows random rows, and at the skewed workload all rows of the hottest expert),
    extrapolated to all N kept rows. The oracle's FFN costs a fixed amount per expert (its weights are
    upcast to float64 once) plus a cost per row, so the estimate is the sample's time plus the rows not
    in the sample at the marginal cost of a row, measured on the busiest expert (its FFN over all its
    rows against over two of them). The combine reads an x_perm-shaped stand-in for the expert outputs
    (its cost does not depend on their values)."""
    import numpy as np
    import threadpoolctl
    import oracle as O

    T, k = cfg.T, cfg.top_k
    x = inp["x"].cpu()
    wg = inp["w_gate"].cpu()
    bias = None if inp["bias"] is None else inp["bias"].cpu()
    # every expert's weights in host memory (bf16 or f32 as stored) before timing
    host_w = {key: (None if inp[key] is None else inp[key].cpu()) for key in ("w1", "w3", "w2")}
    info = threadpoolctl.threadpool_info()
    threads = max((i.get("num_threads", 1) for i in info), default=1)
    t = {}
    t0 = time.perf_counter()
    r = O.route(x, wg, bias, k, cfg.gate, cfg.n_groups, cfg.topk_groups)
    t["route"] = time.perf_counter() - t0
    C = O.capacity(cfg.capacity_factor, T, k, cfg.E)
    t0 = time.perf_counter()
    lay = O.dispatch_layout(r["topk_idx"], cfg.E, cfg.ep_size, C)
    t["layout"] = time.perf_counter() - t0
    N = lay["n_kept"]
    t0 = time.perf_counter()
    xp = O.permute(O.as_f64(x), lay["row_to_pair"], k, N)
    t["permute"] = time.perf_counter() - t0
    # FFN sample
    off = lay["expert_offsets"]
    rng = np.random.default_rng(seed)
    rows = set()
    nonempty = [e for e in range(cfg.E) if off[e + 1] > off[e]]
    for e in nonempty:
        rows |= {int(off[e]), int(off[e + 1] - 1)}
    if N > 0:
        rows |= set(rng.choice(N, size=min(n_random_rows, N), replace=False).tolist())
    if cfg.name == "skew" and nonempty:
        hot = max(nonempty, key=lambda e: off[e + 1] - off[e])
        rows |= set(range(int(off[hot]), int(off[hot + 1])))
    rows = np.array(sorted(rows), dtype=np.int64)
    experts = np.searchsorted(off, rows, side="right") - 1
    t0 = time.perf_counter()
    O.expert_ffn_rows(xp[rows], experts, host_w["w1"], host_w["w3"], host_w["w2"], cfg.act)
    t_ffn_sample = time.perf_counter() - t0
    per_row, busiest = 0.0, -1
    if nonempty:
        busiest = max(nonempty, key=lambda e: off[e + 1] - off[e])
        lo, hi = int(off[busiest]), int(off[busiest + 1])
        one = np.full(hi - lo, busiest)
        t0 = time.perf_counter()
        O.expert_ffn_rows(xp[lo:lo + 2], one[:2], host_w["w1"], host_w["w3"], host_w["w2"], cfg.act)
        t_two = time.perf_counter() - t0
        t0 = time.perf_counter()
        O.expert_ffn_rows(xp[lo:hi], one, host_w["w1"], host_w["w3"], host_w["w2"], cfg.act)
        t_all = time.perf_counter() - t0
        per_row = max(t_all - t_two, 0.0) / max(hi - lo - 2, 1)
    t["ffn"] = t_ffn_sample + max(N - len(rows), 0) * per_row
    t0 = time.perf_counter()
    O.combine(xp, lay["pair_to_row"], r["topk_gate"], T, k)
    t["combine"] = time.perf_counter() - t0
    total = sum(t.values())
    return {"value": round(T / total, 3), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu_count": os.cpu_count(), "cpu_model": cpu_model(),
            "stage_s": {s_: round(v, 3) for s_, v in t.items()},
            "sample": f"route, layout, permute and combine on all {T} tokens ({N} kept rows); the expert FFN "
                      f"on {len(rows)} of {N} rows (first and last row of each of {len(nonempty)} non-empty "
                      f"experts, {min(n_random_rows, N)} random rows" + (", all rows of the hottest expert"
                                                                        if cfg.name == "skew" else "") +
                      f") in {t_ffn_sample:.1f} s, plus the other {max(N - len(rows), 0)} rows at "
                      f"{per_row * 1e3:.3f} ms each, the marginal row cost on expert {busiest} ('sampled'); "
                      f"float64; {threads} BLAS threads on {os.cpu_count()} logical CPUs"}


def measure_cluster(M, W, torch, cfg, d, inp, buf, stream, time_calls, b):
    """Expert parallelism emulated on one GPU at the workload's EP size: every source shard lays out
    its own tokens into one concatenated send buffer; the exchange of all ranks (with each rank's
    per-expert regroup) is one row gather over all N rows, the return one row scatter."""
    n_src = cfg.ep_size
    ts = cfg.T // n_src
    k, E, D = cfg.top_k, cfg.E, cfg.D
    stride = ts * k
    dev = "cuda"
    i32 = dict(dtype=torch.int32, device=dev)
    d_src = M.dims_from_config(cfg.replace(T=ts))
    src_off = torch.empty((n_src, E + 1), **i32)
    p2r = torch.empty((n_src, ts * k), **i32)
    r2p = torch.empty((n_src, ts * k), **i32)
    cnt, rc, ro = torch.empty(E, **i32), torch.empty(cfg.ep_size, **i32), torch.empty(cfg.ep_size + 1, **i32)
    ws = torch.empty(max(1, M.moe_workspace_size(d_src, M.MOE_STAGE_LAYOUT)), dtype=torch.uint8, device=dev)
    send = torch.empty((n_src * stride, D), dtype=W.torch_dtype(cfg.dtype), device=dev)
    for s in range(n_src):
        M.moe_dispatch_layout(d_src, buf.topk_idx[s * ts * k:(s + 1) * ts * k], cnt, src_off[s], rc, ro, p2r[s], r2p[s],
                              ws, stream)
        M.moe_permute(d_src, inp["x"][s * ts:(s + 1) * ts], p2r[s], send[s * stride:(s + 1) * stride], stream)
    matrix = torch.empty((n_src, cfg.ep_size), **i32)
    t_matrix = time_calls(lambda: M.moe_dispatch_matrix(d, buf.topk_idx, n_src, matrix, stream))
    epr = E // cfg.ep_size
    g2s = torch.empty(cfg.T * k, **i32)
    recv_counts, eoff = torch.empty(n_src, **i32), torch.empty(epr + 1, **i32)
    t_recv = time_calls(lambda: M.moe_recv_layout(d, n_src, 0, stride, src_off, recv_counts, eoff, g2s, stream))
    # all ranks' regrouped rows, rank after rank: one map over every sent row
    maps = []
    for r in range(cfg.ep_size):
        M.moe_recv_layout(d, n_src, r, stride, src_off, recv_counts, eoff, g2s, stream)
        torch.cuda.synchronize()
        maps.append(g2s[:int(eoff[-1])].clone())
    full_map = torch.cat(maps)
    n = full_map.numel()
    grouped = torch.empty((n, D), dtype=send.dtype, device=dev)
    back = torch.empty_like(send)
    t_gather = time_calls(lambda: M.moe_gather_rows(d, full_map, send, grouped, stream))
    t_scatter = time_calls(lambda: M.moe_scatter_rows(d, full_map, grouped, back, stream))
    moved = 2.0 * n * D * b + n * 4
    out = {"n_src": n_src, "rows": n, "dispatch_matrix_ms": t_matrix, "recv_layout_ms": t_recv,
           "exchange_gather_ms": t_gather, "return_scatter_ms": t_scatter,
           "exchange_gbps": round(moved / (t_gather * 1e-3) / 1e9, 1),
           "return_gbps": round(moved / (t_scatter * 1e-3) / 1e9, 1)}
    del send, grouped, back
    return out


def measure_padded(M, W, torch, cfg, inp, stream, time_calls, cf=1.25):
    """The fixed-capacity padded layout against the compact layout with the same capacity."""
    c = cfg.replace(capacity_factor=cfg.capacity_factor if cfg.capacity_factor > 0 else cf)
    d = M.dims_from_config(c)
    buf = M.MoELayerBuffers(d, device="cuda")
    C = M.moe_capacity(d)
    R = c.E * C
    dt = W.torch_dtype(c.dtype)
    i32 = dict(dtype=torch.int32, device="cuda")
    p2s, s2p, poff = torch.empty(c.T * c.top_k, **i32), torch.empty(R, **i32), torch.empty(c.E + 1, **i32)
    x_pad = torch.empty((R, c.D), dtype=dt, device="cuda")
    h_pad = torch.empty((R, c.F), dtype=dt, device="cuda")
    y_pad = torch.empty((R, c.D), dtype=dt, device="cuda")
    M.moe_route(d, inp["x"], inp["w_gate"], inp["bias"], buf.topk_idx, buf.topk_gate, None, stream)

    def layout():
        M.moe_dispatch_layout(d, buf.topk_idx, buf.expert_counts, buf.expert_offsets, buf.rank_counts,
                              buf.rank_offsets, buf.pair_to_row, buf.row_to_pair, buf.layout_ws, stream)

    def compact():
        layout()
        M.moe_permute(d, inp["x"], buf.pair_to_row, buf.x_perm, stream)
        M.moe_expert_ffn_up(d, buf.x_perm, buf.expert_offsets, inp["w1"], inp["w3"], buf.h, stream)
        M.moe_expert_ffn_down(d, buf.h, buf.expert_offsets, inp["w2"], buf.y_perm, stream)
        M.moe_unpermute_combine(d, buf.y_perm, buf.pair_to_row, buf.topk_gate, buf.y, stream)

    def padded():
        layout()
        M.moe_padded_layout(d, buf.topk_idx, buf.expert_offsets, buf.pair_to_row, buf.row_to_pair, p2s, s2p, poff,
                            stream)
        M.moe_permute_padded(d, inp["x"], s2p, x_pad, stream)
        M.moe_expert_ffn_padded_up(d, x_pad, poff, inp["w1"], inp["w3"], h_pad, stream)
        M.moe_expert_ffn_padded_down(d, h_pad, poff, inp["w2"], y_pad, stream)
        M.moe_unpermute_combine(d, y_pad, p2s, buf.topk_gate, buf.y, stream, n_rows=R)

    t_compact = time_calls(compact, reps=5)
    t_padded = time_calls(padded, reps=5)
    N = int(buf.expert_offsets[-1].item())
    out = {"capacity_factor": c.capacity_factor, "C": C, "slots": R, "kept": N,
           "padding_frac": round((R - N) / R, 4), "dropped": c.T * c.top_k - N,
           "compact_ms": round(t_compact, 4), "padded_ms": round(t_padded, 4)}
    del buf, x_pad, h_pad, y_pad
    return out


def measure_overlap(M, W, torch, cfg, inp, stream, time_calls, n_chunks=2):
    """The layer executor (permute inside the up-projection, as in the step): one stream vs n_chunks
    micro-batches on two streams, without and with a shared expert of the routed experts' hidden size."""
    d = M.dims_from_config(cfg)
    fs = cfg.F
    sh_cfg = cfg.replace(shared_F=fs)
    sh = W.make_inputs(sh_cfg, "cuda", with_experts=False)
    shared = (sh["shared_w1"], sh["shared_w3"], sh["shared_w2"])
    out = {"n_chunks": n_chunks, "shared_F": fs}
    for key, nc, two, use_sh in (("sequential_ms", 1, False, False), ("overlapped_ms", n_chunks, True, False),
                                 ("shared_sequential_ms", 1, False, True), ("shared_overlapped_ms", n_chunks, True, True),
                                 ("shared_concurrent_ms", 1, True, True)):
        ex = M.LayerExecutor(d, n_chunks=nc, two_streams=two, shared_F=fs if use_sh else 0, gather=True)
        out[key] = round(time_calls(lambda: ex.forward(inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"],
                                                       inp["w2"], shared=shared if use_sh else None, stream=stream),
                                    reps=5), 4)
        del ex
    del sh
    return out


def measure_backward(M, W, torch, cfg, inp, stream, reps=3):
    """One training step's backward at the workload shape, stage by stage (HIP events on the stream); the
    data-gradient GEMMs read the weights as stored (no transposed copies to rebuild after an update), and
    no x_perm is kept: the training up-projection and the transposed x operand of the W1/W3 gradient
    gather their rows from x."""
    d = M.dims_from_config(cfg)
    buf = M.MoELayerBuffers(d, device="cuda", logits=True, x_perm=False)
    bw = M.BackwardBuffers(d, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    dy = torch.randn((cfg.T, cfg.D), generator=g, device="cuda").to(torch.bfloat16)
    nm = 2 if cfg.act == W.ACT_SWIGLU else 1
    x, w1, w3, w2 = inp["x"], inp["w1"], inp["w3"], inp["w2"]
    stages = [
        ("backward_combine", lambda: M.moe_backward_combine(d, dy, buf.pair_to_row, buf.topk_gate, buf.y_perm,
                                                            bw.dy_perm, bw.dgate, stream)),
        ("dgrad_down_act", lambda: M.moe_expert_ffn_down_backward_w(d, bw.dy_perm, buf.expert_offsets, w2, bw.pre,
                                                                    bw.da, stream)),
        ("dgrad_up", lambda: M.moe_expert_ffn_up_backward_w(d, bw.da, buf.expert_offsets, w1, w3, bw.dx_perm, stream)),
        ("router_backward", lambda: M.moe_router_backward(d, x, buf.logits, buf.topk_idx, buf.topk_gate, bw.dgate,
                                                          bw.dl, bw.dw_gate, bw.dbias, bw.router_ws, stream,
                                                          all_expert_offsets=buf.expert_offsets,
                                                          all_row_to_pair=buf.row_to_pair)),
        ("backward_dx", lambda: M.moe_backward_dx(d, bw.dx_perm, buf.pair_to_row, buf.topk_idx, bw.dl, inp["w_gate"],
                                                  bw.dx, stream)),
        ("transpose_dy_h", lambda: (M.moe_group_transpose(d, bw.dy_perm, d.D, buf.expert_offsets, bw.koff, bw.dyp_t,
                                                          stream),
                                    M.moe_group_transpose(d, buf.h, d.F, buf.expert_offsets, bw.koff, bw.h_t, stream))),
        ("wgrad_w2", lambda: M.moe_expert_wgrad(d, bw.dyp_t, bw.h_t, bw.koff, d.D, d.F, bw.dw2, stream=stream)),
        ("transpose_da_x", lambda: (M.moe_group_transpose(d, bw.da, nm * d.F, buf.expert_offsets, bw.koff, bw.da_t,
                                                          stream),
                                    M.moe_group_transpose_gather(d, x, d.D, buf.expert_offsets, buf.row_to_pair,
                                                                 bw.koff, bw.xp_t, stream))),
        ("wgrad_w13", lambda: M.moe_expert_wgrad(d, bw.da_t, bw.xp_t, bw.koff, nm * d.F, d.D, bw.dw1, bw.dw3,
                                                 split=d.F, stream=stream)),
    ]
    fwd = lambda: M.forward_train(buf, bw, x, inp["w_gate"], inp["bias"], w1, w3, w2, stream)
    fwd()
    for _, f in stages:
        f()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 2)] for _ in range(reps)]
    for r in range(reps):
        ev[r][0].record(stream)
        fwd()
        ev[r][1].record(stream)
        for i, (_, f) in enumerate(stages):
            f()
            ev[r][i + 2].record(stream)
    torch.cuda.synchronize()
    st = {name: sum(ev[r][i + 1].elapsed_time(ev[r][i + 2]) for r in range(reps)) / reps
          for i, (name, _) in enumerate(stages)}
    fwd_ms = sum(ev[r][0].elapsed_time(ev[r][1]) for r in range(reps)) / reps
    N = int(buf.expert_offsets[-1].item())
    gemm_flops = 2.0 * N * cfg.D * cfg.F * (1 + nm + 1 + nm)
    gemm_ms = st["dgrad_down_act"] + st["dgrad_up"] + st["wgrad_w2"] + st["wgrad_w13"]
    total = sum(st.values())
    out = {"stage_ms": {k_: round(v, 4) for k_, v in st.items()}, "total_ms": round(total, 4),
           "forward_train_ms": round(fwd_ms, 4), "train_step_ms": round(fwd_ms + total, 4),
           "gemm_tflops": round(gemm_flops / (gemm_ms * 1e-3) / 1e12, 1),
           "train_tokens_per_s": round(cfg.T / ((fwd_ms + total) * 1e-3), 1)}
    del buf, bw, dy
    torch.cuda.empty_cache()
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the forward step (no load-balancing, cluster, padded, executor or backward "
                         "measurements), e.g. under a profiler")
    ap.add_argument("--cpu-random-rows", type=int, default=512,
                    help="random rows in the CPU oracle's expert-FFN sample (besides each expert's first and last)")
    ap.add_argument("--copy-calib-bytes", type=int, default=0,
                    help="before the timed steps, copy a buffer of this many bytes 3 times (a plain copy kernel "
                         "of known size, to scale HBM byte counters)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures the one-GPU share of the MoE layer only: run it with --gpus 1 "
              "(the library runs one GPU's share; multi-GPU expert parallelism is not implemented).", file=sys.stderr)
        return 2

    import torch
    import combine_experts_amd as M
    import workloads as W

    M.load_library()
    cfg = W.get_config(args.workload)
    dev = "cuda"
    log(f"[bench] {cfg.desc}")
    t0 = time.time()
    inp = W.make_inputs(cfg, dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs drawn on GPU in {time.time() - t0:.1f} s")
    d = M.dims_from_config(cfg)
    buf = M.MoELayerBuffers(d, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        M.moe_route(d, inp["x"], inp["w_gate"], inp["bias"], buf.topk_idx, buf.topk_gate, None, stream)
        if ev is not None:
            ev[1].record(stream)
        M.moe_dispatch_layout(d, buf.topk_idx, buf.expert_counts, buf.expert_offsets, buf.rank_counts,
                              buf.rank_offsets, buf.pair_to_row, buf.row_to_pair, buf.layout_ws, stream)
        if ev is not None:
            ev[2].record(stream)
        M.moe_expert_ffn_up_gather(d, inp["x"], buf.row_to_pair, buf.expert_offsets, inp["w1"], inp["w3"], buf.h,
                                   stream)
        if ev is not None:
            ev[3].record(stream)
        M.moe_expert_ffn_down_splitk(d, buf.h, buf.expert_offsets, inp["w2"], buf.y_perm, buf.down_ws, stream)
        if ev is not None:
            ev[4].record(stream)
        M.moe_unpermute_combine(d, buf.y_perm, buf.pair_to_row, buf.topk_gate, buf.y, stream)
        if ev is not None:
            ev[5].record(stream)

    if args.copy_calib_bytes > 0:
        src = torch.ones(args.copy_calib_bytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    stage_ms = {s: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps for j, s in enumerate(STAGES)}
    per_step = {s: sorted(e[j].elapsed_time(e[j + 1]) for e in evs) for j, s in enumerate(STAGES)}
    stage_med = {s: v[len(v) // 2] for s, v in per_step.items()}
    stage_min = {s: v[0] for s, v in per_step.items()}
    # the standalone permute kernel (outside the timed steps), for its bandwidth: each timed call starts
    # from a cold cache (a 768 MiB copy, three times the 256 MiB Infinity Cache, runs before it), so
    # neither x nor x_perm is served from a cache a previous repetition filled; the back-to-back figure
    # (same buffers, warm) is reported beside it
    M.moe_permute(d, inp["x"], buf.pair_to_row, buf.x_perm, stream)
    flush_src = torch.empty(384 << 20, dtype=torch.uint8, device=dev)
    flush_dst = torch.empty_like(flush_src)
    cold = []
    for _ in range(10):
        flush_dst.copy_(flush_src)
        ca, cz = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ca.record(stream)
        M.moe_permute(d, inp["x"], buf.pair_to_row, buf.x_perm, stream)
        cz.record(stream)
        cold.append((ca, cz))
    pa, pz = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pa.record(stream)
    for _ in range(20):
        M.moe_permute(d, inp["x"], buf.pair_to_row, buf.x_perm, stream)
    pz.record(stream)
    torch.cuda.synchronize()
    permute_ms = sum(a.elapsed_time(z) for a, z in cold) / len(cold)
    permute_warm_ms = pa.elapsed_time(pz) / 20
    del flush_src, flush_dst
    # the same step captured once in a HIP graph and replayed (one launch per step)
    gl = M.GraphLayer(d, inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"], device=dev)
    for _ in range(args.warmup):
        gl.replay()
    ga, gz = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ga.record(stream)
    for _ in range(args.steps):
        gl.replay()
    gz.record(stream)
    torch.cuda.synchronize()
    graph_ms = ga.elapsed_time(gz) / args.steps
    del gl

    N = int(buf.expert_offsets[-1].item())
    counts = buf.expert_counts.cpu()
    b = 2 if cfg.dtype == W.DT_BF16 else 4
    nm = 3 if cfg.act == W.ACT_SWIGLU else 2
    up_flops = 2.0 * N * cfg.D * cfg.F * (nm - 1)
    ffn_flops = 2.0 * N * cfg.D * cfg.F * nm
    peak = PEAK_BF16_TFLOPS if cfg.dtype == W.DT_BF16 else PEAK_F32_TFLOPS
    up_tflops = up_flops / (stage_ms[DOMINANT] * 1e-3) / 1e12
    ffn_tflops = ffn_flops / ((stage_ms["ffn_up"] + stage_ms["ffn_down"]) * 1e-3) / 1e12
    permute_bytes = cfg.T * cfg.D * b + N * cfg.D * b + cfg.T * cfg.top_k * 4
    combine_bytes = N * cfg.D * b + cfg.T * cfg.D * b + cfg.T * cfg.top_k * 8
    permute_gbs = permute_bytes / (permute_ms * 1e-3) / 1e9
    permute_warm_gbs = permute_bytes / (permute_warm_ms * 1e-3) / 1e9
    combine_gbs = combine_bytes / (stage_ms["combine"] * 1e-3) / 1e9
    traffic = read_traffic(cfg.name)
    # every stage against its own roofline: algorithmic bytes and flops at the realised N, spec peaks
    T_, D_, E_, k_, F_ = cfg.T, cfg.D, cfg.E, cfg.top_k, cfg.F
    algo = {
        "route": (T_ * D_ * b + E_ * D_ * b + T_ * k_ * 8, 2.0 * T_ * D_ * E_),
        "layout": (3 * T_ * k_ * 4 + (2 * E_ + 2 * cfg.ep_size + 2) * 4, 0.0),
        "ffn_up": (E_ * (nm - 1) * F_ * D_ * b + T_ * D_ * b + N * 4 + N * F_ * b, up_flops),
        "ffn_down": (E_ * D_ * F_ * b + N * F_ * b + N * D_ * b, 2.0 * N * D_ * F_),
        "combine": (combine_bytes, 2.0 * N * D_),
    }
    stage_roof = {}
    for s_, (by, fl) in algo.items():
        t_hbm = by / (PEAK_HBM_GBS * 1e9) * 1e3
        t_cmp = fl / (peak * 1e12) * 1e3
        bound = max(t_hbm, t_cmp)
        stage_roof[s_] = {"bound": "hbm" if t_hbm >= t_cmp else ("mfma" if cfg.dtype == W.DT_BF16 else "alu"),
                          "bound_ms": round(bound, 5), "frac": round(bound / stage_ms[s_], 4),
                          "algorithmic_bytes": by, "algorithmic_flops": fl}
    layer_bound = sum(v["bound_ms"] for v in stage_roof.values())
    roofline = {"bound": "mfma" if cfg.dtype == W.DT_BF16 else "alu", "achieved": round(up_tflops, 2), "peak": peak,
                "unit": "TFLOP/s",
                "frac": round(up_tflops / peak, 4), "traffic": traffic,
                "kernel": "ffn_gemm_bf16 (grouped up-projection, fused SwiGLU)" if cfg.dtype == W.DT_BF16
                else "ffn_gemm_f32 (grouped up-projection)",
                "algorithmic_flops_per_launch": up_flops}
    log(f"[bench] N={N} kept rows, max/mean expert count {float(counts.max()) / float(counts.float().mean()):.2f}")
    for s in STAGES:
        log(f"[bench]   {s:9s} {stage_ms[s] * 1e3:9.1f} us")
    log(f"[bench] step as a HIP graph replay: {graph_ms * 1e3:.1f} us")
    log(f"[bench] permute {permute_gbs:.0f} GB/s from a cold cache ({permute_warm_gbs:.0f} GB/s back to back), "
        f"combine {combine_gbs:.0f} GB/s, "
        f"FFN {ffn_tflops:.0f} TFLOP/s ({ffn_tflops / peak * 100:.1f}% of peak)")

    extra_ms, cluster, padded, overlap, bwd = {}, None, None, None, None
    if not args.no_extras:
        # Stages beyond the forward step, timed on their own after it (not part of `value`):
        # load balancing = the router with a selection-only bias and probability sums, then the
        # statistics / bias-step kernel.
        def time_calls(fn, reps=20):
            fn()
            a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                fn()
            z.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(z) / reps

        sb = W.make_select_bias(cfg, dev)
        part = torch.empty(M.moe_workspace_size(d, M.MOE_STAGE_ROUTE_STATS) // 4, dtype=torch.float32, device=dev)
        stats = torch.empty(2 * cfg.E + 2, dtype=torch.float32, device=dev)
        extra_ms = {
            "route_ex": time_calls(lambda: M.moe_route_ex(d, inp["x"], inp["w_gate"], inp["bias"], sb, buf.topk_idx,
                                                          buf.topk_gate, None, part, stream)),
            "load_balance": time_calls(lambda: M.moe_load_balance(d, buf.expert_counts, part, 0.01, stats, 0.0, None,
                                                                  stream)),
        }
        # the routing the step left in buf is restored before the cluster and padded measurements
        M.moe_route(d, inp["x"], inp["w_gate"], inp["bias"], buf.topk_idx, buf.topk_gate, None, stream)
        M.moe_dispatch_layout(d, buf.topk_idx, buf.expert_counts, buf.expert_offsets, buf.rank_counts,
                              buf.rank_offsets, buf.pair_to_row, buf.row_to_pair, buf.layout_ws, stream)
        cluster = measure_cluster(M, W, torch, cfg, d, inp, buf, stream, time_calls, b)
        padded = measure_padded(M, W, torch, cfg, inp, stream, time_calls)
        overlap = measure_overlap(M, W, torch, cfg, inp, stream, time_calls)
        bwd = measure_backward(M, W, torch, cfg, inp, stream) if cfg.dtype == W.DT_BF16 else None
        extra_ms.update({"dispatch_matrix": cluster["dispatch_matrix_ms"], "recv_layout": cluster["recv_layout_ms"],
                         "exchange_gather": cluster["exchange_gather_ms"], "return_scatter": cluster["return_scatter_ms"]})
        for s_, v in extra_ms.items():
            log(f"[bench]   {s_:15s} {v * 1e3:9.1f} us (outside the step)")
        log(f"[bench] emulated exchange over {cluster['n_src']} sources: {cluster['rows']} rows, gather "
            f"{cluster['exchange_gbps']:.0f} GB/s, scatter {cluster['return_gbps']:.0f} GB/s")
        log(f"[bench] padded layout at CF {padded['capacity_factor']}: C={padded['C']}, padding "
            f"{padded['padding_frac']:.1%}, dropped {padded['dropped']}; compact path {padded['compact_ms']:.3f} ms, "
            f"padded path {padded['padded_ms']:.3f} ms")
        log(f"[bench] executor: 1 stream {overlap['sequential_ms']:.3f} ms, {overlap['n_chunks']} micro-batches on 2 streams "
            f"{overlap['overlapped_ms']:.3f} ms; with a shared expert (F={overlap['shared_F']}) "
            f"{overlap['shared_sequential_ms']:.3f} / {overlap['shared_overlapped_ms']:.3f} ms, shared expert beside the "
            f"routed FFN on one batch {overlap['shared_concurrent_ms']:.3f} ms")
        if bwd is not None:
            log(f"[bench] backward {bwd['total_ms']:.3f} ms (weights read as stored); grouped GEMMs {bwd['gemm_tflops']:.0f} TFLOP/s; training step (forward with saved "
                f"pre-activations + backward) {bwd['train_step_ms']:.3f} ms")
            for s_, v in bwd["stage_ms"].items():
                log(f"[bench]     bwd {s_:20s} {v * 1e3:9.1f} us")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline ...")
        cpu = cpu_baseline(cfg, inp, args.cpu_random_rows)
        log(f"[bench] CPU oracle: {cpu['value']:.2f} tokens/s, stages {cpu['stage_s']} s ({cpu['sample']}; "
            f"{cpu['cpu_model']})")

    out = {
        "metric": METRIC, "value": round(cfg.T / (ms_per_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == W.DT_BF16 else "f32", "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "D": cfg.D, "E": cfg.E, "top_k": cfg.top_k, "F": cfg.F,
                   "act": "swiglu" if cfg.act == W.ACT_SWIGLU else "gelu", "capacity_factor": cfg.capacity_factor,
                   "ep_size_emulated": cfg.ep_size, "n_groups": cfg.n_groups, "topk_groups": cfg.topk_groups,
                   "kept_rows": N, "parallelism": "1 GPU"},
        "stage_ms": {s: round(v, 4) for s, v in stage_ms.items()},
        "stage_ms_median": {s: round(v, 4) for s, v in stage_med.items()},
        "stage_ms_min": {s: round(v, 4) for s, v in stage_min.items()},
        "stage_roofline": stage_roof,
        "layer_roofline": {"bound_ms": round(layer_bound, 4), "frac": round(layer_bound / ms_per_step, 4),
                           "note": "sum of the stages' spec-peak bounds over the measured step"},
        "permute": "inside ffn_up (rows gathered from x by the GEMM's loads)",
        "graph": {"ms_per_step": round(graph_ms, 4), "tokens_per_s": round(cfg.T / (graph_ms * 1e-3), 1),
                  "note": "the same step captured once in a HIP graph and replayed"},
        "extra_stage_ms": {"permute_standalone": round(permute_ms, 4), "permute_standalone_warm": round(permute_warm_ms, 4),
                           **{s: round(v, 4) for s, v in extra_ms.items()}},
        "cluster_emulation": cluster,
        "padded_capacity": padded,
        "overlap": overlap,
        "backward": bwd,
        "permute_gbps": round(permute_gbs, 1), "permute_gbps_warm": round(permute_warm_gbs, 1),
        "combine_gbps": round(combine_gbs, 1),
        "gemm_mfma_frac": round(ffn_tflops / peak, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
