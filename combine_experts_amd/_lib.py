"""ctypes binding of libmoe.so: argument marshalling only.

Every function here has the name of the C entry point it calls (see include/moe.h), takes torch
tensors for the device buffers, checks their device, dtype, shape and contiguity, passes raw
pointers plus the current HIP stream, and raises ``MoEError`` on a non-zero status. All work of
the layer runs in the library's HIP kernels; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, 1, 2, 3, 4
MOE_GATE_SOFTMAX_TOPK, MOE_GATE_SIGMOID_TOPK, MOE_GATE_SOFTMAX_FULL = 0, 1, 2
MOE_ACT_SWIGLU, MOE_ACT_GELU = 0, 1
MOE_F32, MOE_BF16 = 0, 1
MOE_STAGE_LAYOUT, MOE_STAGE_FFN, MOE_STAGE_ROUTE_STATS, MOE_STAGE_ROUTER_BWD, MOE_STAGE_FFN_DOWN = 0, 1, 2, 3, 4


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


class moe_dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "D", "E", "top_k", "F", "ep_size", "ep_rank", "n_groups", "topk_groups",
                 "gate", "act", "dtype")] + [("capacity_factor", ctypes.c_double)]


_P = ctypes.c_void_p
_I32P = ctypes.POINTER(ctypes.c_int32)


class moe_layer_args(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("x", "w_gate", "bias", "w1", "w3", "w2", "y", "topk_idx", "topk_gate",
                                  "pair_to_row", "row_to_pair", "x_perm", "h", "y_perm", "expert_counts",
                                  "expert_offsets", "rank_counts", "rank_offsets", "layout_ws")] + \
        [("layout_ws_bytes", ctypes.c_size_t)] + \
        [(n, _P) for n in ("shared_w1", "shared_w3", "shared_w2")] + [("shared_F", ctypes.c_int32)] + \
        [(n, _P) for n in ("shared_h", "shared_y", "shared_offsets", "logits", "pre", "down_ws")] + \
        [("down_ws_bytes", ctypes.c_size_t)]


class moe_backward_args(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("x", "w_gate", "w1", "w3", "w2", "logits", "topk_idx", "topk_gate",
                                  "expert_offsets", "pair_to_row", "row_to_pair", "x_perm", "h", "pre", "y_perm",
                                  "dy", "w13t", "w2t")] + [("refresh_weights", ctypes.c_int32)] + \
        [(n, _P) for n in ("dy_perm", "dgate", "da", "dx_perm", "dl", "router_ws")] + \
        [("router_ws_bytes", ctypes.c_size_t), ("koff", _P)] + \
        [(n, _P) for n in ("dy_perm_t", "h_t", "da_t", "x_perm_t")] + [("ld", ctypes.c_int64)] + \
        [(n, _P) for n in ("dx", "dw_gate", "dbias", "dw1", "dw3", "dw2")]
_SIG = {
    "moe_abi_version": (ctypes.c_int, []),
    "moe_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_capacity": (ctypes.c_int, [ctypes.POINTER(moe_dims), _I32P]),
    "moe_workspace_size": (ctypes.c_int, [ctypes.POINTER(moe_dims), ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]),
    "moe_route": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, _P, _P, _P, _P, _P, _P]),
    "moe_route_ex": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_load_balance": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, _P, ctypes.c_float, _P, ctypes.c_float, _P, _P]),
    "moe_dispatch_matrix": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, ctypes.c_int32, _P, _P]),
    "moe_recv_layout": (ctypes.c_int, [ctypes.POINTER(moe_dims), ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, _P, _P,
                                       _P, _P, ctypes.c_int32, _P]),
    "moe_gather_rows": (ctypes.c_int, [ctypes.POINTER(moe_dims), ctypes.c_int64, _P, _P, _P, _P]),
    "moe_scatter_rows": (ctypes.c_int, [ctypes.POINTER(moe_dims), ctypes.c_int64, _P, _P, _P, _P]),
    "moe_padded_layout": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_permute_padded": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, _P, _P, _P]),
    "moe_expert_ffn_padded_up": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, _P, _P, _P, _P, _P]),
    "moe_expert_ffn_padded_down": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, _P, _P, _P, _P]),
    "moe_unpermute_combine_add": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, _P, _P, _P, _P, _P]),
    "moe_layer_forward": (ctypes.c_int, [ctypes.POINTER(moe_dims), ctypes.POINTER(moe_layer_args), ctypes.c_int32, _P,
                                         _P, _P]),
    "moe_event_create": (ctypes.c_int, [ctypes.POINTER(_P)]),
    "moe_expert_ffn_up_train": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, _P, _P, _P, _P, _P, _P]),
    "moe_expert_ffn_up_train_gather": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_transpose_weights": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, _P, _P, _P, _P, _P]),
    "moe_backward_combine": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, _P, _P, _P, _P, _P, _P]),
    "moe_expert_ffn_down_backward": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, _P, _P, _P, _P, _P]),
    "moe_expert_ffn_up_backward": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, _P, _P, _P, _P]),
    "moe_expert_ffn_down_backward_w": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, _P, _P, _P, _P, _P]),
    "moe_expert_ffn_up_backward_w": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, _P, _P, _P, _P, _P]),
    "moe_router_backward": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                           ctypes.c_size_t, _P]),
    "moe_backward_dx": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, _P, _P, _P, _P, _P, _P]),
    "moe_wgrad_ld": (ctypes.c_int, [ctypes.POINTER(moe_dims), ctypes.POINTER(ctypes.c_int64)]),
    "moe_group_transpose": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, ctypes.c_int32, _P, _P, _P, ctypes.c_int64,
                                           _P]),
    "moe_group_transpose_gather": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, ctypes.c_int32, _P, _P, _P, _P,
                                                  ctypes.c_int64, _P]),
    "moe_expert_wgrad": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, _P, _P, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int64, _P, _P, ctypes.c_int32, _P]),
    "moe_event_destroy": (ctypes.c_int, [_P]),
    "moe_layer_backward": (ctypes.c_int, [ctypes.POINTER(moe_dims), ctypes.POINTER(moe_backward_args), _P]),
    "moe_dispatch_layout": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, _P, _P, _P, _P, _P, _P, _P,
                                           ctypes.c_size_t, _P]),
    "moe_dispatch_layout_noalloc": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_permute": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, _P, _P, _P]),
    "moe_expert_ffn": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_expert_ffn_up": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, _P, _P, _P, _P, _P]),
    "moe_expert_ffn_up_gather": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, _P, _P, _P, _P, _P, _P]),
    "moe_expert_ffn_down": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, _P, _P, _P, _P]),
    "moe_expert_ffn_down_splitk": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_unpermute_combine": (ctypes.c_int, [ctypes.POINTER(moe_dims), _P, _P, _P, _P, _P]),
}

_lib: Optional[ctypes.CDLL] = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmoe.so (built in-tree by ``combine_experts_amd.build``). Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libmoe.so not found at {path}: build it with `python -m combine_experts_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIG.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != MOE_OK:
        msg = load_library().moe_status_str(status).decode()
        raise MoEError(fn, status, msg)


def make_dims(T, D, E, top_k, F, *, ep_size=1, ep_rank=0, n_groups=0, topk_groups=0,
              gate=MOE_GATE_SOFTMAX_TOPK, act=MOE_ACT_SWIGLU, dtype=MOE_BF16, capacity_factor=0.0) -> moe_dims:
    return moe_dims(T, D, E, top_k, F, ep_size, ep_rank, n_groups, topk_groups, gate, act, dtype,
                    float(capacity_factor))


def dims_from_config(cfg) -> moe_dims:
    """moe_dims of a workloads.MoEConfig (or anything with the same attribute names)."""
    return make_dims(cfg.T, cfg.D, cfg.E, cfg.top_k, cfg.F, ep_size=cfg.ep_size, ep_rank=cfg.ep_rank,
                     n_groups=cfg.n_groups, topk_groups=cfg.topk_groups, gate=cfg.gate, act=cfg.act,
                     dtype=cfg.dtype, capacity_factor=cfg.capacity_factor)


def _elem_dtype(d: moe_dims) -> torch.dtype:
    return torch.bfloat16 if d.dtype == MOE_BF16 else torch.float32


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None, numel=None, nullable=False) -> Optional[int]:
    if t is None:
        if nullable:
            return None
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} needs at least {numel} elements, has {t.numel()}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# ----------------------------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ----------------------------------------------------------------------------------------------

def moe_abi_version() -> int:
    return load_library().moe_abi_version()


def moe_status_str(status: int) -> str:
    return load_library().moe_status_str(status).decode()


def moe_capacity(d: moe_dims) -> int:
    c = ctypes.c_int32(0)
    _check("moe_capacity", load_library().moe_capacity(ctypes.byref(d), ctypes.byref(c)))
    return c.value


def moe_workspace_size(d: moe_dims, stage: int) -> int:
    b = ctypes.c_size_t(0)
    _check("moe_workspace_size", load_library().moe_workspace_size(ctypes.byref(d), stage, ctypes.byref(b)))
    return b.value


def moe_route(d: moe_dims, x, w_gate, bias, topk_idx, topk_gate, logits=None, stream=None) -> None:
    dt = _elem_dtype(d)
    st = load_library().moe_route(
        ctypes.byref(d), _ptr(x, "x", dt, d.T * d.D), _ptr(w_gate, "w_gate", dt, d.E * d.D),
        _ptr(bias, "bias", torch.float32, d.E, nullable=True),
        _ptr(topk_idx, "topk_idx", torch.int32, d.T * d.top_k), _ptr(topk_gate, "topk_gate", torch.float32, d.T * d.top_k),
        _ptr(logits, "logits", torch.float32, d.T * d.E, nullable=True), _stream(stream))
    _check("moe_route", st)


def moe_route_ex(d: moe_dims, x, w_gate, bias, select_bias, topk_idx, topk_gate, logits=None, prob_partials=None,
                 stream=None) -> None:
    dt = _elem_dtype(d)
    n_part = (d.T + 63) // 64
    st = load_library().moe_route_ex(
        ctypes.byref(d), _ptr(x, "x", dt, d.T * d.D), _ptr(w_gate, "w_gate", dt, d.E * d.D),
        _ptr(bias, "bias", torch.float32, d.E, nullable=True),
        _ptr(select_bias, "select_bias", torch.float32, d.E, nullable=True),
        _ptr(topk_idx, "topk_idx", torch.int32, d.T * d.top_k), _ptr(topk_gate, "topk_gate", torch.float32, d.T * d.top_k),
        _ptr(logits, "logits", torch.float32, d.T * d.E, nullable=True),
        _ptr(prob_partials, "prob_partials", torch.float32, n_part * d.E, nullable=True), _stream(stream))
    _check("moe_route_ex", st)


def moe_load_balance(d: moe_dims, expert_counts, prob_partials, alpha: float, stats, gamma: float = 0.0,
                     select_bias=None, stream=None) -> None:
    n_part = (d.T + 63) // 64
    st = load_library().moe_load_balance(
        ctypes.byref(d), _ptr(expert_counts, "expert_counts", torch.int32, d.E),
        _ptr(prob_partials, "prob_partials", torch.float32, n_part * d.E, nullable=d.T == 0), float(alpha),
        _ptr(stats, "stats", torch.float32, 2 * d.E + 2), float(gamma),
        _ptr(select_bias, "select_bias", torch.float32, d.E, nullable=True), _stream(stream))
    _check("moe_load_balance", st)


def moe_dispatch_layout(d: moe_dims, topk_idx, expert_counts, expert_offsets, rank_counts, rank_offsets,
                        pair_to_row, row_to_pair, ws, stream=None) -> None:
    P = d.T * d.top_k
    i32 = torch.int32
    st = load_library().moe_dispatch_layout(
        ctypes.byref(d), _ptr(topk_idx, "topk_idx", i32, P), _ptr(expert_counts, "expert_counts", i32, d.E),
        _ptr(expert_offsets, "expert_offsets", i32, d.E + 1), _ptr(rank_counts, "rank_counts", i32, d.ep_size),
        _ptr(rank_offsets, "rank_offsets", i32, d.ep_size + 1), _ptr(pair_to_row, "pair_to_row", i32, P),
        _ptr(row_to_pair, "row_to_pair", i32, P), _ptr(ws, "ws", nullable=True),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check("moe_dispatch_layout", st)


MOE_LAYOUT_NOALLOC_SCRATCH_BYTES = 1 << 20


def moe_dispatch_layout_noalloc(d: moe_dims, topk_idx, expert_counts, expert_offsets, rank_counts, rank_offsets,
                                pair_to_row, row_to_pair, stream=None) -> None:
    """moe_dispatch_layout with its scratch in the library's static per-GPU array (no workspace)."""
    P = d.T * d.top_k
    i32 = torch.int32
    st = load_library().moe_dispatch_layout_noalloc(
        ctypes.byref(d), _ptr(topk_idx, "topk_idx", i32, P), _ptr(expert_counts, "expert_counts", i32, d.E),
        _ptr(expert_offsets, "expert_offsets", i32, d.E + 1), _ptr(rank_counts, "rank_counts", i32, d.ep_size),
        _ptr(rank_offsets, "rank_offsets", i32, d.ep_size + 1), _ptr(pair_to_row, "pair_to_row", i32, P),
        _ptr(row_to_pair, "row_to_pair", i32, P), _stream(stream))
    _check("moe_dispatch_layout_noalloc", st)


def moe_permute(d: moe_dims, x, pair_to_row, x_perm, stream=None) -> None:
    dt = _elem_dtype(d)
    P = d.T * d.top_k
    st = load_library().moe_permute(
        ctypes.byref(d), _ptr(x, "x", dt, d.T * d.D), _ptr(pair_to_row, "pair_to_row", torch.int32, P),
        _ptr(x_perm, "x_perm", dt, P * d.D), _stream(stream))
    _check("moe_permute", st)


def moe_expert_ffn_up(d: moe_dims, x_perm, expert_offsets, w1, w3, h, stream=None) -> None:
    dt = _elem_dtype(d)
    P = d.T * d.top_k
    st = load_library().moe_expert_ffn_up(
        ctypes.byref(d), _ptr(x_perm, "x_perm", dt, P * d.D), _ptr(expert_offsets, "expert_offsets", torch.int32, d.E + 1),
        _ptr(w1, "w1", dt, d.E * d.F * d.D), _ptr(w3, "w3", dt, d.E * d.F * d.D, nullable=d.act == MOE_ACT_GELU),
        _ptr(h, "h", dt, P * d.F), _stream(stream))
    _check("moe_expert_ffn_up", st)


def moe_expert_ffn_up_gather(d: moe_dims, x, row_to_pair, expert_offsets, w1, w3, h, stream=None) -> None:
    dt = _elem_dtype(d)
    P = d.T * d.top_k
    st = load_library().moe_expert_ffn_up_gather(
        ctypes.byref(d), _ptr(x, "x", dt, d.T * d.D, nullable=d.T == 0),
        _ptr(row_to_pair, "row_to_pair", torch.int32, P, nullable=d.T == 0),
        _ptr(expert_offsets, "expert_offsets", torch.int32, d.E + 1),
        _ptr(w1, "w1", dt, d.E * d.F * d.D), _ptr(w3, "w3", dt, d.E * d.F * d.D, nullable=d.act == MOE_ACT_GELU),
        _ptr(h, "h", dt, P * d.F, nullable=d.T == 0), _stream(stream))
    _check("moe_expert_ffn_up_gather", st)


def moe_expert_ffn_down(d: moe_dims, h, expert_offsets, w2, y_perm, stream=None) -> None:
    dt = _elem_dtype(d)
    P = d.T * d.top_k
    st = load_library().moe_expert_ffn_down(
        ctypes.byref(d), _ptr(h, "h", dt, P * d.F), _ptr(expert_offsets, "expert_offsets", torch.int32, d.E + 1),
        _ptr(w2, "w2", dt, d.E * d.D * d.F), _ptr(y_perm, "y_perm", dt, P * d.D), _stream(stream))
    _check("moe_expert_ffn_down", st)


def moe_expert_ffn_down_splitk(d: moe_dims, h, expert_offsets, w2, y_perm, ws, stream=None) -> None:
    """moe_expert_ffn_down with the optional split-K workspace (moe_workspace_size(MOE_STAGE_FFN_DOWN)
    bytes; None: the plain down-projection)."""
    dt = _elem_dtype(d)
    P = d.T * d.top_k
    st = load_library().moe_expert_ffn_down_splitk(
        ctypes.byref(d), _ptr(h, "h", dt, P * d.F), _ptr(expert_offsets, "expert_offsets", torch.int32, d.E + 1),
        _ptr(w2, "w2", dt, d.E * d.D * d.F), _ptr(y_perm, "y_perm", dt, P * d.D), _ptr(ws, "ws", nullable=True),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check("moe_expert_ffn_down_splitk", st)


def moe_expert_ffn(d: moe_dims, x_perm, expert_offsets, w1, w3, w2, y_perm, ws, stream=None) -> None:
    dt = _elem_dtype(d)
    P = d.T * d.top_k
    st = load_library().moe_expert_ffn(
        ctypes.byref(d), _ptr(x_perm, "x_perm", dt, P * d.D), _ptr(expert_offsets, "expert_offsets", torch.int32, d.E + 1),
        _ptr(w1, "w1", dt, d.E * d.F * d.D), _ptr(w3, "w3", dt, d.E * d.F * d.D, nullable=d.act == MOE_ACT_GELU),
        _ptr(w2, "w2", dt, d.E * d.D * d.F), _ptr(y_perm, "y_perm", dt, P * d.D), _ptr(ws, "ws", nullable=True),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check("moe_expert_ffn", st)


def moe_unpermute_combine(d: moe_dims, y_perm, pair_to_row, topk_gate, y, stream=None, n_rows=None) -> None:
    """n_rows: rows y_perm holds (default T*top_k; E*C for the padded buffer)."""
    dt = _elem_dtype(d)
    P = d.T * d.top_k
    rows = P if n_rows is None else int(n_rows)
    st = load_library().moe_unpermute_combine(
        ctypes.byref(d), _ptr(y_perm, "y_perm", dt, rows * d.D), _ptr(pair_to_row, "pair_to_row", torch.int32, P),
        _ptr(topk_gate, "topk_gate", torch.float32, P), _ptr(y, "y", dt, d.T * d.D), _stream(stream))
    _check("moe_unpermute_combine", st)


# ---- cluster view and padded layout ----------------------------------------------------------------

def moe_dispatch_matrix(d: moe_dims, topk_idx, n_src: int, matrix, stream=None) -> None:
    st = load_library().moe_dispatch_matrix(
        ctypes.byref(d), _ptr(topk_idx, "topk_idx", torch.int32, d.T * d.top_k, nullable=d.T == 0), int(n_src),
        _ptr(matrix, "matrix", torch.int32, n_src * d.ep_size), _stream(stream))
    _check("moe_dispatch_matrix", st)


def moe_recv_layout(d: moe_dims, n_src: int, rank: int, src_stride: int, src_expert_offsets, recv_counts,
                    expert_offsets, grouped_to_src_row, stream=None) -> None:
    epr = d.E // d.ep_size
    n_rows_max = 0 if grouped_to_src_row is None else grouped_to_src_row.numel()
    i32 = torch.int32
    st = load_library().moe_recv_layout(
        ctypes.byref(d), int(n_src), int(rank), int(src_stride),
        _ptr(src_expert_offsets, "src_expert_offsets", i32, n_src * (d.E + 1)),
        _ptr(recv_counts, "recv_counts", i32, n_src), _ptr(expert_offsets, "expert_offsets", i32, epr + 1),
        _ptr(grouped_to_src_row, "grouped_to_src_row", i32, nullable=True), n_rows_max, _stream(stream))
    _check("moe_recv_layout", st)


def _rows(t, name, d):
    if t.numel() % d.D != 0:
        raise ValueError(f"{name} must hold whole rows of {d.D} elements")
    return t.numel() // d.D


def moe_gather_rows(d: moe_dims, row_map, src, dst, stream=None) -> None:
    """dst[i] = src[row_map[i]] for row_map[i] >= 0, i < row_map.numel(); rows of D elements."""
    dt = _elem_dtype(d)
    n = row_map.numel()
    _ptr(src, "src", dt)
    if _rows(dst, "dst", d) < n:
        raise ValueError("dst has fewer rows than row_map")
    st = load_library().moe_gather_rows(ctypes.byref(d), n, _ptr(row_map, "row_map", torch.int32), src.data_ptr(),
                                        _ptr(dst, "dst", dt), _stream(stream))
    _check("moe_gather_rows", st)


def moe_scatter_rows(d: moe_dims, row_map, src, dst, stream=None) -> None:
    """dst[row_map[i]] = src[i] for row_map[i] >= 0, i < row_map.numel()."""
    dt = _elem_dtype(d)
    n = row_map.numel()
    _ptr(dst, "dst", dt)
    if _rows(src, "src", d) < n:
        raise ValueError("src has fewer rows than row_map")
    st = load_library().moe_scatter_rows(ctypes.byref(d), n, _ptr(row_map, "row_map", torch.int32),
                                         _ptr(src, "src", dt), dst.data_ptr(), _stream(stream))
    _check("moe_scatter_rows", st)


def moe_padded_layout(d: moe_dims, topk_idx, expert_offsets, pair_to_row, row_to_pair, pair_to_slot, slot_to_pair,
                      padded_offsets, stream=None) -> None:
    P = d.T * d.top_k
    C = moe_capacity(d)
    i32 = torch.int32
    st = load_library().moe_padded_layout(
        ctypes.byref(d), _ptr(topk_idx, "topk_idx", i32, P, nullable=P == 0),
        _ptr(expert_offsets, "expert_offsets", i32, d.E + 1, nullable=P == 0),
        _ptr(pair_to_row, "pair_to_row", i32, P, nullable=P == 0), _ptr(row_to_pair, "row_to_pair", i32, P, nullable=P == 0),
        _ptr(pair_to_slot, "pair_to_slot", i32, P, nullable=P == 0), _ptr(slot_to_pair, "slot_to_pair", i32, d.E * C),
        _ptr(padded_offsets, "padded_offsets", i32, d.E + 1), _stream(stream))
    _check("moe_padded_layout", st)


def moe_permute_padded(d: moe_dims, x, slot_to_pair, x_pad, stream=None) -> None:
    dt = _elem_dtype(d)
    C = moe_capacity(d)
    st = load_library().moe_permute_padded(
        ctypes.byref(d), _ptr(x, "x", dt, d.T * d.D, nullable=d.T == 0),
        _ptr(slot_to_pair, "slot_to_pair", torch.int32, d.E * C), _ptr(x_pad, "x_pad", dt, d.E * C * d.D),
        _stream(stream))
    _check("moe_permute_padded", st)


def moe_expert_ffn_padded_up(d: moe_dims, x_pad, padded_offsets, w1, w3, h_pad, stream=None) -> None:
    dt = _elem_dtype(d)
    R = d.E * moe_capacity(d)
    st = load_library().moe_expert_ffn_padded_up(
        ctypes.byref(d), _ptr(x_pad, "x_pad", dt, R * d.D), _ptr(padded_offsets, "padded_offsets", torch.int32, d.E + 1),
        _ptr(w1, "w1", dt, d.E * d.F * d.D), _ptr(w3, "w3", dt, d.E * d.F * d.D, nullable=d.act == MOE_ACT_GELU),
        _ptr(h_pad, "h_pad", dt, R * d.F), _stream(stream))
    _check("moe_expert_ffn_padded_up", st)


def moe_expert_ffn_padded_down(d: moe_dims, h_pad, padded_offsets, w2, y_pad, stream=None) -> None:
    dt = _elem_dtype(d)
    R = d.E * moe_capacity(d)
    st = load_library().moe_expert_ffn_padded_down(
        ctypes.byref(d), _ptr(h_pad, "h_pad", dt, R * d.F), _ptr(padded_offsets, "padded_offsets", torch.int32, d.E + 1),
        _ptr(w2, "w2", dt, d.E * d.D * d.F), _ptr(y_pad, "y_pad", dt, R * d.D), _stream(stream))
    _check("moe_expert_ffn_padded_down", st)



def moe_unpermute_combine_add(d: moe_dims, y_perm, pair_to_row, topk_gate, addend, y, stream=None) -> None:
    dt = _elem_dtype(d)
    P = d.T * d.top_k
    st = load_library().moe_unpermute_combine_add(
        ctypes.byref(d), _ptr(y_perm, "y_perm", dt, P * d.D), _ptr(pair_to_row, "pair_to_row", torch.int32, P),
        _ptr(topk_gate, "topk_gate", torch.float32, P), _ptr(addend, "addend", dt, d.T * d.D, nullable=True),
        _ptr(y, "y", dt, d.T * d.D), _stream(stream))
    _check("moe_unpermute_combine_add", st)


def moe_event_create() -> int:
    e = _P()
    _check("moe_event_create", load_library().moe_event_create(ctypes.byref(e)))
    return e.value


def moe_event_destroy(event: int) -> None:
    _check("moe_event_destroy", load_library().moe_event_destroy(event))


def moe_layer_forward(d: moe_dims, args: moe_layer_args, n_chunks: int, stream=None, side_stream=None,
                      events=None) -> None:
    """Marshalling only: ``args`` is filled by ``layer.LayerExecutor`` from its torch buffers."""
    ev = None
    if side_stream is not None:
        if events is None or len(events) < 2 * n_chunks:
            raise ValueError("two events per micro-batch are needed with a side stream")
        ev = (_P * len(events))(*events)
    st = load_library().moe_layer_forward(ctypes.byref(d), ctypes.byref(args), int(n_chunks), _stream(stream),
                                          None if side_stream is None else _stream(side_stream), ev)
    _check("moe_layer_forward", st)



# ---- backward ----------------------------------------------------------------------------------------

def _nm(d):
    return 2 if d.act == MOE_ACT_SWIGLU else 1


def moe_expert_ffn_up_train(d: moe_dims, x_perm, expert_offsets, w1, w3, h, pre, stream=None) -> None:
    dt = _elem_dtype(d)
    P = d.T * d.top_k
    st = load_library().moe_expert_ffn_up_train(
        ctypes.byref(d), _ptr(x_perm, "x_perm", dt, P * d.D), _ptr(expert_offsets, "expert_offsets", torch.int32, d.E + 1),
        _ptr(w1, "w1", dt, d.E * d.F * d.D), _ptr(w3, "w3", dt, d.E * d.F * d.D, nullable=d.act == MOE_ACT_GELU),
        _ptr(h, "h", dt, P * d.F), _ptr(pre, "pre", dt, P * d.F * _nm(d)), _stream(stream))
    _check("moe_expert_ffn_up_train", st)


def moe_expert_ffn_up_train_gather(d: moe_dims, x, row_to_pair, expert_offsets, w1, w3, h, pre, stream=None) -> None:
    dt = _elem_dtype(d)
    P = d.T * d.top_k
    st = load_library().moe_expert_ffn_up_train_gather(
        ctypes.byref(d), _ptr(x, "x", dt, d.T * d.D), _ptr(row_to_pair, "row_to_pair", torch.int32, P),
        _ptr(expert_offsets, "expert_offsets", torch.int32, d.E + 1),
        _ptr(w1, "w1", dt, d.E * d.F * d.D), _ptr(w3, "w3", dt, d.E * d.F * d.D, nullable=d.act == MOE_ACT_GELU),
        _ptr(h, "h", dt, P * d.F), _ptr(pre, "pre", dt, P * d.F * _nm(d)), _stream(stream))
    _check("moe_expert_ffn_up_train_gather", st)


def moe_transpose_weights(d: moe_dims, w1, w3, w2, w13t, w2t, stream=None) -> None:
    dt = _elem_dtype(d)
    n = d.E * d.F * d.D
    st = load_library().moe_transpose_weights(
        ctypes.byref(d), _ptr(w1, "w1", dt, n), _ptr(w3, "w3", dt, n, nullable=d.act == MOE_ACT_GELU),
        _ptr(w2, "w2", dt, n), _ptr(w13t, "w13t", dt, n * _nm(d)), _ptr(w2t, "w2t", dt, n), _stream(stream))
    _check("moe_transpose_weights", st)


def moe_backward_combine(d: moe_dims, dy, pair_to_row, topk_gate, y_perm, dy_perm, dgate, stream=None) -> None:
    dt = _elem_dtype(d)
    P = d.T * d.top_k
    st = load_library().moe_backward_combine(
        ctypes.byref(d), _ptr(dy, "dy", dt, d.T * d.D), _ptr(pair_to_row, "pair_to_row", torch.int32, P),
        _ptr(topk_gate, "topk_gate", torch.float32, P), _ptr(y_perm, "y_perm", dt, P * d.D),
        _ptr(dy_perm, "dy_perm", dt, P * d.D), _ptr(dgate, "dgate", torch.float32, P), _stream(stream))
    _check("moe_backward_combine", st)


def moe_expert_ffn_down_backward(d: moe_dims, dy_perm, expert_offsets, w2t, pre, da, stream=None) -> None:
    dt = _elem_dtype(d)
    P = d.T * d.top_k
    st = load_library().moe_expert_ffn_down_backward(
        ctypes.byref(d), _ptr(dy_perm, "dy_perm", dt, P * d.D),
        _ptr(expert_offsets, "expert_offsets", torch.int32, d.E + 1), _ptr(w2t, "w2t", dt, d.E * d.F * d.D),
        _ptr(pre, "pre", dt, P * d.F * _nm(d)), _ptr(da, "da", dt, P * d.F * _nm(d)), _stream(stream))
    _check("moe_expert_ffn_down_backward", st)


def moe_expert_ffn_up_backward(d: moe_dims, da, expert_offsets, w13t, dx_perm, stream=None) -> None:
    dt = _elem_dtype(d)
    P = d.T * d.top_k
    st = load_library().moe_expert_ffn_up_backward(
        ctypes.byref(d), _ptr(da, "da", dt, P * d.F * _nm(d)),
        _ptr(expert_offsets, "expert_offsets", torch.int32, d.E + 1), _ptr(w13t, "w13t", dt, d.E * d.F * d.D * _nm(d)),
        _ptr(dx_perm, "dx_perm", dt, P * d.D), _stream(stream))
    _check("moe_expert_ffn_up_backward", st)


def moe_expert_ffn_down_backward_w(d: moe_dims, dy_perm, expert_offsets, w2, pre, da, stream=None) -> None:
    dt = _elem_dtype(d)
    P = d.T * d.top_k
    st = load_library().moe_expert_ffn_down_backward_w(
        ctypes.byref(d), _ptr(dy_perm, "dy_perm", dt, P * d.D),
        _ptr(expert_offsets, "expert_offsets", torch.int32, d.E + 1), _ptr(w2, "w2", dt, d.E * d.D * d.F),
        _ptr(pre, "pre", dt, P * d.F * _nm(d)), _ptr(da, "da", dt, P * d.F * _nm(d)), _stream(stream))
    _check("moe_expert_ffn_down_backward_w", st)


def moe_expert_ffn_up_backward_w(d: moe_dims, da, expert_offsets, w1, w3, dx_perm, stream=None) -> None:
    dt = _elem_dtype(d)
    P = d.T * d.top_k
    st = load_library().moe_expert_ffn_up_backward_w(
        ctypes.byref(d), _ptr(da, "da", dt, P * d.F * _nm(d)),
        _ptr(expert_offsets, "expert_offsets", torch.int32, d.E + 1), _ptr(w1, "w1", dt, d.E * d.F * d.D),
        _ptr(w3, "w3", dt, d.E * d.F * d.D, nullable=d.act == MOE_ACT_GELU), _ptr(dx_perm, "dx_perm", dt, P * d.D),
        _stream(stream))
    _check("moe_expert_ffn_up_backward_w", st)


def moe_router_backward(d: moe_dims, x, logits, topk_idx, topk_gate, dgate, dl, dw_gate, dbias=None, ws=None,
                        stream=None, all_expert_offsets=None, all_row_to_pair=None) -> None:
    dt = _elem_dtype(d)
    P = d.T * d.top_k
    f32, i32 = torch.float32, torch.int32
    st = load_library().moe_router_backward(
        ctypes.byref(d), _ptr(x, "x", dt, d.T * d.D, nullable=d.T == 0),
        _ptr(logits, "logits", f32, d.T * d.E, nullable=d.T == 0), _ptr(topk_idx, "topk_idx", i32, P, nullable=d.T == 0),
        _ptr(topk_gate, "topk_gate", f32, P, nullable=d.T == 0), _ptr(dgate, "dgate", f32, P, nullable=d.T == 0),
        _ptr(all_expert_offsets, "all_expert_offsets", i32, d.E + 1, nullable=True),
        _ptr(all_row_to_pair, "all_row_to_pair", i32, P, nullable=True),
        _ptr(dl, "dl", f32, d.T * d.E, nullable=d.T == 0), _ptr(dw_gate, "dw_gate", f32, d.E * d.D),
        _ptr(dbias, "dbias", f32, d.E, nullable=True), _ptr(ws, "ws", nullable=True),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check("moe_router_backward", st)


def moe_backward_dx(d: moe_dims, dx_perm, pair_to_row, topk_idx, dl, w_gate, dx, stream=None) -> None:
    dt = _elem_dtype(d)
    P = d.T * d.top_k
    st = load_library().moe_backward_dx(
        ctypes.byref(d), _ptr(dx_perm, "dx_perm", dt, P * d.D), _ptr(pair_to_row, "pair_to_row", torch.int32, P),
        _ptr(topk_idx, "topk_idx", torch.int32, P), _ptr(dl, "dl", torch.float32, d.T * d.E),
        _ptr(w_gate, "w_gate", dt, d.E * d.D), _ptr(dx, "dx", dt, d.T * d.D), _stream(stream))
    _check("moe_backward_dx", st)


def moe_wgrad_ld(d: moe_dims) -> int:
    v = ctypes.c_int64(0)
    _check("moe_wgrad_ld", load_library().moe_wgrad_ld(ctypes.byref(d), ctypes.byref(v)))
    return v.value


def moe_group_transpose(d: moe_dims, src, n_cols: int, expert_offsets, koff, dst, stream=None) -> None:
    dt = _elem_dtype(d)
    ld = dst.numel() // max(1, n_cols)
    st = load_library().moe_group_transpose(
        ctypes.byref(d), _ptr(src, "src", dt, nullable=d.T == 0), int(n_cols),
        _ptr(expert_offsets, "expert_offsets", torch.int32, d.E + 1),
        _ptr(koff, "koff", torch.int32, d.E + 1), _ptr(dst, "dst", dt, n_cols * moe_wgrad_ld(d)), ld, _stream(stream))
    _check("moe_group_transpose", st)


def moe_group_transpose_gather(d: moe_dims, x, n_cols: int, expert_offsets, row_to_pair, koff, dst,
                               stream=None) -> None:
    dt = _elem_dtype(d)
    ld = dst.numel() // max(1, n_cols)
    st = load_library().moe_group_transpose_gather(
        ctypes.byref(d), _ptr(x, "x", dt, nullable=d.T == 0), int(n_cols),
        _ptr(expert_offsets, "expert_offsets", torch.int32, d.E + 1),
        _ptr(row_to_pair, "row_to_pair", torch.int32, nullable=d.T == 0),
        _ptr(koff, "koff", torch.int32, d.E + 1), _ptr(dst, "dst", dt, n_cols * moe_wgrad_ld(d)), ld, _stream(stream))
    _check("moe_group_transpose_gather", st)


def moe_expert_wgrad(d: moe_dims, a_t, b_t, koff, M: int, N: int, out0, out1=None, split=None, stream=None) -> None:
    split = M if split is None else int(split)
    ld = a_t.numel() // max(1, M)
    if b_t.numel() // max(1, N) != ld:
        raise ValueError("a_t and b_t must have the same row length")
    f32 = torch.float32
    st = load_library().moe_expert_wgrad(
        ctypes.byref(d), _ptr(a_t, "a_t", _elem_dtype(d), M * ld), _ptr(b_t, "b_t", _elem_dtype(d), N * ld),
        _ptr(koff, "koff", torch.int32, d.E + 1), int(M), int(N), ld, _ptr(out0, "out0", f32, d.E * split * N),
        _ptr(out1, "out1", f32, d.E * (M - split) * N, nullable=split == M), split, _stream(stream))
    _check("moe_expert_wgrad", st)


def moe_layer_backward(d: moe_dims, args: moe_backward_args, stream=None) -> None:
    """Marshalling only: ``args`` is filled by ``layer.backward`` from its torch buffers."""
    _check("moe_layer_backward", load_library().moe_layer_backward(ctypes.byref(d), ctypes.byref(args), _stream(stream)))
