"""Host-side bounds check of the direct loads of the bf16 grouped GEMM and router.

The GEMM's buffer resources set no range clamp (num_records = 0xFFFFFFFF), so nothing on the GPU stops a
wrong 32-bit offset from reading outside its operand; this is the guard. tests/bounds/load_bounds.cpp
walks every block of a launch as launch_ffn_bf16 / launch_wgrad_bf16 / launch_route issue it, every
lane and every load (first and last K stage, and the stages where the K-major form switches matrix),
with the per-lane positions and offsets computed by the kernels' own geometry headers, and checks that
each 16-byte access lies inside its operand, that no 32-bit offset wraps, and that the block -> tile
map runs every tile exactly once. Shapes: the five workloads at full size, per-expert counts at and
around every row-tile edge, all rows on one expert, 600 experts (the tile map's multi-pass branch).
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "bounds", "load_bounds.cpp")
INC = os.path.join(ROOT, "combine_experts_amd", "csrc")
GBM = 320  # tile rows of the grouped GEMM (gemm_geometry.h)


@pytest.fixture(scope="module")
def lib(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("bounds") / "libbounds.so")
    subprocess.run(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", f"-I{INC}", SRC, "-o", out], check=True)
    L = ctypes.CDLL(out)
    P = ctypes.c_void_p
    L.moe_check_ffn_loads.restype = ctypes.c_int64
    L.moe_check_ffn_loads.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int, P, ctypes.c_int, ctypes.c_int64, ctypes.c_int, P]
    L.moe_check_wgrad_loads.restype = ctypes.c_int64
    L.moe_check_wgrad_loads.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64, P]
    L.moe_check_route_loads.restype = ctypes.c_int64
    L.moe_check_route_loads.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P]
    return L


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _ffn(lib, off, n_rows_max, K, nout, dual=False, bt=False, ksplit=0, gather=None, gdiv=1, a_rows=0, splits=1):
    off = np.ascontiguousarray(off, dtype=np.int32)
    g = None if gather is None else np.ascontiguousarray(gather, dtype=np.int32)
    st = np.zeros(8, dtype=np.int64)
    bad = lib.moe_check_ffn_loads(_ptr(off), len(off) - 1, n_rows_max, K, nout, int(dual), int(bt), ksplit, _ptr(g),
                                  gdiv, a_rows, splits, _ptr(st))
    assert st[1] > 0
    assert bad == 0, (f"{st[0]} accesses out of bounds (first: block {st[4]}, wave {st[5]}, lane {st[6]}, "
                      f"load {st[7]}), {st[3]} tiles not run exactly once")
    return st


def _layout_maps(counts, T, k, rng):
    """Offsets and a row_to_pair of the given per-expert counts: row r holds a distinct pair id < T*k."""
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    N = int(off[-1])
    r2p = np.full(T * k, -1, dtype=np.int64)
    r2p[:N] = rng.permutation(T * k)[:N]
    return off, r2p


def _check_layer(lib, cfg, counts, rng):
    T, D, E, k, F = cfg.T, cfg.D, cfg.E, cfg.top_k, cfg.F
    P_ = T * k
    off, r2p = _layout_maps(counts, T, k, rng)
    dual = cfg.act == W.ACT_SWIGLU
    nm = 2 if dual else 1
    # forward: up-projection from x_perm and with rows gathered from x; down-projection
    _ffn(lib, off, P_, D, F, dual=dual)
    _ffn(lib, off, P_, D, F, dual=dual, gather=r2p, gdiv=k, a_rows=T)
    _ffn(lib, off, P_, F, D)
    if F % 64 == 0 and F // 64 >= 32:
        for S in (2, 4, 8):   # the split-K down-projection
            _ffn(lib, off, P_, F, D, splits=S)
    # training forward (pre-activations stored: same loads) and the data-gradient GEMMs on the weights
    # as stored: dh = dy_perm W2 (W2[e] read K-major as [D][F]); dx_perm = [da1 da3] [W1; W3] (K-major,
    # the reduction split between W1 and W3 at F)
    _ffn(lib, off, P_, D, F, bt=True, ksplit=D)
    _ffn(lib, off, P_, nm * F, D, bt=True, ksplit=F)
    # weight gradients over 64-padded groups (the operand row stride is the padded total)
    koff = np.concatenate([[0], np.cumsum((np.asarray(counts) + 63) // 64 * 64)]).astype(np.int32)
    ld = max(int(koff[-1]), 64)
    for M_, N_ in ((D, F), (nm * F, D)):
        st = np.zeros(8, dtype=np.int64)
        assert lib.moe_check_wgrad_loads(_ptr(koff), E, M_, N_, ld, _ptr(st)) == 0, f"wgrad {M_}x{N_}: {st}"


def _near_even(N, E, rng):
    c = rng.multinomial(N, np.ones(E) / E)
    return c


FULL = ["tiny_fp32", "switch_cap", "mixtral", "dsv3", "skew"]


@pytest.mark.parametrize("name", FULL)
def test_full_workloads_near_even_and_skewed_counts(lib, name):
    cfg = W.get_config(name)
    rng = np.random.default_rng(5)
    P_ = cfg.T * cfg.top_k
    C = min(P_, int(np.ceil(cfg.capacity_factor * P_ / cfg.E))) if cfg.capacity_factor > 0 else P_
    even = np.minimum(_near_even(P_, cfg.E, rng), C)
    _check_layer(lib, cfg, even, rng)
    # the skewed profile: Zipf-like popularity, capped
    p = 1.0 / np.arange(1, cfg.E + 1) ** 1.2
    skew = np.minimum(rng.multinomial(P_, p / p.sum()), C)
    _check_layer(lib, cfg, skew, rng)


@pytest.mark.parametrize("where", ["first", "last"])
def test_all_rows_on_one_expert(lib, where):
    cfg = W.get_config("mixtral", T=4096, D=512, F=448)
    counts = np.zeros(cfg.E, dtype=np.int64)
    counts[0 if where == "first" else -1] = cfg.T * cfg.top_k
    _check_layer(lib, cfg, counts, np.random.default_rng(6))


def test_counts_at_row_tile_edges(lib):
    # every expert's count sits on or next to a 32-row block or a 320-row tile edge
    edges = [0, 1, 31, 32, 33, 63, 64, 65, 288, 289, 319, 320, 321, 352, 639, 640, 641, 959, 960, 961, 3201]
    cfg = W.MoEConfig(name="edges", T=sum(edges), D=256, E=len(edges), top_k=1, F=192, ep_size=1, seed=1)
    _check_layer(lib, cfg, np.array(edges), np.random.default_rng(7))
    cfg2 = cfg.replace(act=W.ACT_GELU, D=128, F=320)
    _check_layer(lib, cfg2, np.array(edges[::-1]), np.random.default_rng(8))


def test_six_hundred_experts(lib):
    # more experts than the 512 threads of a block: the tile map's multi-pass branch
    rng = np.random.default_rng(9)
    E, k = 600, 4
    counts = rng.integers(0, 700, size=E)
    counts[rng.choice(E, 100, replace=False)] = 0
    T = int(np.ceil(counts.sum() / k))
    cfg = W.MoEConfig(name="e600", T=T, D=128, E=E, top_k=k, F=128, ep_size=1, seed=2)
    pad = T * k - counts.sum()
    counts[np.argmax(counts)] += pad
    _check_layer(lib, cfg, counts, rng)


@pytest.mark.parametrize("T,D,E", [(256, 128, 8), (4096, 1024, 16), (8192, 4096, 8), (16384, 7168, 256),
                                   (32768, 4096, 64), (77, 64, 3), (65, 192, 33), (1, 64, 1), (130, 256, 100),
                                   (129, 64, 200)])
def test_router_loads(lib, T, D, E):
    st = np.zeros(8, dtype=np.int64)
    assert lib.moe_check_route_loads(T, D, E, _ptr(st)) == 0, f"router loads out of bounds: {st}"
    assert st[1] > 0


def test_checker_catches_a_bad_offset(lib):
    # the check itself: one more expert's worth of rows than the operand holds must be reported
    off = np.array([0, 320, 700], dtype=np.int32)
    st = np.zeros(8, dtype=np.int64)
    bad = lib.moe_check_ffn_loads(_ptr(off), 2, 600, 128, 256, 0, 0, 0, None, 1, 0, 1, _ptr(st))
    assert bad > 0 and st[0] > 0
    # and a gather index past the source rows
    off = np.array([0, 4], dtype=np.int32)
    g = np.array([0, 1, 2, 1000], dtype=np.int32)
    bad = lib.moe_check_ffn_loads(_ptr(off), 1, 4, 128, 256, 0, 0, 0, _ptr(g), 1, 8, 1, _ptr(st))
    assert bad > 0
