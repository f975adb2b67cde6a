"""Host-side checks of libmoe's C ABI: it loads, exports every declared entry point, and its host
logic (capacity, workspace sizes, argument validation) behaves. No kernel is launched here."""
import ctypes
import os
import re

import pytest

import combine_experts_amd as M
from combine_experts_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(moe_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = M.load_library()
    names = _declared_functions()
    assert len(names) >= 11, names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in moe.h but not exported"
    assert set(names) == set(L._SIG), "binding and header disagree"


def test_abi_version_and_status_strings():
    assert M.moe_abi_version() == 108
    for s in range(5):
        assert M.moe_status_str(s).startswith("MOE_")
    assert "unknown" in M.moe_status_str(99)


def test_struct_layout_matches_header():
    # 12 int32 fields then one double: 48 + 8 bytes, double at offset 48
    assert ctypes.sizeof(M.moe_dims) == 56
    assert M.moe_dims.capacity_factor.offset == 48


def test_capacity_matches_closed_form():
    d = M.make_dims(4096, 1024, 16, 1, 4096, capacity_factor=1.25, act=M.MOE_ACT_GELU)
    assert M.moe_capacity(d) == 320
    d = M.make_dims(4096, 1024, 8, 2, 4096, capacity_factor=1.0)
    assert M.moe_capacity(d) == 1024
    d = M.make_dims(1000, 64, 7, 2, 64, capacity_factor=1.5)
    assert M.moe_capacity(d) == 429
    d = M.make_dims(100, 64, 4, 2, 64)          # dropless
    assert M.moe_capacity(d) == 200
    d = M.make_dims(100, 64, 4, 2, 64, capacity_factor=1000.0)  # capped at T*k
    assert M.moe_capacity(d) == 200


def test_split_k_workspace_only_for_tile_starved_down_projections():
    # the Switch-style layer (C = 320 rows per expert, 16 experts, D = 1024: 64 down-projection tiles,
    # F = 4096 = 64 stages) splits its reduction 4 ways: 4 planes of T*k x D float32 partials
    d = M.make_dims(4096, 1024, 16, 1, 4096, capacity_factor=1.25, act=M.MOE_ACT_GELU, dtype=M.MOE_BF16)
    assert M.moe_workspace_size(d, M.MOE_STAGE_FFN_DOWN) == 4 * 4096 * 1024 * 4
    assert M.moe_workspace_size(d, M.MOE_STAGE_FFN) == 4096 * 4096 * 2 + 4 * 4096 * 1024 * 4
    # enough tiles (Mixtral- and DeepSeek-V3-shaped layers), a short F, or float32: no split
    for dd in (M.make_dims(8192, 4096, 8, 2, 14336, dtype=M.MOE_BF16), M.make_dims(16384, 7168, 256, 8, 2048,
               dtype=M.MOE_BF16), M.make_dims(4096, 1024, 16, 1, 1024, capacity_factor=1.25, dtype=M.MOE_BF16),
               M.make_dims(4096, 1024, 16, 1, 4096, capacity_factor=1.25, dtype=M.MOE_F32)):
        assert M.moe_workspace_size(dd, M.MOE_STAGE_FFN_DOWN) == 0


def test_workspace_sizes():
    d = M.make_dims(16384, 7168, 256, 8, 2048)
    assert M.moe_workspace_size(d, M.MOE_STAGE_FFN) >= 16384 * 8 * 2048 * 2
    assert M.moe_workspace_size(d, M.MOE_STAGE_LAYOUT) >= 256 * 4
    # one row of E float32 router-probability sums per 64-token router block
    assert M.moe_workspace_size(d, M.MOE_STAGE_ROUTE_STATS) == 256 * 256 * 4
    assert M.moe_workspace_size(M.make_dims(65, 64, 8, 2, 64), M.MOE_STAGE_ROUTE_STATS) == 2 * 8 * 4
    with pytest.raises(M.MoEError) as ei:
        M.moe_workspace_size(d, 7)
    assert ei.value.status == M.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [
    dict(top_k=0), dict(top_k=9), dict(E=8, ep_size=3), dict(ep_rank=4, ep_size=4),
    dict(n_groups=3), dict(n_groups=4, topk_groups=0), dict(n_groups=4, topk_groups=5),
    dict(n_groups=4, topk_groups=1, top_k=3), dict(gate=7), dict(act=5), dict(dtype=9), dict(D=0),
    dict(T=-1), dict(capacity_factor=float("nan")),
])
def test_invalid_dims_rejected_on_host(kw):
    base = dict(T=16, D=64, E=8, top_k=2, F=64, ep_size=4)
    base.update(kw)
    d = M.make_dims(base.pop("T"), base.pop("D"), base.pop("E"), base.pop("top_k"), base.pop("F"), **base)
    lib = M.load_library()
    c = ctypes.c_int32()
    assert lib.moe_capacity(ctypes.byref(d), ctypes.byref(c)) == M.MOE_ERR_INVALID_ARG
    # entry points reject before touching the device, even with null pointers
    assert lib.moe_route(ctypes.byref(d), None, None, None, None, None, None, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_permute(ctypes.byref(d), None, None, None, None) == M.MOE_ERR_INVALID_ARG


def test_null_and_misaligned_pointers_rejected():
    lib = M.load_library()
    d = M.make_dims(16, 64, 8, 2, 64)
    assert lib.moe_route(ctypes.byref(d), None, None, None, None, None, None, None) == M.MOE_ERR_INVALID_ARG
    fake = 0x1000
    assert lib.moe_permute(ctypes.byref(d), fake + 2, fake, fake, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_unpermute_combine(ctypes.byref(d), fake, fake, fake, fake + 8, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_ffn_up(ctypes.byref(d), fake, fake, fake, None, fake, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_ffn_up_gather(ctypes.byref(d), fake, None, fake, fake, fake, fake, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_ffn_up_gather(ctypes.byref(d), fake + 4, fake, fake, fake, fake, fake, None) == M.MOE_ERR_INVALID_ARG


def test_unsupported_shapes_reported():
    lib = M.load_library()
    fake = 0x1000
    d = M.make_dims(16, 64, 512, 2, 64)                    # E beyond the router's 256
    assert lib.moe_route(ctypes.byref(d), fake, fake, None, fake, fake, None, None) == M.MOE_ERR_UNSUPPORTED
    d = M.make_dims(16, 96, 8, 2, 64)                      # bf16 FFN needs D % 64 == 0
    assert lib.moe_expert_ffn_up(ctypes.byref(d), fake, fake, fake, fake, fake, None) == M.MOE_ERR_UNSUPPORTED
    # the bf16 GEMMs address operands with 32-bit offsets: x of 4 GiB cannot be gathered from (the
    # same x through x_perm is fine), nor can a weight-gradient tile span 4 GiB; both refused on the host
    d = M.make_dims(1 << 19, 4096, 8, 2, 64)              # T*D*2 = 4 GiB
    assert lib.moe_expert_ffn_up_gather(ctypes.byref(d), fake, fake, fake, fake, fake, fake, None) == \
        M.MOE_ERR_UNSUPPORTED
    assert lib.moe_expert_ffn_up_train_gather(ctypes.byref(d), fake, fake, fake, fake, fake, fake, fake, None) == \
        M.MOE_ERR_UNSUPPORTED
    d = M.make_dims(16, 64, 8, 2, 64)
    ld = (1 << 32) // 640 // 64 * 64 + 64                  # 320 rows of ld bf16 columns reach 4 GiB
    assert lib.moe_expert_wgrad(ctypes.byref(d), fake, fake, fake, 64, 64, ld, fake, None, 64, None) == \
        M.MOE_ERR_UNSUPPORTED


def test_noalloc_layout_limit_checked_on_host():
    # the allocation-free layout refuses, before any GPU call, a problem whose chunk histograms
    # (ceil(T*k/512) * E int32) exceed its static 1 MiB array
    lib = M.load_library()
    fake = 0x1000
    assert M.MOE_LAYOUT_NOALLOC_SCRATCH_BYTES == 1 << 20
    d = M.make_dims(16384 + 64, 64, 1024, 8, 64, ep_size=8)     # 257 chunks x 1024 experts x 4 B > 1 MiB
    assert lib.moe_dispatch_layout_noalloc(ctypes.byref(d), fake, fake, fake, fake, fake, fake, fake, None) == \
        M.MOE_ERR_WORKSPACE
    d = M.make_dims(16, 64, 8, 2, 64)
    assert lib.moe_dispatch_layout_noalloc(ctypes.byref(d), None, fake, fake, fake, fake, fake, fake, None) == \
        M.MOE_ERR_INVALID_ARG


def test_workspace_checks():
    lib = M.load_library()
    fake = 0x1000
    d = M.make_dims(1000, 64, 8, 2, 64)
    need = M.moe_workspace_size(d, M.MOE_STAGE_LAYOUT)
    args = [fake] * 7
    assert lib.moe_dispatch_layout(ctypes.byref(d), *args, None, need, None) == M.MOE_ERR_WORKSPACE
    assert lib.moe_dispatch_layout(ctypes.byref(d), *args, fake, need - 1, None) == M.MOE_ERR_WORKSPACE
    ffn_need = M.moe_workspace_size(d, M.MOE_STAGE_FFN)
    assert lib.moe_expert_ffn(ctypes.byref(d), fake, fake, fake, fake, fake, fake, fake, ffn_need - 1,
                              None) == M.MOE_ERR_WORKSPACE


def test_binding_refuses_host_tensors():
    import torch
    d = M.make_dims(4, 64, 8, 2, 64)
    with pytest.raises(ValueError):
        M.moe_permute(d, torch.zeros(4, 64, dtype=torch.bfloat16), torch.zeros(8, dtype=torch.int32),
                      torch.zeros(8, 64, dtype=torch.bfloat16))


def test_product_path_does_not_import_oracle():
    # the library package and the oracle share no code: nothing under combine_experts_amd names it
    pkg = os.path.join(ROOT, "combine_experts_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f


def test_load_balance_host_checks():
    lib = M.load_library()
    d = M.make_dims(16, 64, 8, 2, 64)
    fake = ctypes.c_void_p(256)
    # counts and stats are required; partials are required when T > 0
    assert lib.moe_load_balance(ctypes.byref(d), None, fake, 0.01, fake, 0.0, None, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_load_balance(ctypes.byref(d), fake, None, 0.01, fake, 0.0, None, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_load_balance(ctypes.byref(d), fake, fake, 0.01, None, 0.0, None, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_load_balance(ctypes.byref(d), fake, fake, float("inf"), fake, 0.0, None, None) == \
        M.MOE_ERR_INVALID_ARG
    assert lib.moe_load_balance(ctypes.byref(d), ctypes.c_void_p(258), fake, 0.01, fake, 0.0, None, None) == \
        M.MOE_ERR_INVALID_ARG


def test_route_ex_host_checks():
    lib = M.load_library()
    d = M.make_dims(16, 64, 8, 2, 64)
    fake = ctypes.c_void_p(256)
    mis = ctypes.c_void_p(258)
    assert lib.moe_route_ex(ctypes.byref(d), None, fake, None, None, fake, fake, None, None, None) == \
        M.MOE_ERR_INVALID_ARG
    assert lib.moe_route_ex(ctypes.byref(d), fake, fake, None, mis, fake, fake, None, None, None) == \
        M.MOE_ERR_INVALID_ARG
    assert lib.moe_route_ex(ctypes.byref(d), fake, fake, None, None, fake, fake, None, mis, None) == \
        M.MOE_ERR_INVALID_ARG
    d = M.make_dims(16, 64, 300, 2, 64)
    assert lib.moe_route_ex(ctypes.byref(d), fake, fake, None, fake, fake, fake, None, fake, None) == \
        M.MOE_ERR_UNSUPPORTED


def test_cluster_and_padded_host_checks():
    lib = M.load_library()
    fake = ctypes.c_void_p(256)
    d = M.make_dims(16, 64, 8, 2, 64, ep_size=4)
    # T must split evenly over the sources
    assert lib.moe_dispatch_matrix(ctypes.byref(d), fake, 3, fake, None) == M.MOE_ERR_INVALID_ARG
    # rank out of range; a source stride that overflows int32 rows
    assert lib.moe_recv_layout(ctypes.byref(d), 4, 4, 32, fake, fake, fake, fake, 8, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_recv_layout(ctypes.byref(d), 4, 0, 2**30, fake, fake, fake, fake, 8, None) == M.MOE_ERR_INVALID_ARG
    # too many (source, local expert) pairs for the receive tables
    big = M.make_dims(16, 64, 8192, 2, 64, ep_size=1)
    assert lib.moe_recv_layout(ctypes.byref(big), 4, 0, 32, fake, fake, fake, fake, 8, None) == M.MOE_ERR_UNSUPPORTED
    # the padded layout and its FFN need a capacity
    assert lib.moe_padded_layout(ctypes.byref(d), fake, fake, fake, fake, fake, fake, fake, None) == \
        M.MOE_ERR_INVALID_ARG
    assert lib.moe_permute_padded(ctypes.byref(d), fake, fake, fake, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_ffn_padded_up(ctypes.byref(d), fake, fake, fake, fake, fake, None) == M.MOE_ERR_INVALID_ARG
    # row moves: misaligned buffers are rejected, zero rows are a no-op
    assert lib.moe_gather_rows(ctypes.byref(d), 4, fake, ctypes.c_void_p(264), fake, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_scatter_rows(ctypes.byref(d), 0, None, None, None, None) == M.MOE_OK


def test_layer_args_struct_layout():
    # 19 pointers, a size_t, 3 pointers, an int32 (padded to 8), 6 pointers, a size_t
    assert ctypes.sizeof(M.moe_layer_args) == 19 * 8 + 8 + 3 * 8 + 8 + 6 * 8 + 8
    assert M.moe_layer_args.layout_ws_bytes.offset == 19 * 8
    assert M.moe_layer_args.shared_F.offset == 19 * 8 + 8 + 3 * 8
    assert M.moe_layer_args.down_ws.offset == 19 * 8 + 8 + 3 * 8 + 8 + 5 * 8


def test_layer_forward_host_checks():
    lib = M.load_library()
    d = M.make_dims(16, 64, 8, 2, 64)
    a = M.moe_layer_args()
    # T must split evenly; a side stream needs events; a layout workspace is required
    assert lib.moe_layer_forward(ctypes.byref(d), ctypes.byref(a), 3, None, None, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_layer_forward(ctypes.byref(d), ctypes.byref(a), 2, None, ctypes.c_void_p(8), None) == \
        M.MOE_ERR_INVALID_ARG
    assert lib.moe_layer_forward(ctypes.byref(d), ctypes.byref(a), 2, None, None, None) == M.MOE_ERR_WORKSPACE
    # a shared expert without its scratch buffers
    a.layout_ws, a.layout_ws_bytes = 256, 1 << 20
    a.shared_w1, a.shared_F = 256, 64
    assert lib.moe_layer_forward(ctypes.byref(d), ctypes.byref(a), 2, None, None, None) == M.MOE_ERR_INVALID_ARG


def test_backward_host_checks():
    lib = M.load_library()
    fake = ctypes.c_void_p(256)
    d32 = M.make_dims(16, 64, 8, 2, 64, dtype=M.MOE_F32)
    # the training GEMMs are bf16 only
    assert lib.moe_expert_ffn_up_train(ctypes.byref(d32), fake, fake, fake, fake, fake, fake, None) == \
        M.MOE_ERR_UNSUPPORTED
    assert lib.moe_expert_ffn_down_backward(ctypes.byref(d32), fake, fake, fake, fake, fake, None) == \
        M.MOE_ERR_UNSUPPORTED
    d = M.make_dims(16, 64, 8, 2, 64)
    # the padded column count of the transposed wgrad operands
    assert M.moe_wgrad_ld(d) == (16 * 2 + 63 * 8 + 63) // 64 * 64
    # a too-short transposed buffer, and a split past M
    assert lib.moe_group_transpose(ctypes.byref(d), fake, 64, fake, fake, fake, 64, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_wgrad(ctypes.byref(d), fake, fake, fake, 64, 64, 576, fake, fake, 65, None) == \
        M.MOE_ERR_INVALID_ARG
    # dbias without its workspace
    assert lib.moe_router_backward(ctypes.byref(d), fake, fake, fake, fake, fake, None, None, fake, fake, fake, None, 0,
                                   None) == M.MOE_ERR_WORKSPACE
    # the grouped form needs both arrays of the dropless layout
    assert lib.moe_router_backward(ctypes.byref(d), fake, fake, fake, fake, fake, fake, None, fake, fake, None, None, 0,
                                   None) == M.MOE_ERR_INVALID_ARG
    assert M.moe_workspace_size(d, M.MOE_STAGE_ROUTER_BWD) == 1 * 8 * 4


def test_backward_args_struct_layout():
    # 18 pointers, int32 (padded), 6 pointers, size_t, pointer, 4 pointers, int64, 6 pointers
    assert M.moe_backward_args.refresh_weights.offset == 18 * 8
    assert M.moe_backward_args.router_ws_bytes.offset == 18 * 8 + 8 + 6 * 8
    assert M.moe_backward_args.ld.offset == 18 * 8 + 8 + 6 * 8 + 8 + 8 + 4 * 8
    assert ctypes.sizeof(M.moe_backward_args) == 18 * 8 + 8 + 6 * 8 + 8 + 8 + 4 * 8 + 8 + 6 * 8
