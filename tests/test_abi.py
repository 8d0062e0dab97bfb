"""The C-ABI library loads and exports every entry point that include/moe.h declares;
host-side argument checks return their status codes without touching a GPU."""
import ctypes
import os
import re

import pytest

import mixture_experts_expert_softmax_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*([a-z_0-9]+)\s*\(", src, flags=re.M))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(M.library_path):
        pytest.skip("library not built")
    return M.lib()


def test_header_lists_the_bound_exports():
    assert _declared() == set(M.EXPORTS), _declared() ^ set(M.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(9):
        s = M.status_string(code)
        assert s.startswith("MOE_"), s
    assert "unknown" in M.status_string(99)
    assert b"gfx950" in lib.moe_version()


def test_host_side_errors_need_no_gpu(lib):
    # shape / null / dtype errors are decided on the host before any launch
    assert lib.moe_route(None, 4, 0, 1, None, None, None) == 2          # E < 1
    assert lib.moe_route(None, 4, 8, 9, None, None, None) == 2          # k > E
    assert lib.moe_route(None, 4, 8, 2, None, None, None) == 1          # null
    assert lib.moe_route(None, 0, 8, 2, None, None, None) == 0          # T == 0: no-op
    assert lib.grouped_gemm_fwd(None, None, None, 0, 4, 64, 100, 64, None, None, 0, None) == 2   # N % 32
    assert lib.grouped_gemm_fwd(None, None, None, 5, 4, 64, 64, 64, None, None, 0, None) == 3    # offs kind
    assert lib.grouped_gemm_fwd(None, None, None, 0, 4, 64, 64, 64, None, None, 0, None) == 1    # null
    p = ctypes.c_void_p(16)
    q = ctypes.c_void_p(24)  # misaligned
    assert lib.grouped_gemm_fwd(p, q, p, 0, 4, 64, 64, 64, p, None, 0, None) == 4
    assert lib.grouped_gemm_wgrad(p, p, p, 0, 4, 64, 64, 64, p, 7, None, 0, None) == 3  # out dtype
    assert lib.moe_finalize(None, None, None, 4, 2, 12, None, None) == 2  # H % 8
    assert lib.moe_sort(None, 4, 2, 8, 4, 6, None, None, None, None, None, None, 0, None) == 2  # L+off > E
    z = ctypes.c_void_p(256)
    assert lib.moe_sort(z, 4, 2, 8, 8, 0, z, None, z, z, z, None, 0, None) == 6  # workspace


def test_workspace_queries(lib):
    assert lib.moe_sort_workspace_size(4096, 2, 8) >= 8 * 4
    d = M.MoeFfnDesc(4096, 4096, 14336, 8, 8, 0, 2, 0, 0)
    ws = lib.moe_ffn_workspace_size(ctypes.byref(d))
    # act [T*k, I] + y [T*k, H] in bf16 dominate
    assert ws >= 8192 * (14336 + 4096) * 2
    d.finalize_mode = 1
    assert lib.moe_ffn_workspace_size(ctypes.byref(d)) < ws
    d.H = 100
    assert lib.moe_ffn_workspace_size(ctypes.byref(d)) == 0
    bad = M.MoeFfnDesc(16, 128, 256, 8, 8, 0, 2, 0, 5)
    assert lib.moe_ffn_forward(ctypes.byref(bad), None, None, 0, None) == 3


def test_noalloc_rejects_requests_beyond_its_scratch(lib):
    # decided from the shapes on the host, before the device or the scratch is touched
    d = M.MoeFfnDesc(4096, 4096, 14336, 8, 8, 0, 2, 0, 0)
    assert lib.moe_ffn_workspace_size(ctypes.byref(d)) > M.NOALLOC_SCRATCH_BYTES
    t = M.MoeFfnTensors()
    assert lib.moe_ffn_forward_noalloc(ctypes.byref(d), ctypes.byref(t), None) == 8
    assert "scratch" in M.status_string(8)
    bad = M.MoeFfnDesc(16, 100, 256, 8, 8, 0, 2, 0, 0)   # H % 64
    assert lib.moe_ffn_forward_noalloc(ctypes.byref(bad), ctypes.byref(t), None) == 2
