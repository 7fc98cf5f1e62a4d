"""CPU-side checks of the C-ABI library: it loads, exports every entry point
declared in include/q8gemv.h, and rejects bad arguments on the host before
any device work (no GPU is touched by these tests)."""
import ctypes
import os
import re

import pytest

import block_quantized_gemv_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q8gemv.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(q8_0_\w+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 11
    L = q.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(q.EXPORTS) == set(names)


def test_version_and_strerror():
    assert q.q8_0_version() == 10000
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert q.strerror(code) and q.strerror(code) != "unknown status"
    assert q.strerror(-99) == "unknown status"


def test_packed_size():
    assert q.q8_0_packed_size(896, 896) == (14 * 64 * 896, 14 * 7 * 64 * 8)
    assert q.q8_0_packed_size(65, 96) == (2 * 64 * 96, 2 * 1 * 64 * 8)
    assert q.q8_0_packed_size(0, 32) == (0, 0)
    for M, K in [(-1, 32), (4, 0), (4, 33), (4, 48), (4, (1 << 20) + 32)]:
        with pytest.raises(q.Q8Error) as e:
            q.q8_0_packed_size(M, K)
        assert e.value.code == q.Q8_EINVAL


def _desc(M, K, n=1):
    return q.q8_0_weights(None, None, M, K, n, 0, 0)


def test_gemv_rejects_bad_shapes_on_host():
    L = q.lib()
    dummy = ctypes.c_void_p(16)
    for (M, K, N, wM, wK) in [(64, 33, 1, 64, 33), (64, 32, 0, 64, 32), (64, 32, 9, 64, 32),
                              (64, 32, 1, 65, 32), (64, 64, 1, 64, 32), (-1, 32, 1, -1, 32)]:
        W = _desc(wM, wK)
        rc = L.q8_0_gemv(ctypes.byref(W), dummy, dummy, M, K, N, None, 0, None)
        assert rc == q.Q8_EINVAL, (M, K, N, rc)
    W = _desc(64, 32)
    assert L.q8_0_gemv(ctypes.byref(W), None, dummy, 64, 32, 1, None, 0, None) == q.Q8_ENULL
    assert L.q8_0_gemv(None, dummy, dummy, 64, 32, 1, None, 0, None) == q.Q8_ENULL
    W2 = _desc(64, 32, n=2)  # a stack is not a dense matrix
    assert L.q8_0_gemv(ctypes.byref(W2), dummy, dummy, 64, 32, 1, None, 0, None) == q.Q8_EINVAL


def test_fused_rejects_bad_flags_on_host():
    L = q.lib()
    dummy = ctypes.c_void_p(16)
    W = _desc(128, 64)
    bad = [q.make_fusion(epilogue=q.Q8_EPI_SWIGLU | q.Q8_EPI_RESIDUAL),
           q.make_fusion(epilogue=q.Q8_EPI_SWIGLU | q.Q8_EPI_ARGMAX),
           q.make_fusion(epilogue=64),
           q.make_fusion(prologue=7),
           q.make_fusion(prologue=q.Q8_PRO_GQA, n_heads=3, n_kv_heads=2, head_dim=32),
           q.make_fusion(prologue=q.Q8_PRO_GQA, n_heads=2, n_kv_heads=1, head_dim=16),
           q.make_fusion(prologue=q.Q8_PRO_RMSNORM, eps=-1.0)]
    for f in bad:
        assert L.q8_0_gemv_fused(ctypes.byref(W), dummy, dummy, 128, 64, ctypes.byref(f), None,
                                 0, None) == q.Q8_EINVAL
    W3 = _desc(96, 64)  # SWIGLU needs (M/2) % 64 == 0
    f = q.make_fusion(epilogue=q.Q8_EPI_SWIGLU)
    assert L.q8_0_gemv_fused(ctypes.byref(W3), dummy, dummy, 96, 64, ctypes.byref(f), None, 0,
                             None) == q.Q8_EINVAL


def test_moe_and_router_reject_bad_arguments_on_host():
    L = q.lib()
    dummy = ctypes.c_void_p(16)
    We = _desc(128, 64, n=4)
    We.qs_stride, We.d_stride = q.q8_0_packed_size(128, 64)
    args = lambda S, mode: (ctypes.byref(We), dummy, dummy, dummy, dummy, 128, 64, S, mode, None,
                            None, None, None, 0, None)
    assert L.q8_0_moe_gemv(*args(0, q.Q8_MOE_SCATTER)) == q.Q8_EINVAL
    assert L.q8_0_moe_gemv(*args(9, q.Q8_MOE_SCATTER)) == q.Q8_EINVAL
    assert L.q8_0_moe_gemv(*args(2, 3)) == q.Q8_EINVAL
    assert L.q8_0_moe_gemv(*args(2, q.Q8_MOE_COMBINE | q.Q8_MOE_SWIGLU)) == q.Q8_EINVAL
    We.qs_stride = 16  # stride smaller than one packed matrix
    assert L.q8_0_moe_gemv(*args(2, q.Q8_MOE_SCATTER)) == q.Q8_EINVAL
    for (E, k) in [(0, 1), (1025, 1), (60, 0), (60, 9), (3, 4)]:
        assert L.q8_0_route_topk(dummy, E, k, dummy, dummy, None) == q.Q8_EINVAL
    assert L.q8_0_route_topk(None, 60, 4, dummy, dummy, None) == q.Q8_ENULL
    assert L.q8_0_argmax(dummy, -1, dummy, None, 0, None) == q.Q8_EINVAL
    assert L.q8_0_argmax(None, 5, dummy, None, 0, None) == q.Q8_ENULL
    assert L.q8_0_argmax(dummy, 0, dummy, None, 0, None) == q.Q8_OK  # empty: no-op


def test_empty_problems_are_noops():
    L = q.lib()
    dummy = ctypes.c_void_p(16)
    W = _desc(0, 64)
    assert L.q8_0_gemv(ctypes.byref(W), dummy, dummy, 0, 64, 1, None, 0, None) == q.Q8_OK
    assert L.q8_0_repack(dummy, 0, 64, dummy, dummy, None) == q.Q8_OK


def test_plans_and_workspace_sizes():
    p = q.q8_0_gemv_plan(151936, 896)
    assert p["wgs_per_tile"] == 1 and p["workgroups"] == 2374
    assert q.q8_0_workspace_bytes(q.Q8_OP_GEMV, 151936, 896, 1) == 0
    p = q.q8_0_gemv_plan(896, 4864)
    assert p["wgs_per_tile"] > 1
    ws = q.q8_0_workspace_bytes(q.Q8_OP_GEMV, 896, 4864, 1)
    assert ws >= 14 * p["units_per_tile"] * 64 * 4
    # argmax epilogue always needs the per-tile partials
    assert q.q8_0_workspace_bytes(q.Q8_OP_GEMV_FUSED, 151936, 896, q.Q8_EPI_ARGMAX) > 0
    assert q.q8_0_workspace_bytes(q.Q8_OP_ARGMAX, 151936, 0, 0) > 0
    assert q.q8_0_workspace_bytes(q.Q8_OP_GEMV, 64, 33, 1) == 0  # invalid shape
    for N in range(1, 9):
        assert q.q8_0_gemv_plan(4096, 12288, N)["workgroups"] > 0
