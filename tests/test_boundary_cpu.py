"""CPU-side checks of the C-ABI library: it loads, exports every entry point
declared in include/q8gemv.h, and rejects bad arguments on the host before
any device work (no GPU is touched by these tests)."""
import ctypes
import os
import re

import numpy as np
import pytest

import block_quantized_gemv_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q8gemv.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b((?:q8|q4k|q5k|q6k)_\w+)\s*\(", src)))


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


def test_repack_host_staging_and_host_checks():
    """q8_0_repack_host: staging size is one 64-row tile of 34-byte blocks;
    shape, layout and null arguments are rejected before any copy."""
    L = q.lib()
    assert q.q8_0_repack_staging_bytes(896, 896) == 64 * 28 * 34
    assert q.q8_0_repack_staging_bytes(1, 32) == 64 * 34
    assert q.q8_0_repack_staging_bytes(0, 32) == 0
    assert q.q8_0_repack_staging_bytes(4, 33) == 0
    dummy = ctypes.c_void_p(16)
    big = 1 << 30
    for M, K, layout in [(4, 33, 0), (-1, 32, 0), (96, 64, 1), (64, 64, 2)]:
        assert L.q8_0_repack_host(dummy, M, K, layout, dummy, dummy, dummy, big,
                                  None) == q.Q8_EINVAL, (M, K, layout)
    assert L.q8_0_repack_host(None, 64, 64, 0, dummy, dummy, dummy, big, None) == q.Q8_ENULL
    assert L.q8_0_repack_host(dummy, 64, 64, 0, dummy, dummy, None, big, None) == q.Q8_ENULL
    assert L.q8_0_repack_host(dummy, 0, 64, 0, dummy, dummy, dummy, 0, None) == q.Q8_OK


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


def _chain(n_layers=2, hidden=896, n_heads=14, n_kv=2, hd=64, inter=4864, vocab=2048, eps=1e-6,
           gu_layout=q.Q8_LAYOUT_GATE_UP_PAIRS, lm=True):
    """A chain description with fake (host) weight pointers; only the scalar
    checks that precede any pointer query can pass with it."""
    mq = (n_heads + 2 * n_kv) * hd
    mk = lambda M, K, lay=q.Q8_LAYOUT_ROWS: q.q8_0_weights(16, 16, M, K, 1, 0, 0, lay, 0)
    arrs = {
        "qkv": (q.q8_0_weights * max(n_layers, 1))(*[mk(mq, hidden)] * max(n_layers, 1)),
        "wo": (q.q8_0_weights * max(n_layers, 1))(*[mk(hidden, n_heads * hd)] * max(n_layers, 1)),
        "gate_up": (q.q8_0_weights * max(n_layers, 1))(
            *[mk(2 * inter, hidden, gu_layout)] * max(n_layers, 1)),
        "down": (q.q8_0_weights * max(n_layers, 1))(*[mk(hidden, inter)] * max(n_layers, 1)),
    }
    lmw = mk(vocab, hidden) if lm else None
    d = q.q8_0_chain_desc(n_layers, hidden, n_heads, n_kv, hd, inter, vocab if lm else 0, eps,
                          arrs["qkv"], arrs["wo"], arrs["gate_up"], arrs["down"],
                          ctypes.pointer(lmw) if lm else None)
    return d, (arrs, lmw)


def test_chain_workspace_bytes_and_host_validation():
    L = q.lib()
    d, keep = _chain()
    nbytes = L.q8_0_chain_workspace_bytes(ctypes.byref(d))
    # header + table + 2 layers of tagged records (8 bytes per entry) + argmax partials
    assert nbytes >= 256 + 2 * 8 * (1152 + 896 + 4864 + 896)
    bad = [dict(gu_layout=q.Q8_LAYOUT_ROWS),   # gate_up must use the pairs layout
           dict(hidden=900), dict(inter=4870), dict(n_kv=3), dict(hd=40),
           dict(hidden=1056),                  # rows longer than one task covers (1024)
           dict(inter=8224),                   # down's K slice per XCD longer than 1024
           dict(eps=-1.0), dict(n_layers=-1)]
    for kw in bad:
        d, keep = _chain(**kw)
        assert L.q8_0_chain_workspace_bytes(ctypes.byref(d)) == 0, kw
        plan = q.q8_0_chain_plan()
        rc = L.q8_0_chain_prepare(ctypes.byref(d), ctypes.c_void_p(256), 1 << 30,
                                  ctypes.byref(plan), None)
        assert rc == q.Q8_EINVAL, (kw, rc)
    # vocab > 0 without an LM head descriptor
    d, keep = _chain()
    d.lm_head = None
    assert L.q8_0_chain_prepare(ctypes.byref(d), ctypes.c_void_p(256), 1 << 30,
                                ctypes.byref(q.q8_0_chain_plan()), None) == q.Q8_ENULL
    # NULL plan / description
    d, keep = _chain()
    assert L.q8_0_chain_prepare(ctypes.byref(d), ctypes.c_void_p(256), 1 << 30, None,
                                None) == q.Q8_ENULL
    assert L.q8_0_chain_prepare(None, ctypes.c_void_p(256), 1 << 30,
                                ctypes.byref(q.q8_0_chain_plan()), None) == q.Q8_ENULL
    # a host pointer where the workspace must be device memory
    buf = ctypes.create_string_buffer(1 << 12)
    aligned = (ctypes.addressof(buf) + 255) // 256 * 256
    rc = L.q8_0_chain_prepare(ctypes.byref(d), ctypes.c_void_p(aligned), 1 << 30,
                              ctypes.byref(q.q8_0_chain_plan()), None)
    assert rc in (q.Q8_EHOSTPTR, q.Q8_ELAUNCH), rc
    # run / read reject an empty plan before touching anything
    plan = q.q8_0_chain_plan()
    assert L.q8_0_chain_run(ctypes.byref(plan), None, None, None, None, None, None) == q.Q8_EINVAL
    assert L.q8_0_chain_read(ctypes.byref(plan), None, 0, 0, None, None) == q.Q8_EINVAL


def test_gemv_argmax_rejects_bad_arguments_on_host():
    L = q.lib()
    dummy = ctypes.c_void_p(16)
    W = _desc(64, 32)
    assert L.q8_0_gemv_argmax(ctypes.byref(W), dummy, dummy, 64, 32, 2, None, None, 0,
                              None) == q.Q8_ENULL
    for N in (0, 9):
        assert L.q8_0_gemv_argmax(ctypes.byref(W), dummy, dummy, 64, 32, N, dummy, None, 0,
                                  None) == q.Q8_EINVAL
    assert L.q8_0_gemv_argmax(ctypes.byref(W), dummy, dummy, 64, 33, 1, dummy, None, 0,
                              None) == q.Q8_EINVAL
    # the per-column partials need workspace for every column
    one = q.q8_0_workspace_bytes(q.Q8_OP_GEMV_ARGMAX, 151936, 896, 1)
    eight = q.q8_0_workspace_bytes(q.Q8_OP_GEMV_ARGMAX, 151936, 896, 8)
    assert 0 < one < eight
    assert q.q8_0_workspace_bytes(q.Q8_OP_GEMV_ARGMAX, 151936, 896, 9) == 0


def test_q8act_rejects_bad_arguments_on_host():
    """Shape and null checks of the integer-activation entry points run
    before any device access."""
    L = q.lib()
    dummy = ctypes.c_void_p(16)
    for K, N in ((33, 1), (0, 1), (64, 0), (64, 9)):
        assert L.q8_0_quantize_act(dummy, K, N, dummy, dummy, None) == q.Q8_EINVAL, (K, N)
    assert L.q8_0_quantize_act(None, 64, 1, dummy, dummy, None) == q.Q8_ENULL
    assert L.q8_0_quantize_act(dummy, 64, 1, dummy, None, None) == q.Q8_ENULL
    W = _desc(64, 32)
    for N in (0, 9):
        assert L.q8_0_gemv_q8act(ctypes.byref(W), dummy, dummy, dummy, 64, 32, N, None, 0,
                                 None) == q.Q8_EINVAL
    assert L.q8_0_gemv_q8act(ctypes.byref(W), dummy, dummy, dummy, 64, 33, 1, None, 0,
                             None) == q.Q8_EINVAL
    assert L.q8_0_gemv_q8act(ctypes.byref(W), None, dummy, dummy, 64, 32, 1, None, 0,
                             None) == q.Q8_ENULL
    assert L.q8_0_gemv_q8act(ctypes.byref(W), dummy, None, dummy, 64, 32, 1, None, 0,
                             None) == q.Q8_ENULL


def test_q4k_rejects_bad_arguments_on_host():
    """Shape and null checks of the Q4_K entry points (no device access)."""
    L = q.lib()
    dummy = ctypes.c_void_p(16)
    qb, mb = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.q4k_packed_size(130, 512, ctypes.byref(qb), ctypes.byref(mb)) == q.Q8_OK
    assert (qb.value, mb.value) == (192 * 256, 192 * 2 * 16)  # 3 tiles of 64 rows
    for K in (0, 32, 288, 500):
        assert L.q4k_packed_size(64, K, ctypes.byref(qb), ctypes.byref(mb)) == q.Q8_EINVAL, K
        assert L.q4k_repack(dummy, 64, K, dummy, dummy, None) == q.Q8_EINVAL, K
    assert L.q4k_packed_size(64, 256, None, ctypes.byref(mb)) == q.Q8_ENULL
    assert L.q4k_repack(None, 64, 256, dummy, dummy, None) == q.Q8_ENULL
    W = q.q4k_weights(16, 16, 64, 256)
    for N in (0, 9):
        assert L.q4k_gemv(ctypes.byref(W), dummy, dummy, 64, 256, N, None, 0, None) == q.Q8_EINVAL
    assert L.q4k_gemv(ctypes.byref(W), dummy, dummy, 64, 512, 1, None, 0, None) == q.Q8_EINVAL
    assert L.q4k_gemv(None, dummy, dummy, 64, 256, 1, None, 0, None) == q.Q8_ENULL
    assert L.q4k_gemv(ctypes.byref(W), None, dummy, 64, 256, 1, None, 0, None) == q.Q8_ENULL
    # every column runs in the one launch, so a split plan's partials grow with
    # N; they always follow the 64 KiB counter region
    for op in (q.Q8_OP_Q4K_GEMV, q.Q8_OP_Q5K_GEMV, q.Q8_OP_Q6K_GEMV):
        ws = {N: q.q8_0_workspace_bytes(op, 4096, 12288, N) for N in range(1, 9)}
        assert all(ws[N] < ws[N + 1] for N in range(1, 8)), ws
        assert all(v >= 65536 + 64 * 64 * 4 * N for N, v in ws.items()), ws  # 64 tiles, split K
        assert q.q8_0_workspace_bytes(op, 64, 256, 1) == 0  # one quad: one unit
    for op in (q.Q8_OP_Q4K_GEMV, q.Q8_OP_Q5K_GEMV, q.Q8_OP_Q6K_GEMV):
        assert q.q8_0_workspace_bytes(op, 4096, 4000, 1) == 0
        assert q.q8_0_workspace_bytes(op, 4096, 4096, 9) == 0


def test_q6k_rejects_bad_arguments_on_host():
    L = q.lib()
    dummy = ctypes.c_void_p(16)
    a, b, c = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    assert L.q6k_packed_size(130, 512, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)) == 0
    assert (a.value, b.value, c.value) == (192 * 256, 192 * 128, 192 * 4 * 16)
    for K in (0, 32, 288):
        assert L.q6k_packed_size(64, K, ctypes.byref(a), ctypes.byref(b),
                                 ctypes.byref(c)) == q.Q8_EINVAL
        assert L.q6k_repack(dummy, 64, K, dummy, dummy, dummy, None) == q.Q8_EINVAL
    assert L.q6k_repack(dummy, 64, 256, dummy, None, dummy, None) == q.Q8_ENULL
    W = q.q6k_weights(16, 16, 16, 64, 256)
    for N in (0, 9):
        assert L.q6k_gemv(ctypes.byref(W), dummy, dummy, 64, 256, N, None, 0, None) == q.Q8_EINVAL
    assert L.q6k_gemv(ctypes.byref(W), dummy, dummy, 64, 512, 1, None, 0, None) == q.Q8_EINVAL
    W2 = q.q6k_weights(16, None, 16, 64, 256)
    assert L.q6k_gemv(ctypes.byref(W2), dummy, dummy, 64, 256, 1, None, 0, None) == q.Q8_ENULL


def test_q5k_rejects_bad_arguments_on_host():
    L = q.lib()
    dummy = ctypes.c_void_p(16)
    a, b, c = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    assert L.q5k_packed_size(130, 512, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)) == 0
    assert (a.value, b.value, c.value) == (192 * 256, 192 * 64, 192 * 2 * 16)
    for K in (0, 32, 288):
        assert L.q5k_packed_size(64, K, ctypes.byref(a), ctypes.byref(b),
                                 ctypes.byref(c)) == q.Q8_EINVAL
        assert L.q5k_repack(dummy, 64, K, dummy, dummy, dummy, None) == q.Q8_EINVAL
    assert L.q5k_repack(dummy, 64, 256, dummy, None, dummy, None) == q.Q8_ENULL
    assert L.q5k_packed_size(64, 256, None, ctypes.byref(b), ctypes.byref(c)) == q.Q8_ENULL
    W = q.q5k_weights(16, 16, 16, 64, 256)
    for N in (0, 9):
        assert L.q5k_gemv(ctypes.byref(W), dummy, dummy, 64, 256, N, None, 0, None) == q.Q8_EINVAL
    assert L.q5k_gemv(ctypes.byref(W), dummy, dummy, 64, 512, 1, None, 0, None) == q.Q8_EINVAL
    assert L.q5k_gemv(None, dummy, dummy, 64, 256, 1, None, 0, None) == q.Q8_ENULL
    W2 = q.q5k_weights(16, None, 16, 64, 256)
    assert L.q5k_gemv(ctypes.byref(W2), dummy, dummy, 64, 256, 1, None, 0, None) == q.Q8_ENULL
    # M = 0: nothing to do, nothing touched
    W0 = q.q5k_weights(16, 16, 16, 0, 256)
    assert L.q5k_gemv(ctypes.byref(W0), dummy, dummy, 0, 256, 1, None, 0, None) == q.Q8_OK
    assert L.q5k_repack(dummy, 0, 256, dummy, dummy, dummy, None) == q.Q8_OK
    # at N = 1 the plan is the Q4_K one (same quads, same wave count)
    for (M, K) in [(151936, 1024), (4096, 12288), (64, 256)]:
        assert (q.q8_0_workspace_bytes(q.Q8_OP_Q5K_GEMV, M, K, 1) ==
                q.q8_0_workspace_bytes(q.Q8_OP_Q4K_GEMV, M, K, 1))


def test_plan_invariants_over_random_shapes():
    """The planner's output is a valid launch for every shape: waves per
    workgroup within the kernel's launch bound, units within the K range,
    workgroups covering every unit of every tile with none empty, and a
    workspace large enough for the cross-workgroup partials."""
    g = np.random.default_rng(123)
    shapes = [(int(g.integers(1, 200000)), 32 * int(g.integers(1, 600)), int(g.integers(1, 9)))
              for _ in range(1500)]
    shapes += [(24576, 4096, N) for N in range(1, 9)] + [(151936, 896, N) for N in range(1, 9)]
    shapes += [(64 * t, 4096, N) for t in (255, 256, 257, 383, 384, 511, 512, 513) for N in (1, 2, 8)]
    for (M, K, N) in shapes:
        p = q.q8_0_gemv_plan(M, K, N)
        T, quads = -(-M // 64), -(-K // 128)
        W, U, P = p["waves_per_wg"], p["units_per_tile"], p["wgs_per_tile"]
        assert 1 <= W <= (16 if N <= 2 else 8), (M, K, N, p)
        assert 1 <= U <= quads, (M, K, N, p)
        assert P == -(-U // W) and U > (P - 1) * W, (M, K, N, p)
        assert p["workgroups"] == T * P, (M, K, N, p)
        ws = q.q8_0_workspace_bytes(q.Q8_OP_GEMV, M, K, N)
        if P > 1:
            assert ws >= 65536 + T * U * N * 64 * 4, (M, K, N, p, ws)
        else:
            assert ws == 0, (M, K, N, p, ws)
