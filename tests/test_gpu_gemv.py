"""GPU parity of the repack and the Q8_0 GEMV (N = 1..8) against the fp64
oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import block_quantized_gemv_amd as q
import oracle
import q8tol
import workloads as W
from gpu_util import DEV, expected_packed, host, pack, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K", [(1, 32), (64, 64), (65, 96), (130, 160), (200, 896),
                                 (333, 1408), (64, 4864)])
def test_repack_layout_bit_exact(M, K):
    m = W.draw_matrix(W.rng(10, M, K), M, K)
    p = pack(m)
    eq, ed = expected_packed(m.qs, m.d)
    assert np.array_equal(host(p.qs), eq)
    assert np.array_equal(host(p.d), ed)


SHAPES = [(1, 32), (7, 64), (64, 896), (65, 96), (130, 160), (200, 224), (896, 896),
          (1152, 896), (300, 4864), (333, 1408), (129, 2048), (64, 5632), (40, 12288)]


@pytest.mark.parametrize("M,K", SHAPES)
@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 6, 7, 8])
def test_gemv_matches_oracle(M, K, N):
    g = W.rng(20, M * 7 + N, K)
    m = W.draw_matrix(g, M, K)
    x = W.draw_x(g, N, K)
    p = pack(m)
    y = q.q8_0_gemv(p, to_dev(x))
    yr, S = oracle.gemv(m.aos(), x)
    q8tol.check(host(y), yr, S, f"gemv {M}x{K} N={N}")


def test_constant_quants_exact():
    """All quants q, scales d = 2^e, x in {-1, 0, 1}: every partial sum is an
    exact small integer times d, so the GPU result equals d*q*sum(x) exactly."""
    for (M, K) in [(64, 896), (130, 4864), (896, 896), (65, 12288)]:
        g = np.random.default_rng(M + K)
        x = g.integers(-1, 2, size=(2, K)).astype(np.float32)
        for qv in (-128, 127, -1, 0):
            for dbits in (0x3C00, 0x2000, 0x0001, 0x4400):
                d = np.array([dbits], dtype=np.uint16).view(np.float16)[0]
                m = W.Q8Matrix(np.full((M, K), qv, np.int8), np.full((M, K // 32), d))
                y = host(q.q8_0_gemv(pack(m), to_dev(x)))
                want = float(d) * qv * x.astype(np.float64).sum(axis=1)
                assert np.array_equal(y.astype(np.float64), np.repeat(want[:, None], M, 1)), \
                    (M, K, qv, dbits)


def test_one_hot_exact():
    """x = e_k selects d[r, k/32] * q[r, k], exact in fp32 (11 x 8 bits)."""
    M, K = 200, 1408
    m = W.draw_matrix(W.rng(21), M, K)
    # include subnormal, zero, negative and extreme scales
    d = m.d.view(np.uint16).copy()
    d[0, :] = 0x0001
    d[1, :] = 0x8000
    d[2, :] = 0xFBFF
    d[3, :] = 0x03FF
    m = W.Q8Matrix(m.qs, d.view(np.float16))
    m.qs[4, :] = -128
    p = pack(m)
    ks = [0, 1, 31, 32, 33, 127, 128, 700, K - 33, K - 1]
    x = np.zeros((len(ks[:8]), K), dtype=np.float32)
    for i, k in enumerate(ks[:8]):
        x[i, k] = 1.0
    y = host(q.q8_0_gemv(p, to_dev(x)))
    for i, k in enumerate(ks[:8]):
        want = (m.d[:, k // 32].astype(np.float64) * m.qs[:, k].astype(np.float64))
        assert np.array_equal(y[i].astype(np.float64), want), k
    x1 = np.zeros((1, K), dtype=np.float32)
    x1[0, K - 1] = -2.0
    y = host(q.q8_0_gemv(p, to_dev(x1)))[0]
    assert np.array_equal(y.astype(np.float64),
                          -2.0 * m.d[:, -1].astype(np.float64) * m.qs[:, -1].astype(np.float64))


def test_edge_scales_and_quants_within_tolerance():
    M, K = 256, 896
    g = W.rng(22)
    m = W.draw_matrix(g, M, K)
    d = m.d.view(np.uint16).copy()
    d[:64, ::3] = 0x0001       # smallest subnormal
    d[64:128, ::2] = 0x8000    # negative zero
    d[128:160, :] = 0x7BFF     # 65504
    d[160:192, :] |= 0x8000    # negative scales
    qs = m.qs.copy()
    qs[192:, ::5] = -128
    qs[200:210, :] = 0         # all-zero rows: tolerance is the 1e-6 floor
    m = W.Q8Matrix(qs, d.view(np.float16))
    x = W.draw_x(g, 3, K)
    y = host(q.q8_0_gemv(pack(m), to_dev(x)))
    yr, S = oracle.gemv(m.aos(), x)
    q8tol.check(y, yr, S, "edge scales")
    assert np.all(y[:, 200:210] == 0)


@pytest.mark.parametrize("N", [5, 8])
def test_matrix_core_split_edge_values(N):
    """N >= 5 runs each block as bf16 matrix-core products, with every fp32
    activation cut into three bf16 parts whose sum is exact.  Activations
    with all 24 significand bits, values just above each bf16 cut, huge and
    tiny magnitudes and signed zeros, with edge scales.  Then one-hot
    columns holding full-significand values against power-of-two scales: the
    block sum q * x is then one product, so the result must be exact."""
    M, K = 200, 1408
    g = W.rng(25, N)
    m = W.draw_matrix(g, M, K)
    d = m.d.view(np.uint16).copy()
    d[:32, ::3] = 0x0001       # smallest subnormal
    d[32:64, :] = 0x7BFF       # 65504
    d[64:96, :] |= 0x8000      # negative scales
    qs = m.qs.copy()
    qs[96:128, ::5] = -128
    m = W.Q8Matrix(qs, d.view(np.float16))
    x = W.draw_x(g, N, K)
    bits = x.view(np.uint32)
    bits[0, ::2] |= 0x007FFFFF                        # all significand bits set
    bits[1 % N, ::3] = (bits[1 % N, ::3] & 0xFFFF0000) | 0x00008001  # just above the cuts
    x[2 % N, ::7] *= np.float32(1e25)   # d = 65504 rows stay far below fp32 overflow
    x[3 % N, ::11] *= np.float32(1e-30)
    x[4 % N, ::13] = np.float32(-0.0)
    y = host(q.q8_0_gemv(pack(m), to_dev(x)))
    yr, S = oracle.gemv(m.aos(), x)
    q8tol.check(y, yr, S, f"matrix-core edge values N={N}")

    dpow = np.full((M, K // 32), np.float16(0.5))
    dpow[::2] = np.float16(-4.0)
    mp = W.Q8Matrix(m.qs, dpow)
    xo = np.zeros((N, K), dtype=np.float32)
    ks = [0, 31, 32, 100, 700, 1000, K - 33, K - 1][:N]
    vals = (np.array([1.0 + 2.0 ** -23, -3.14159274, 1.0e-20, 7.0e20, 0.1, -1.9999999, 1234.5678,
                      2.0 ** -100], dtype=np.float32))[:N]
    for i, k in enumerate(ks):
        xo[i, k] = vals[i]
    y = host(q.q8_0_gemv(pack(mp), to_dev(xo)))
    for i, k in enumerate(ks):
        want = np.float32(dpow[:, k // 32].astype(np.float32)
                          * (m.qs[:, k].astype(np.float32) * np.float32(vals[i])))
        assert np.array_equal(y[i], want.astype(np.float32)), (N, i, k)


@pytest.mark.parametrize("M,K,N", [(896, 4864, 1), (896, 896, 1), (4096, 12288, 2),
                                   (9728, 896, 1), (1152, 896, 8)])
def test_repeated_calls_bitwise_identical(M, K, N):
    g = W.rng(23, M, K)
    m = W.draw_matrix(g, M, K)
    p = pack(m)
    x = to_dev(W.draw_x(g, N, K))
    y0 = q.q8_0_gemv(p, x).clone()
    for _ in range(20):
        y = q.q8_0_gemv(p, x)
        assert torch.equal(y, y0)


def test_rejects_host_and_misaligned_pointers():
    m = W.draw_matrix(W.rng(24), 64, 64)
    p = pack(m)
    x_host = torch.zeros(64, dtype=torch.float32)
    y = torch.empty(64, dtype=torch.float32, device=DEV)
    L = q.lib()
    import ctypes
    rc = L.q8_0_gemv(ctypes.byref(p.desc), x_host.data_ptr(), y.data_ptr(), 64, 64, 1, None, 0,
                     None)
    assert rc == q.Q8_EHOSTPTR
    xb = torch.zeros(65, dtype=torch.float32, device=DEV)
    raw = xb.data_ptr() + 2  # not 4-byte aligned
    rc = L.q8_0_gemv(ctypes.byref(p.desc), raw, y.data_ptr(), 64, 64, 1, None, 0, None)
    assert rc == q.Q8_EALIGN
    # workspace too small for a split-K plan
    m2 = W.draw_matrix(W.rng(25), 896, 4864)
    p2 = pack(m2)
    x2 = torch.zeros(4864, dtype=torch.float32, device=DEV)
    y2 = torch.empty(896, dtype=torch.float32, device=DEV)
    need = q.q8_0_workspace_bytes(q.Q8_OP_GEMV, 896, 4864, 1)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    rc = L.q8_0_gemv(ctypes.byref(p2.desc), x2.data_ptr(), y2.data_ptr(), 896, 4864, 1,
                     ws.data_ptr(), need - 1, None)
    assert rc == q.Q8_EWORKSPACE
    rc = L.q8_0_gemv(ctypes.byref(p2.desc), x2.data_ptr(), y2.data_ptr(), 896, 4864, 1,
                     None, 0, None)
    assert rc == q.Q8_EWORKSPACE


def test_one_workspace_serves_interleaved_shapes():
    """Split-K GEMVs, fused argmax and standalone argmax of different shapes
    share one workspace: counters never land on another call's partials."""
    g = W.rng(26)
    shapes = [(896, 4864), (5000, 896), (130, 12288), (4096, 2048)]
    mats = [W.draw_matrix(g, M, K) for (M, K) in shapes]
    packs = [pack(m) for m in mats]
    xs = [W.draw_x(g, 1, K)[0] for (_, K) in shapes]
    need = max([q.q8_0_workspace_bytes(q.Q8_OP_GEMV, M, K, 1) for (M, K) in shapes] +
               [q.q8_0_workspace_bytes(q.Q8_OP_GEMV_FUSED, M, K, q.Q8_EPI_ARGMAX)
                for (M, K) in shapes] + [q.q8_0_workspace_bytes(q.Q8_OP_ARGMAX, 100003, 0, 0)])
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    refs = [oracle.gemv(m.aos(), x) for m, x in zip(mats, xs)]
    v = W.draw_x(g, 1, 100003)[0]
    am = torch.zeros(1, dtype=torch.int32, device=DEV)
    for rnd in range(3):
        for i, (M, K) in enumerate(shapes):
            y = q.q8_0_gemv(packs[i], to_dev(xs[i]), workspace=ws)
            q8tol.check(host(y), refs[i][0], refs[i][1], f"round {rnd} gemv {M}x{K}")
            y2 = torch.empty(M, dtype=torch.float32, device=DEV)
            f = q.make_fusion(epilogue=q.Q8_EPI_ARGMAX, argmax_out=am)
            q.q8_0_gemv_fused(packs[i], to_dev(xs[i]), y2, f, workspace=ws)
            yh = host(y2)
            assert int(host(am)[0]) == int(np.argmax(yh)), (rnd, M, K)
            out = q.q8_0_argmax(to_dev(v), workspace=ws)
            assert int(host(out)[0]) == int(np.argmax(v))
    # every counter is back at zero
    assert int(ws[:65536].view(torch.int32).abs().sum().item()) == 0


@pytest.mark.parametrize("M,K", [(64, 96), (128, 896), (9728, 896), (2816, 2048)])
def test_repack_gate_up_pairs_layout_bit_exact(M, K):
    m = W.draw_matrix(W.rng(11, M, K), M, K)
    p = pack(m, layout=q.Q8_LAYOUT_GATE_UP_PAIRS)
    eq, ed = expected_packed(m.qs, m.d, q.Q8_LAYOUT_GATE_UP_PAIRS)
    assert np.array_equal(host(p.qs), eq)
    assert np.array_equal(host(p.d), ed)


@pytest.mark.parametrize("M,K,layout", [(1, 32, 0), (65, 96, 0), (200, 896, 0), (333, 1408, 0),
                                         (128, 96, 1), (9728, 896, 1), (2816, 2048, 1)])
@pytest.mark.parametrize("tiles", [1, 2.5, 1000])
def test_repack_from_host_memory_bit_exact(M, K, layout, tiles):
    """q8_0_repack_host moves the blocks from a numpy array through a staging
    buffer of one tile, two and a half tiles (ragged last band) or the whole
    matrix; the packed bytes equal the layout written out from the header."""
    m = W.draw_matrix(W.rng(12, M, K), M, K)
    aos = np.ascontiguousarray(m.aos().reshape(-1))
    smin = q.q8_0_repack_staging_bytes(M, K)
    assert smin == 64 * (K // 32) * 34
    staging = torch.empty(int(smin * tiles), dtype=torch.uint8, device=DEV)
    qb, db = q.q8_0_packed_size(M, K)
    qs = torch.full((qb,), 0xA5, dtype=torch.uint8, device=DEV)
    d = torch.full((db,), 0xA5, dtype=torch.uint8, device=DEV)
    q.q8_0_repack_host(aos, M, K, qs, d, staging, layout=layout)
    eq, ed = expected_packed(m.qs, m.d, layout)
    assert np.array_equal(host(qs), eq)
    assert np.array_equal(host(d), ed)


def test_repack_from_host_rejects_small_staging():
    M, K = 100, 64
    m = W.draw_matrix(W.rng(13, M, K), M, K)
    aos = np.ascontiguousarray(m.aos().reshape(-1))
    qb, db = q.q8_0_packed_size(M, K)
    qs = torch.empty(qb, dtype=torch.uint8, device=DEV)
    d = torch.empty(db, dtype=torch.uint8, device=DEV)
    staging = torch.empty(q.q8_0_repack_staging_bytes(M, K) - 1, dtype=torch.uint8, device=DEV)
    with pytest.raises(q.Q8Error) as e:
        q.q8_0_repack_host(aos, M, K, qs, d, staging)
    assert e.value.code == q.Q8_EWORKSPACE


@pytest.mark.parametrize("M,K,N", [(128, 96, 1), (9728, 896, 1), (640, 2048, 3)])
def test_gemv_on_pairs_layout_writes_row_order(M, K, N):
    g = W.rng(27, M, K)
    m = W.draw_matrix(g, M, K)
    x = W.draw_x(g, N, K)
    y = host(q.q8_0_gemv(pack(m, layout=q.Q8_LAYOUT_GATE_UP_PAIRS), to_dev(x)))
    yr, S = oracle.gemv(m.aos(), x)
    q8tol.check(y, yr, S, f"pairs layout {M}x{K} N={N}")


@pytest.mark.parametrize("M,K", [(128, 96), (9728, 896), (2816, 2048), (192, 64)])
def test_fused_rmsnorm_swiglu_pairs_layout(M, K):
    """SwiGLU epilogue on the gate/up pairs layout against the oracle: gate and
    up rows each within the GEMV tolerance plus the fp32 RMS scale's rounding,
    propagated to first order through silu(g)*u."""
    U = 2.0 ** -24
    g = W.rng(28, M, K)
    m = W.draw_matrix(g, M, K)
    x = W.draw_x(g, 1, K)[0]
    I = M // 2
    y = torch.empty(I, dtype=torch.float32, device=DEV)
    f = q.make_fusion(prologue=q.Q8_PRO_RMSNORM, epilogue=q.Q8_EPI_SWIGLU, eps=1e-6)
    q.q8_0_gemv_fused(pack(m, layout=q.Q8_LAYOUT_GATE_UP_PAIRS), to_dev(x), y, f)
    gu, S = oracle.gemv(m.aos(), oracle.rmsnorm(x.astype(np.float64), 1e-6))
    gr, ur = gu[:I], gu[I:]
    tg = q8tol.bound(S[:I]) + 34 * U * np.abs(gr)
    tu = q8tol.bound(S[I:]) + 34 * U * np.abs(ur)
    sg = 1.0 / (1.0 + np.exp(-gr))
    sil = gr * sg
    b = (np.abs(sg * (1.0 + gr * (1.0 - sg))) * np.abs(ur) * tg + (np.abs(sil) + 1.2 * tg) * tu
         + 0.5 * tg * tg * np.abs(ur) + 8 * U * np.abs(sil * ur))
    err = np.abs(host(y).astype(np.float64) - oracle.swiglu(gr, ur))
    assert np.all(err <= b), float((err / b).max())


# ---- one argmax per column (verify chunk) ------------------------------------
@pytest.mark.parametrize("M,K", [(1, 32), (65, 96), (1000, 128), (4097, 896), (2816, 2048)])
@pytest.mark.parametrize("N", [1, 2, 4, 8])
def test_gemv_argmax_columns(M, K, N):
    """Each column's pick is the lowest index of that column's largest GPU
    logit (bit-exact against numpy on the GPU's own values), the logits equal
    the plain GEMV's bit for bit, and they match the oracle."""
    g = W.rng(30, M * 5 + N, K)
    m = W.draw_matrix(g, M, K)
    x = W.draw_x(g, N, K)
    p = pack(m)
    y, am = q.q8_0_gemv_argmax(p, to_dev(x))
    yh, amh = host(y).reshape(N, M), host(am)
    assert np.array_equal(amh, np.argmax(yh, axis=1)), (amh, np.argmax(yh, axis=1))
    y_plain = host(q.q8_0_gemv(p, to_dev(x))).reshape(N, M)
    assert np.array_equal(yh.view(np.uint32), y_plain.view(np.uint32))
    yr, S = oracle.gemv(m.aos(), x)
    q8tol.check(yh, yr.reshape(N, M), S.reshape(N, M), f"gemv_argmax {M}x{K} N={N}")


@pytest.mark.parametrize("N", [2, 8])
def test_gemv_argmax_lm_head_shape_and_planted_ties(N):
    """lm_head 151936 x 896 with N verify columns.  Copies of the best row of
    each column planted at a lower and a higher index give bitwise-equal
    logits (per-row arithmetic does not depend on the row index); the pick
    must be the lowest copy.  Against the fp64 oracle the pick lies within the
    tolerance band of the true maximum."""
    M, K = 151936, 896
    m = W.matrix(3, 0, W.MAT_LM_HEAD, M, K)
    x = W.activations(31, N, K)
    qs, d = m.qs.copy(), m.d.copy()
    # the oracle's best row of column 0, copied to a lower and a higher index
    y0, S0 = oracle.gemv(m.aos(), x[:1])
    order = np.argsort(-y0[0])
    best = int(order[0])
    lo = best // 2 if best > 0 else M - 2
    hi = (best + M) // 2 if best < M - 1 else 1
    for r in (lo, hi):
        qs[r], d[r] = qs[best], d[best]
    planted = W.Q8Matrix(qs, d)
    p = pack(planted)
    y, am = q.q8_0_gemv_argmax(p, to_dev(x))
    yh, amh = host(y).reshape(N, M), host(am)
    assert np.array_equal(amh, np.argmax(yh, axis=1))
    assert yh[0, lo] == yh[0, best] == yh[0, hi]
    # the runner-up among rows that are not copies of the best one
    second = next(int(r) for r in order[1:] if r not in (lo, hi))
    tol = 2e-5 * S0[0] + 1e-6
    if y0[0][best] - y0[0][second] > tol[best] + tol[second]:
        assert amh[0] == min(lo, best, hi)
    for n in range(N):
        pick = int(amh[n])
        cand = np.unique(np.concatenate([[pick], np.argsort(-yh[n])[:8]]))
        yr, S = oracle.gemv(planted.aos()[cand], x[n:n + 1])
        top = float(yr[0].max())
        tol = 2e-5 * S[0] + 1e-6
        assert yr[0][list(cand).index(pick)] >= top - 2 * tol.max()


def test_gemv_argmax_rejects_bad_arguments():
    M, K = 64, 64
    m = W.draw_matrix(W.rng(32, M, K), M, K)
    p = pack(m)
    x = to_dev(W.draw_x(W.rng(33, 2, K), 2, K))
    y = torch.empty(2, M, device=DEV)
    lib = q.lib()
    ws = q.Workspace(q.q8_0_workspace_bytes(q.Q8_OP_GEMV_ARGMAX, M, K, 2))
    wsp, wsb = ws.get(ws.buf.numel())
    assert lib.q8_0_gemv_argmax(p.desc, x.data_ptr(), y.data_ptr(), M, K, 2, None, wsp, wsb,
                                None) == q.Q8_ENULL
    am = torch.empty(2, dtype=torch.int32, device=DEV)
    assert lib.q8_0_gemv_argmax(p.desc, x.data_ptr(), y.data_ptr(), M, K, 9, am.data_ptr(), wsp,
                                wsb, None) == q.Q8_EINVAL
    host_am = np.zeros(2, dtype=np.int32)
    assert lib.q8_0_gemv_argmax(p.desc, x.data_ptr(), y.data_ptr(), M, K, 2,
                                host_am.ctypes.data, wsp, wsb, None) == q.Q8_EHOSTPTR
    assert lib.q8_0_gemv_argmax(p.desc, x.data_ptr(), y.data_ptr(), M, K, 2, am.data_ptr() + 2,
                                wsp, wsb, None) == q.Q8_EALIGN


def test_split_plans_replay_bitwise_in_a_graph():
    """GEMVs whose tiles span several workgroups (ticketed cross-workgroup
    fold, counters the kernel itself returns to zero) captured in a HIP graph:
    every replay, with eager calls on the same workspace between replays,
    equals the eager result bitwise.  Q8_0 at N = 1 and 8 and Q6_K at N = 1."""
    from test_gpu_q6k import pack6
    g = W.rng(21)
    cases = []
    m = W.draw_matrix(g, 896, 4864)
    p = pack(m)
    for N in (1, 8):
        x = to_dev(W.draw_x(g, N, 4864))
        assert q.q8_0_gemv_plan(896, 4864, N)["wgs_per_tile"] > 1
        cases.append(lambda y, ws, p=p, x=x: q.q8_0_gemv(p, x, y, ws))
    m6 = W.draw_q6k(g, 256, 12288)
    p6 = pack6(m6)
    x6 = to_dev(W.draw_x(g, 1, 12288))
    cases.append(lambda y, ws: q.q6k_gemv(p6, x6, y, ws))
    ws = q.Workspace(1 << 22)
    for run in cases:
        eager = run(None, ws).clone()
        torch.cuda.synchronize()
        y = torch.empty_like(eager)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            run(y, ws)
        for _ in range(4):
            y.zero_()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(y, eager)
            assert torch.equal(run(None, ws), eager)  # eager call between replays
            torch.cuda.synchronize()
