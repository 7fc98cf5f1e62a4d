"""Parity at the workloads' full sizes, in the launch configuration the
benchmark uses: every output of the single 896 x 896 GEMV, of the LM head
(151,936 rows) and of the 9B-class verify-chunk shapes at every N, against
the threaded fp64 oracle; sampled rows only for the K-quant formats."""
import numpy as np
import pytest

import block_quantized_gemv_amd as q
import oracle
import q8tol
import workloads as W
from gpu_util import host, pack, to_dev

pytestmark = pytest.mark.gpu


def test_single_gemv_896():
    c = W.C1
    m = W.matrix(c["cfg"], 0, 0, c["M"], c["K"])
    x = W.activations(c["cfg"], c["N"], c["K"])
    y = host(q.q8_0_gemv(pack(m), to_dev(x)))
    yr, S = oracle.gemv(m.aos(), x)
    q8tol.check(y, yr, S, "C1 896x896")


def test_lm_head_plain_gemv_every_row():
    c = W.C3
    m = W.matrix(c["cfg"], 0, W.MAT_LM_HEAD, c["M"], c["K"])
    x = W.activations(c["cfg"], 1, c["K"])
    y = host(q.q8_0_gemv(pack(m), to_dev(x)))
    yr, S = oracle.gemv(m.aos(), x)
    assert y.shape == (1, c["M"])
    q8tol.check(y, yr, S, "lm_head every row")


@pytest.mark.parametrize("mat", [W.MAT_GATE_UP, W.MAT_DOWN])
def test_verify_chunk_9b_shapes_every_row(mat):
    c = W.C4
    M, K = W.C4_SHAPES[mat]
    m = W.matrix(c["cfg"], 0, mat, M, K)
    p = pack(m)
    aos = m.aos()
    for N in (1,) + tuple(c["Ns"]):
        x = W.activations(c["cfg"], N, K, layer=N)
        y = host(q.q8_0_gemv(p, to_dev(x)))
        yr, S = oracle.gemv(aos, x)
        assert y.shape == (N, M)
        q8tol.check(y, yr, S, f"C4 {M}x{K} N={N} every row")


@pytest.mark.parametrize("N", [1, 8])
def test_integer_activation_9b_gate_up_every_row(N):
    """The opt-in integer-activation pair at the benchmarked shape: codes and
    binary16 scales bit-exact over the whole activation, every output of the
    product within the tolerance of the oracle on the same codes."""
    c = W.C4
    M, K = W.C4_SHAPES[W.MAT_GATE_UP]
    m = W.matrix(c["cfg"], 0, W.MAT_GATE_UP, M, K)
    x = W.activations(c["cfg"], N, K, layer=10 + N)
    qx, dx = q.q8_0_quantize_act(to_dev(x))
    eq, ed = oracle.quantize_act(x)
    assert np.array_equal(host(qx), eq)
    assert np.array_equal(host(dx).view(np.uint16), ed)
    y = host(q.q8_0_gemv_q8act(pack(m), qx, dx))
    yr, S = oracle.gemv_q8act(m.aos(), eq, ed)
    q8tol.check(y, yr, S, f"C4 gate_up int8 activations N={N} every row")


@pytest.mark.parametrize("mat", [W.MAT_GATE_UP, W.MAT_DOWN])
def test_q4k_9b_shapes_sampled(mat):
    """Q4_K weights (NEXT-2) at the 9B-class shapes the benchmark times, N = 1
    and 8, sampled rows against the oracle; tolerance as in test_gpu_q4k."""
    from test_gpu_q4k import check, pack4, s2_bound
    M, K = W.C4_SHAPES[mat]
    m = W.draw_q4k(W.rng(90, mat), M, K)
    p = pack4(m)
    g = np.random.default_rng(91 + mat)
    rows = np.unique(np.concatenate([g.integers(0, M, 256), [0, 63, 64, M - 1]]))
    sub = W.Q4KMatrix(m.q[rows], m.s[rows], m.m[rows], m.d[rows], m.dmin[rows])
    for N in (1, 8):
        x = W.activations(90, N, K, layer=N)
        y = host(q.q4k_gemv(p, to_dev(x)))
        yr, _ = oracle.q4k_gemv(sub.blocks(), x)
        check(y[:, rows], yr, s2_bound(sub, x), f"Q4_K {M}x{K} N={N}")


@pytest.mark.parametrize("mat", [W.MAT_GATE_UP, W.MAT_DOWN])
def test_q6k_9b_shapes_sampled(mat):
    """Q6_K weights (NEXT-2) at the 9B-class shapes the benchmark times, N = 1
    and 8, sampled rows against the oracle; tolerance as in test_gpu_q6k."""
    from test_gpu_q6k import check, pack6, s2_bound
    M, K = W.C4_SHAPES[mat]
    m = W.draw_q6k(W.rng(92, mat), M, K)
    p = pack6(m)
    g = np.random.default_rng(93 + mat)
    rows = np.unique(np.concatenate([g.integers(0, M, 256), [0, 63, 64, M - 1]]))
    sub = W.Q6KMatrix(m.code[rows], m.sc[rows], m.d[rows])
    for N in (1, 8):
        x = W.activations(92, N, K, layer=N)
        y = host(q.q6k_gemv(p, to_dev(x)))
        yr, _ = oracle.q6k_gemv(sub.blocks(), x)
        check(y[:, rows], yr, s2_bound(sub, x), f"Q6_K {M}x{K} N={N}")


@pytest.mark.parametrize("mat", [W.MAT_GATE_UP, W.MAT_DOWN])
def test_q5k_9b_shapes_sampled(mat):
    """Q5_K weights (NEXT-2) at the 9B-class shapes the benchmark times, N = 1
    and 8, sampled rows against the oracle; tolerance as in test_gpu_q5k."""
    from test_gpu_q5k import check, pack5, s2_bound
    M, K = W.C4_SHAPES[mat]
    m = W.draw_q5k(W.rng(94, mat), M, K)
    p = pack5(m)
    g = np.random.default_rng(95 + mat)
    rows = np.unique(np.concatenate([g.integers(0, M, 256), [0, 63, 64, M - 1]]))
    sub = W.Q5KMatrix(m.code[rows], m.s[rows], m.m[rows], m.d[rows], m.dmin[rows])
    for N in (1, 8):
        x = W.activations(94, N, K, layer=N)
        y = host(q.q5k_gemv(p, to_dev(x)))
        yr, _ = oracle.q5k_gemv(sub.blocks(), x)
        check(y[:, rows], yr, s2_bound(sub, x), f"Q5_K {M}x{K} N={N}")


@pytest.mark.parametrize("N", [1, 5])
def test_gemv_at_the_largest_k(N):
    """K = Q8_MAX_K (2^20, the largest the boundary accepts) with a ragged
    row count: every output against the oracle.  The longest units and the
    largest in-kernel offsets of the Q8_0 path."""
    M, K = 130, q.Q8_MAX_K
    g = W.rng(97, N, K)
    m = W.draw_matrix(g, M, K)
    x = W.draw_x(g, N, K)
    y = host(q.q8_0_gemv(pack(m), to_dev(x)))
    yr, S = oracle.gemv(m.aos(), x)
    q8tol.check(y, yr, S, f"gemv {M}x{K} N={N}")


def test_q4k_gemv_at_the_largest_k():
    """The same for Q4_K weights (K = 2^20, ragged M, N = 1 and 5)."""
    from test_gpu_q4k import check, pack4, s2_bound
    M, K = 65, q.Q8_MAX_K
    g = W.rng(98, M, K)
    m = W.draw_q4k(g, M, K)
    p = pack4(m)
    for N in (1, 5):
        x = W.draw_x(g, N, K)
        y = host(q.q4k_gemv(p, to_dev(x)))
        yr, _ = oracle.q4k_gemv(m.blocks(), x)
        check(y, yr, s2_bound(m, x), f"Q4_K {M}x{K} N={N}")
