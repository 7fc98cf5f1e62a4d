"""GPU argmax (standalone and fused into the LM-head GEMV) and the MoE
router, against numpy's first-occurrence argmax and the oracle router."""
import numpy as np
import pytest
import torch

import block_quantized_gemv_amd as q
import oracle
import q8tol
import workloads as W
from gpu_util import DEV, host, pack, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [1, 5, 64, 1000, 2049, 151936, (1 << 20) + 3])
def test_argmax_matches_numpy_first_occurrence(n):
    g = np.random.default_rng(n)
    v = g.standard_normal(n).astype(np.float32)
    out = q.q8_0_argmax(to_dev(v))
    assert int(host(out)[0]) == int(np.argmax(v)) == oracle.argmax(v)


def test_argmax_ties_and_specials():
    g = np.random.default_rng(7)
    v = g.standard_normal(151936).astype(np.float32)
    m = np.float32(v.max() + 1)
    for idx in ([151935, 7, 80000], [3, 2, 1], [0, 151935]):
        w = v.copy()
        w[idx] = m
        assert int(host(q.q8_0_argmax(to_dev(w)))[0]) == min(idx)
    w = np.full(100000, -3.0, dtype=np.float32)
    assert int(host(q.q8_0_argmax(to_dev(w)))[0]) == 0
    w = np.full(5000, -np.inf, dtype=np.float32)
    w[4321] = -1e30
    assert int(host(q.q8_0_argmax(to_dev(w)))[0]) == 4321
    w = np.zeros(777, dtype=np.float32)
    w[10] = -0.0
    w[5] = 0.0
    assert int(host(q.q8_0_argmax(to_dev(w)))[0]) == 0


def test_argmax_repeatable():
    v = to_dev(np.random.default_rng(8).standard_normal(151936).astype(np.float32))
    first = int(host(q.q8_0_argmax(v))[0])
    for _ in range(30):
        assert int(host(q.q8_0_argmax(v))[0]) == first


@pytest.mark.parametrize("M,K", [(151936, 896), (1000, 64), (64, 96), (130, 4864)])
def test_fused_lm_head_argmax(M, K):
    """Argmax epilogue: bit-exact against numpy on the GPU's own logits, and
    the logits within tolerance of the oracle on sampled rows (plus the
    picked row and the ends)."""
    g = W.rng(30, M, K)
    m = W.draw_matrix(g, M, K)
    x = W.draw_x(g, 1, K)[0]
    p = pack(m)
    y = torch.empty(M, dtype=torch.float32, device=DEV)
    am = torch.zeros(1, dtype=torch.int32, device=DEV)
    f = q.make_fusion(epilogue=q.Q8_EPI_ARGMAX, argmax_out=am)
    q.q8_0_gemv_fused(p, to_dev(x), y, f)
    yg = host(y)
    pick = int(host(am)[0])
    assert pick == int(np.argmax(yg))
    rows = np.unique(np.concatenate([np.random.default_rng(1).integers(0, M, 2000),
                                     [0, M - 1, pick]]))
    yr, S = oracle.gemv(m.aos()[rows], x)
    q8tol.check(yg[rows], yr, S, "lm_head logits")
    # planted tie: two identical rows give identical logits; the lower wins
    if M >= 1000:
        m2 = W.Q8Matrix(m.qs.copy(), m.d.copy())
        other = (pick + M // 2) % M
        a, b = min(pick, other), max(pick, other)
        m2.qs[a] = m2.qs[b] = m.qs[pick]
        m2.d[a] = m2.d[b] = m.d[pick]
        q.q8_0_gemv_fused(pack(m2), to_dev(x), y, f)
        yg2 = host(y)
        assert yg2[a] == yg2[b]
        assert int(host(am)[0]) == int(np.argmax(yg2)) == a


def test_router_matches_oracle():
    E, k = 60, 4
    for t in range(200):
        lg = W.router_logits(5, t, E)
        if t % 7 == 0:
            lg[np.random.default_rng(t).integers(0, E, 5)] = lg.max()
        ids, w = q.q8_0_route_topk(to_dev(lg), k)
        ids_r, w_r = oracle.route_topk(lg, k)
        assert np.array_equal(host(ids), ids_r), t
        assert np.all(np.abs(host(w).astype(np.float64) - w_r) <= 1e-6), t


@pytest.mark.parametrize("E,k", [(1, 1), (8, 8), (60, 1), (64, 4), (65, 4), (1024, 8), (300, 6)])
def test_router_shapes(E, k):
    g = np.random.default_rng(E * 10 + k)
    lg = g.standard_normal(E).astype(np.float32)
    ids, w = q.q8_0_route_topk(to_dev(lg), k)
    ids_r, w_r = oracle.route_topk(lg, k)
    assert np.array_equal(host(ids), ids_r)
    assert np.all(np.abs(host(w).astype(np.float64) - w_r) <= 1e-6)
    lg = np.zeros(E, dtype=np.float32)
    ids, w = q.q8_0_route_topk(to_dev(lg), k)
    assert list(host(ids)) == list(range(k))
    assert np.allclose(host(w), 1.0 / k, rtol=0, atol=1e-7)
