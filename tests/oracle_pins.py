"""Pins for the fp64 CPU oracle.

Each check ties the oracle to something other than itself: the IEEE binary16
definition, closed forms of the Q8_0 dot product, exact rational brute force,
an independent dense fp64 matrix-vector product (numpy), invariants of the
definition, and library routines (numpy argmax / stable argsort / repeat,
scipy expit).  The checks are plain functions so that the mutation test can
re-run them against deliberately broken builds of the oracle.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
from scipy.special import expit

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# fp64 summation bound for the oracle's ascending loop against any other
# fp64 summation order: |err| <= 2 * K * 2^-53 * S (both sides); use a loose
# multiple that still catches any dropped or wrong term.
def fp64_tol(K, S):
    return 4.0 * K * 2.0 ** -53 * S + 1e-300


def _np_dequant(m: W.Q8Matrix) -> np.ndarray:
    """Independent dequantisation: numpy's binary16 conversion times int8."""
    d = m.d.astype(np.float64)
    return (m.qs.astype(np.float64).reshape(m.M, -1, 32) * d[:, :, None]).reshape(m.M, m.K)


def _mat_from(qs, d) -> W.Q8Matrix:
    return W.Q8Matrix(np.asarray(qs, dtype=np.int8), np.asarray(d, dtype=np.float16))


# ---------------------------------------------------------------------------
# binary16 decoder
# ---------------------------------------------------------------------------
def check_f16_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan_ref), "NaN classification differs"
    ok = ~nan_ref
    assert np.array_equal(ours[ok], ref[ok]), "binary16 decode differs from numpy"
    # signed zero must keep its sign
    assert math.copysign(1.0, ours[0x8000]) == -1.0


def check_f16_golden():
    path = os.path.join(GOLDEN, "f16_reference_values.txt")
    n = 0
    for line in open(path):
        line = line.split("#")[0].strip()
        if not line:
            continue
        hexbits, val = line.split()
        b = int(hexbits, 16)
        got = oracle.f16_to_f64(np.array([b], dtype=np.uint16))[0]
        if val in ("inf", "-inf"):
            assert got == float(val), (hexbits, got)
        else:
            assert Fraction(got) == Fraction(val), (hexbits, got, val)
            if val.startswith("-"):
                assert math.copysign(1.0, got) == -1.0
        n += 1
    assert n >= 15


# ---------------------------------------------------------------------------
# GEMV closed forms and exact cases
# ---------------------------------------------------------------------------
def check_hand_examples():
    path = os.path.join(GOLDEN, "q8_0_hand_examples.txt")
    n = 0
    j = np.arange(32)
    for line in open(path):
        line = line.split("#")[0].strip()
        if not line:
            continue
        dbits, qp, xp, yexact = line.split()
        if qp == "j-16":
            q = j - 16
        else:
            q = np.full(32, int(qp.split(":")[1]))
        x = {"ones": np.ones(32), "j": j.astype(np.float64), "alt": (-1.0) ** j}[xp]
        d = np.array([[int(dbits, 16)]], dtype=np.uint16).view(np.float16)
        m = _mat_from(q.reshape(1, 32), d)
        y, _ = oracle.gemv(m.aos(), x.astype(np.float32))
        assert Fraction(float(y[0])) == Fraction(yexact), (line, y[0])
        n += 1
    assert n >= 6


def check_closed_form_constant():
    """All quants equal q, all scales d: y = d * q * sum(x).  With small
    integer x every partial sum is an exact integer, so equality is exact."""
    g = np.random.default_rng(11)
    for (M, K) in [(3, 32), (5, 896), (2, 4864), (4, 12288)]:
        x = g.integers(-1, 2, size=(2, K)).astype(np.float32)
        for q in (-128, -127, -1, 0, 1, 77, 127):
            for dbits in (0x3C00, 0x3800, 0x2000, 0x0001, 0xC400):
                d = np.array([dbits], dtype=np.uint16).view(np.float16)[0]
                m = _mat_from(np.full((M, K), q), np.full((M, K // 32), d))
                y, S = oracle.gemv(m.aos(), x)
                want = float(d) * q * x.astype(np.float64).sum(axis=1)
                assert np.array_equal(y, np.repeat(want[:, None], M, axis=1)), (M, K, q, dbits)
                assert np.array_equal(S, np.repeat((abs(float(d) * q) *
                                                    np.abs(x).astype(np.float64).sum(axis=1))[:, None],
                                                   M, axis=1))


def check_one_hot():
    """x = e_k selects column k of the dequantised matrix: y[r] = d[r, k/32] *
    q[r, k], exactly."""
    g = np.random.default_rng(12)
    M, K = 7, 1408
    m = W.draw_matrix(g, M, K)
    aos = m.aos()
    for k in [0, 1, 15, 16, 31, 32, 33, 63, 64, 700, K - 33, K - 32, K - 1]:
        x = np.zeros(K, dtype=np.float32)
        x[k] = 1.0
        y, _ = oracle.gemv(aos, x)
        want = m.d[:, k // 32].astype(np.float64) * m.qs[:, k].astype(np.float64)
        assert np.array_equal(y, want), k
        x[k] = -3.0
        y, _ = oracle.gemv(aos, x)
        assert np.array_equal(y, -3.0 * want), k


def check_bruteforce_k32():
    """K = 32: exact rational arithmetic over every quant value and edge
    scales; the fp64 oracle must sit within 32 ulps of the exact sum."""
    g = np.random.default_rng(13)
    qvals = np.arange(-128, 128)
    edge_bits = [0x0000, 0x8000, 0x0001, 0x03FF, 0x0400, 0x3C00, 0xBC00, 0x7BFF, 0xFBFF,
                 0x2E66, 0x1234]
    rows = []
    dbits = []
    for i in range(0, 256, 32):
        for b in edge_bits:
            rows.append(qvals[i:i + 32])
            dbits.append(b)
    for _ in range(40):
        rows.append(g.integers(-128, 128, size=32))
        dbits.append(int(g.integers(0, 0x7C00)) | (int(g.integers(0, 2)) << 15))
    qs = np.array(rows)
    d = np.array(dbits, dtype=np.uint16).view(np.float16).reshape(-1, 1)
    m = _mat_from(qs, d)
    x = g.standard_normal((3, 32)).astype(np.float32)
    x[1] = (g.integers(-50, 50, size=32) * 0.5).astype(np.float32)
    y, S = oracle.gemv(m.aos(), x)
    for n in range(x.shape[0]):
        xf = [Fraction(float(v)) for v in x[n]]
        for r in range(qs.shape[0]):
            dr = Fraction(float(d[r, 0]))
            exact = sum(dr * int(qs[r, j]) * xf[j] for j in range(32))
            sabs = sum(abs(dr * int(qs[r, j]) * xf[j]) for j in range(32))
            err = abs(Fraction(float(y[n, r])) - exact)
            assert err <= Fraction(32 * 2.0 ** -53) * sabs, (n, r)
            assert abs(Fraction(float(S[n, r])) - sabs) <= Fraction(32 * 2.0 ** -53) * sabs


def check_dense_matvec_shapes():
    """The definition is a dense matrix-vector product of the dequantised
    matrix: numpy fp64 matmul (BLAS) must agree at every workload shape (row
    samples of the tall ones)."""
    shapes = [(896, 896, 1), (1152, 896, 1), (9728, 896, 1), (896, 4864, 1),
              (2816, 2048, 1), (2048, 1408, 1), (256, 4096, 2), (128, 12288, 8),
              (11264, 2048, 1), (2048, 5632, 1), (600, 896, 1)]
    for i, (M, K, N) in enumerate(shapes):
        g = W.rng(900 + i)
        Mi = min(M, 384)
        m = W.draw_matrix(g, Mi, K)
        x = W.draw_x(g, N, K)
        y, S = oracle.gemv(m.aos(), x)
        Wd = _np_dequant(m)
        ref = x.astype(np.float64) @ Wd.T
        Sref = np.abs(x.astype(np.float64)) @ np.abs(Wd).T
        assert np.all(np.abs(y - ref) <= fp64_tol(K, Sref)), (M, K, N)
        assert np.allclose(S, Sref, rtol=1e-12, atol=0), (M, K, N)


def check_invariants():
    g = W.rng(950)
    M, K = 40, 1408
    m = W.draw_matrix(g, M, K)
    aos = m.aos()
    # linearity with exactly representable sums (multiples of 1/8 below 2^10)
    x1 = (g.integers(-512, 512, size=K) / 8.0).astype(np.float32)
    x2 = (g.integers(-512, 512, size=K) / 8.0).astype(np.float32)
    y1, S1 = oracle.gemv(aos, x1)
    y2, S2 = oracle.gemv(aos, x2)
    y12, _ = oracle.gemv(aos, (x1 + x2).astype(np.float32))
    assert np.all(np.abs(y12 - (y1 + y2)) <= fp64_tol(K, S1 + S2))
    y3, _ = oracle.gemv(aos, (3 * x1).astype(np.float32))
    assert np.all(np.abs(y3 - 3 * y1) <= fp64_tol(K, 3 * S1))
    # row permutation -> output permutation (bitwise)
    perm = g.permutation(M)
    yp, _ = oracle.gemv(m.aos()[perm], x1)
    assert np.array_equal(yp, y1[perm])
    # joint permutation of blocks and the matching x segments
    bperm = g.permutation(K // 32)
    qs_b = m.qs.reshape(M, -1, 32)[:, bperm].reshape(M, K)
    d_b = m.d[:, bperm]
    xb = x1.reshape(-1, 32)[bperm].reshape(K)
    yb, _ = oracle.gemv(_mat_from(qs_b, d_b).aos(), xb)
    assert np.all(np.abs(yb - y1) <= fp64_tol(K, S1))
    # doubling every scale doubles y exactly (finite scales stay finite)
    d2 = (m.d.astype(np.float32) * 2).astype(np.float16)
    assert np.all(np.isfinite(d2))
    y2d, _ = oracle.gemv(_mat_from(m.qs, d2).aos(), x1)
    assert np.array_equal(y2d, 2 * y1)
    # negating the quants (except -128) negates y exactly
    qn = np.where(m.qs == -128, 0, m.qs)
    ya, _ = oracle.gemv(_mat_from(qn, m.d).aos(), x1)
    yb2, _ = oracle.gemv(_mat_from(-qn, m.d).aos(), x1)
    assert np.array_equal(ya, -yb2)
    # stacked rows: [gate; up] gives gate rows then up rows
    gate = W.draw_matrix(g, 16, K)
    up = W.draw_matrix(g, 16, K)
    both = np.concatenate([gate.aos(), up.aos()], axis=0)
    yg, _ = oracle.gemv(gate.aos(), x1)
    yu, _ = oracle.gemv(up.aos(), x1)
    yb3, _ = oracle.gemv(both, x1)
    assert np.array_equal(yb3, np.concatenate([yg, yu]))


def check_columns_independent():
    """N activation columns give exactly the N single-column results."""
    g = W.rng(951)
    m = W.draw_matrix(g, 33, 4096)
    x = W.draw_x(g, 8, 4096)
    y, S = oracle.gemv(m.aos(), x)
    for n in range(8):
        yn, Sn = oracle.gemv(m.aos(), x[n])
        assert np.array_equal(y[n], yn) and np.array_equal(S[n], Sn)


def check_threads_identical():
    g = W.rng(952)
    m = W.draw_matrix(g, 257, 896)
    x = W.draw_x(g, 2, 896)
    y1, _ = oracle.gemv(m.aos(), x, threads=1)
    y7, _ = oracle.gemv(m.aos(), x, threads=7)
    assert np.array_equal(y1, y7)


# ---------------------------------------------------------------------------
# argmax, router, glue
# ---------------------------------------------------------------------------
def check_argmax():
    g = np.random.default_rng(14)
    for n in [1, 2, 7, 1000, 151936]:
        v = g.standard_normal(n).astype(np.float32)
        assert oracle.argmax(v) == int(np.argmax(v))
        assert oracle.argmax(v.astype(np.float64)) == int(np.argmax(v))
    v = np.zeros(100, dtype=np.float32)
    v[[17, 40, 99]] = 5.0
    assert oracle.argmax(v) == 17
    v = np.full(64, -1.0, dtype=np.float32)
    assert oracle.argmax(v) == 0
    v = np.array([-0.0, 0.0, -1.0], dtype=np.float32)
    assert oracle.argmax(v) == 0
    v = np.array([-np.inf, -3.0, -np.inf], dtype=np.float32)
    assert oracle.argmax(v) == 1
    v = g.standard_normal(5000).astype(np.float32)
    v[4999] = v.max()
    assert oracle.argmax(v) == int(np.argmax(v)) != 4999


def check_router():
    g = np.random.default_rng(15)
    for t in range(50):
        E, k = 60, 4
        lg = g.standard_normal(E).astype(np.float32)
        if t % 5 == 0:
            lg[g.integers(0, E, 6)] = lg.max()  # planted ties at the top
        ids, w = oracle.route_topk(lg, k)
        want = np.argsort(-lg.astype(np.float64), kind="stable")[:k]
        assert np.array_equal(ids, want), (t, ids, want)
        p = np.exp(lg.astype(np.float64) - lg.max())
        p /= p.sum()  # softmax over all experts
        ref = p[want] / p[want].sum()  # renormalised over the selected ones
        assert np.allclose(w, ref, rtol=1e-14, atol=0)
        assert abs(w.sum() - 1.0) < 1e-15
        assert np.all(np.diff(w) <= 0)
    ids, w = oracle.route_topk(np.zeros(60, dtype=np.float32), 4)
    assert list(ids) == [0, 1, 2, 3] and np.all(w == 0.25)
    ids, w = oracle.route_topk(np.array([0, 0, 9, 0], dtype=np.float32), 1)
    assert list(ids) == [2] and w[0] == 1.0


def check_glue():
    zs = np.linspace(-30, 30, 121)
    for z in zs:
        s = oracle.sigmoid(z)
        assert abs(s - expit(z)) <= 1e-15 * max(1.0, abs(expit(z)))
        # silu(z) - silu(-z) = z  and  silu(z) = z * sigmoid(z)
        assert abs((oracle.silu(z) - oracle.silu(-z)) - z) <= 1e-13 * max(1.0, abs(z))
        assert abs(oracle.silu(z) - z * expit(z)) <= 1e-14 * max(1.0, abs(z))
    assert oracle.silu(0.0) == 0.0 and oracle.sigmoid(0.0) == 0.5
    g = np.random.default_rng(16)
    a = g.standard_normal(100)
    b = g.standard_normal(100)
    assert np.allclose(oracle.swiglu(a, b), a * expit(a) * b, rtol=1e-14, atol=1e-300)
    # rmsnorm: constant vector c -> c / sqrt(c^2 + eps); scale invariance at eps = 0;
    # unit mean square at eps = 0.
    c, eps = 3.0, 1e-6
    out = oracle.rmsnorm(np.full(896, c), eps)
    assert np.allclose(out, c / math.sqrt(c * c + eps), rtol=1e-15)
    x = g.standard_normal(896)
    r0 = oracle.rmsnorm(x, 0.0)
    assert abs(np.mean(r0 ** 2) - 1.0) < 1e-14
    assert np.allclose(oracle.rmsnorm(7.5 * x, 0.0), r0, rtol=1e-14)
    # GQA at position 0: query head h takes kv head h // group (numpy repeat)
    v = g.standard_normal((2, 64))
    out = oracle.gqa_position0(v.ravel(), 14, 2, 64)
    assert np.array_equal(out.reshape(14, 64), np.repeat(v, 7, axis=0))


# ---------------------------------------------------------------------------
# Mixture of experts and the decoder layer (composites)
# ---------------------------------------------------------------------------
def _np_swiglu(gu):
    I = gu.size // 2
    return gu[:I] * expit(gu[:I]) * gu[I:]


def check_moe():
    g = W.rng(960)
    E, H, I, Ish = 6, 256, 96, 160
    gu = [W.draw_matrix(g, 2 * I, H) for _ in range(E)]
    dn = [W.draw_matrix(g, H, I) for _ in range(E)]
    sgu = W.draw_matrix(g, 2 * Ish, H)
    sdn = W.draw_matrix(g, H, Ish)
    gu_stack = np.stack([m.aos() for m in gu])
    dn_stack = np.stack([m.aos() for m in dn])
    x = W.draw_x(g, 1, H)[0]
    lg = g.standard_normal(E).astype(np.float32)
    ids, w = oracle.route_topk(lg, 4)
    lam = 0.3
    gamma = float(expit(lam))
    y = oracle.moe_ffn(gu_stack, dn_stack, ids, w, sgu.aos(), sdn.aos(), gamma, x)
    # independent composition with numpy dense algebra
    xd = x.astype(np.float64)
    ref = np.zeros(H)
    for s, e in enumerate(ids):
        h = _np_swiglu(_np_dequant(gu[e]) @ xd)
        ref += w[s] * (_np_dequant(dn[e]) @ h)
    hs = _np_swiglu(_np_dequant(sgu) @ xd)
    ref += gamma * (_np_dequant(sdn) @ hs)
    assert np.allclose(y, ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())
    # one-hot routing weight and no shared gate -> one dense FFN
    w1 = np.array([1.0, 0.0, 0.0, 0.0])
    y1 = oracle.moe_ffn(gu_stack, dn_stack, ids, w1, sgu.aos(), sdn.aos(), 0.0, x)
    e0 = ids[0]
    ref1 = _np_dequant(dn[e0]) @ _np_swiglu(_np_dequant(gu[e0]) @ xd)
    assert np.allclose(y1, ref1, rtol=1e-10, atol=1e-12 * np.abs(ref1).max())
    # slots folded in order: permuting (ids, w) jointly changes nothing beyond
    # rounding; the combine stage equals the stage-wise composition.
    hr = np.stack([_np_swiglu(_np_dequant(gu[e]) @ xd) for e in ids])
    yc, Sabs = oracle.moe_combine(dn_stack, ids, w, hr, sdn.aos(), hs, gamma)
    assert np.allclose(yc, ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())
    sref = sum(abs(w[s]) * (np.abs(_np_dequant(dn[e])) @ np.abs(hr[s])) for s, e in enumerate(ids))
    sref = sref + abs(gamma) * (np.abs(_np_dequant(sdn)) @ np.abs(hs))
    assert np.allclose(Sabs, sref, rtol=1e-12)


def check_qwen_layer():
    g = W.rng(970)
    hidden, nh, nkv, hd, inter = 128, 4, 2, 32, 160
    qkv = W.draw_matrix(g, hidden + 2 * nkv * hd, hidden)
    wo = W.draw_matrix(g, hidden, hidden)
    gu = W.draw_matrix(g, 2 * inter, hidden)
    dn = W.draw_matrix(g, hidden, inter)
    h = W.draw_x(g, 1, hidden)[0].astype(np.float64)
    eps = 1e-6
    out = oracle.qwen_layer(qkv.aos(), wo.aos(), gu.aos(), dn.aos(), h, nh, nkv, hd, eps)

    def rms(v):
        return v / np.sqrt(np.mean(v * v) + eps)

    a = rms(h)
    t = _np_dequant(qkv) @ a
    v = t[hidden + nkv * hd:].reshape(nkv, hd)
    att = np.repeat(v, nh // nkv, axis=0).ravel()
    h1 = h + _np_dequant(wo) @ att
    s = _np_swiglu(_np_dequant(gu) @ rms(h1))
    ref = h1 + _np_dequant(dn) @ s
    assert np.allclose(out, ref, rtol=1e-11, atol=1e-11 * np.abs(ref).max())


# ---- integer-activation variant (opt-in path) ---------------------------------
def check_f32_to_f16_numpy():
    """The oracle's binary16 encoder against numpy's fp32 -> fp16 conversion
    (round to nearest even) over all exponent ranges, subnormals, ties and the
    overflow threshold."""
    g = np.random.default_rng(40)
    vals = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 7e4, 2.0 ** -24, 2.0 ** -25,
            3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11,
            2049.0, 2051.0]
    vals += list(g.standard_normal(3000) * np.exp2(g.integers(-30, 17, 3000)))
    for v in vals:
        f = np.float32(v)
        want = int(np.array([f], dtype=np.float32).astype(np.float16).view(np.uint16)[0])
        assert oracle.f32_to_f16(f) == want, (v, oracle.f32_to_f16(f), want)


def check_quantize_act_closed_forms():
    """Quantizer: constant blocks map to +-127 with scale |c|/127; integer
    grids k * 2^e with max |k| = 127 are reproduced exactly (scale 2^e);
    halves round to even; a zero block gives zeros; negation flips the codes;
    every code is the nearest integer to x / d."""
    f16 = lambda a: np.asarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)
    for c in (1.0, -3.25, 1e-3, 250.0):
        q, d = oracle.quantize_act(np.full((1, 32), c, np.float32))
        assert np.all(q == 127 * np.sign(c)), c
        assert d[0, 0] == f16(np.float32(abs(c)) / np.float32(127))[()], c
    g = np.random.default_rng(41)
    for e in (-12, -3, 0, 5, 9):
        k = g.integers(-127, 128, (3, 64))
        k[:, 0], k[:, 32] = 127, -127
        x = (k * 2.0 ** e).astype(np.float32)
        q, d = oracle.quantize_act(x)
        assert np.array_equal(q, k), e
        assert np.all(d == f16(2.0 ** e)[()]), e
    x = np.array([[127, 2.5, 3.5, -2.5, 0.5, -0.5, 1.5, -3.5] + [0] * 24], np.float32) * 0.25
    q, _ = oracle.quantize_act(x)
    assert list(q[0, :8]) == [127, 2, 4, -2, 0, 0, 2, -4]
    q, d = oracle.quantize_act(np.zeros((1, 32), np.float32))
    assert not q.any() and d[0, 0] == 0
    x = (g.standard_normal((4, 96)) * 3).astype(np.float32)
    q, d = oracle.quantize_act(x)
    qn, dn = oracle.quantize_act(-x)
    assert np.array_equal(qn, -q) and np.array_equal(dn, d)
    dd = (np.float32(1) * np.abs(x).reshape(4, 3, 32).max(axis=2) / np.float32(127))
    r = x.reshape(4, 3, 32).astype(np.float64) / dd[..., None].astype(np.float64)
    assert np.all(np.abs(q.reshape(4, 3, 32) - r) <= 0.5 + 1e-5)
    assert np.abs(q).max() <= 127


def check_gemv_q8act():
    """The integer-activation product equals (a) exact rational brute force at
    small sizes and (b) the pinned fp32-path oracle applied to the dequantized
    activations dx * qx (exact in fp32), at several shapes."""
    g = np.random.default_rng(42)
    m = W.draw_matrix(g, 5, 64)
    x = W.draw_x(g, 2, 64)
    qx, dx = oracle.quantize_act(x)
    y, S = oracle.gemv_q8act(m.aos(), qx, dx)
    dxf = [[Fraction(float(v)) for v in row] for row in dx.view(np.float16).astype(np.float64)]
    for n in range(2):
        for r in range(5):
            tot = Fraction(0)
            for b in range(2):
                isum = sum(int(m.qs[r, 32 * b + j]) * int(qx[n, 32 * b + j]) for j in range(32))
                tot += Fraction(float(m.d[r, b])) * dxf[n][b] * isum
            assert abs(float(tot) - y[n, r]) <= 4 * 2.0 ** -53 * S[n, r] + 1e-300, (n, r)
    for (M, K, N) in [(7, 96, 1), (64, 896, 3), (33, 1408, 2)]:
        m = W.draw_matrix(g, M, K)
        x = W.draw_x(g, N, K)
        qx, dx = oracle.quantize_act(x)
        y, S = oracle.gemv_q8act(m.aos(), qx, dx)
        xd = (qx.astype(np.float32).reshape(N, -1, 32) *
              dx.view(np.float16).astype(np.float32)[:, :, None]).reshape(N, K)
        yr, Sr = oracle.gemv(m.aos(), xd)
        assert np.all(np.abs(y - yr) <= fp64_tol(K, Sr)), (M, K, N)


def q4k_weights_from_fields(mtx: W.Q4KMatrix) -> list:
    """Exact rational weights d * s * q - dmin * m from the drawn fields (never
    from the packed bytes)."""
    M, K = mtx.q.shape
    rows = []
    for r in range(M):
        row = []
        for k in range(K):
            d = Fraction(float(mtx.d[r, k // 256]))
            dmin = Fraction(float(mtx.dmin[r, k // 256]))
            row.append(d * int(mtx.s[r, k // 32]) * int(mtx.q[r, k])
                       - dmin * int(mtx.m[r, k // 32]))
        rows.append(row)
    return rows


def check_q4k_bruteforce():
    """Q4_K oracle against exact rational arithmetic on the drawn fields: the
    packed bytes are decoded only by the oracle, so a wrong scale/min unpack,
    nibble position, sub-block index or sign fails here."""
    g = np.random.default_rng(50)
    mtx = W.draw_q4k(g, 3, 512)
    # extremes of every field in some sub-blocks
    mtx.s[0, :4], mtx.m[0, :4] = [0, 63, 1, 62], [63, 0, 62, 1]
    mtx.s[1, 8:16], mtx.m[1, 8:16] = 63, 63
    mtx.q[2, :64] = 15
    x = W.draw_x(g, 2, 512)
    y, S = oracle.q4k_gemv(mtx.blocks(), x)
    wq = q4k_weights_from_fields(mtx)
    for n in range(2):
        for r in range(3):
            tot = sum((w * Fraction(float(xv)) for w, xv in zip(wq[r], x[n])), Fraction(0))
            mag = sum((abs(w * Fraction(float(xv))) for w, xv in zip(wq[r], x[n])), Fraction(0))
            assert abs(float(tot) - y[n, r]) <= 512 * 2.0 ** -52 * float(mag) + 1e-300, (n, r)
            assert abs(float(mag) - S[n, r]) <= 512 * 2.0 ** -52 * float(mag), (n, r)


def check_q4k_one_hot_every_position():
    """x = e_k returns weight k exactly for every k of two blocks, with every
    sub-block given a distinct (scale, min) pair."""
    g = np.random.default_rng(51)
    mtx = W.draw_q4k(g, 2, 512)
    mtx.s[:] = np.arange(16)[None, :] * 4 + 1
    mtx.m[:] = 62 - np.arange(16)[None, :] * 3
    mtx.q[:] = (np.arange(512)[None, :] * 7 + np.array([[0], [5]])) % 16
    wq = q4k_weights_from_fields(mtx)
    deq = oracle.q4k_dequant_rows(mtx.blocks(), 512)
    for r in range(2):
        assert [float(w) for w in wq[r]] == list(deq[r]), r
    x = np.eye(512, dtype=np.float32)[[0, 31, 32, 63, 64, 200, 255, 256, 300, 511]]
    y, _ = oracle.q4k_gemv(mtx.blocks(), x)
    for i, k in enumerate([0, 31, 32, 63, 64, 200, 255, 256, 300, 511]):
        assert y[i, 0] == float(wq[0][k]) and y[i, 1] == float(wq[1][k]), k


def check_q4k_closed_form_constant():
    """Constant fields: every weight is d * s * q - dmin * m, so
    y = (d s q - dmin m) * sum(x), exact with power-of-two d and dmin."""
    K = 768
    for (qv, sv, mv) in [(15, 63, 0), (0, 0, 63), (7, 33, 21), (1, 1, 1)]:
        mtx = W.Q4KMatrix(np.full((2, K), qv, np.uint8), np.full((2, K // 32), sv, np.uint8),
                          np.full((2, K // 32), mv, np.uint8),
                          np.full((2, K // 256), np.float16(0.25)),
                          np.full((2, K // 256), np.float16(0.5)))
        x = np.random.default_rng(qv).integers(-3, 4, size=(1, K)).astype(np.float32)
        y, _ = oracle.q4k_gemv(mtx.blocks(), x)
        want = (0.25 * sv * qv - 0.5 * mv) * float(x.astype(np.float64).sum())
        assert np.all(y == want), (qv, sv, mv)


def q6k_weights_from_fields(mtx: W.Q6KMatrix) -> list:
    """Exact rational weights d * scale * (code - 32) from the drawn fields."""
    M, K = mtx.code.shape
    return [[Fraction(float(mtx.d[r, k // 256])) * int(mtx.sc[r, k // 16]) *
             (int(mtx.code[r, k]) - 32) for k in range(K)] for r in range(M)]


def check_q6k_bruteforce():
    """Q6_K oracle against exact rational arithmetic on the drawn fields (the
    packed bytes are decoded only by the oracle)."""
    g = np.random.default_rng(60)
    mtx = W.draw_q6k(g, 3, 512)
    mtx.code[0, :64], mtx.code[1, 100:200] = 63, 0
    mtx.sc[2, :8] = [-128, 127, -1, 0, 1, -64, 64, 100]
    x = W.draw_x(g, 2, 512)
    y, S = oracle.q6k_gemv(mtx.blocks(), x)
    wq = q6k_weights_from_fields(mtx)
    for n in range(2):
        for r in range(3):
            terms = [w * Fraction(float(xv)) for w, xv in zip(wq[r], x[n])]
            tot, mag = sum(terms, Fraction(0)), sum((abs(t) for t in terms), Fraction(0))
            assert abs(float(tot) - y[n, r]) <= 512 * 2.0 ** -52 * float(mag) + 1e-300, (n, r)
            assert abs(float(mag) - S[n, r]) <= 512 * 2.0 ** -52 * float(mag), (n, r)


def check_q6k_one_hot_every_position():
    """Every weight of two blocks dequantises to d * scale * (code - 32), each
    16-weight group with its own scale; one-hot x returns it exactly."""
    g = np.random.default_rng(61)
    mtx = W.draw_q6k(g, 2, 512)
    mtx.code[:] = (np.arange(512)[None, :] * 5 + np.array([[0], [17]])) % 64
    mtx.sc[:] = (np.arange(32)[None, :] * 7 - 100).astype(np.int8)
    wq = q6k_weights_from_fields(mtx)
    deq = oracle.q6k_dequant_rows(mtx.blocks(), 512)
    for r in range(2):
        assert [float(w) for w in wq[r]] == list(deq[r]), r
    ks = [0, 15, 16, 31, 32, 63, 64, 127, 128, 160, 200, 255, 256, 300, 450, 511]
    y, _ = oracle.q6k_gemv(mtx.blocks(), np.eye(512, dtype=np.float32)[ks])
    for i, k in enumerate(ks):
        assert y[i, 0] == float(wq[0][k]) and y[i, 1] == float(wq[1][k]), k


def check_q6k_closed_form_constant():
    """Constant code c, scale s and d: y = d s (c - 32) sum(x), exact."""
    K = 768
    for (c, sv) in [(63, 127), (0, -128), (32, 5), (40, -3)]:
        mtx = W.Q6KMatrix(np.full((2, K), c, np.uint8), np.full((2, K // 16), sv, np.int8),
                          np.full((2, K // 256), np.float16(0.125)))
        x = np.random.default_rng(c).integers(-3, 4, size=(1, K)).astype(np.float32)
        y, _ = oracle.q6k_gemv(mtx.blocks(), x)
        assert np.all(y == 0.125 * sv * (c - 32) * float(x.astype(np.float64).sum())), (c, sv)


def q5k_weights_from_fields(mtx: W.Q5KMatrix) -> list:
    M, K = mtx.code.shape
    return [[Fraction(float(mtx.d[r, k // 256])) * int(mtx.s[r, k // 32]) * int(mtx.code[r, k])
             - Fraction(float(mtx.dmin[r, k // 256])) * int(mtx.m[r, k // 32])
             for k in range(K)] for r in range(M)]


def check_q5k_bruteforce():
    """Q5_K oracle against exact rational sums on the drawn fields."""
    g = np.random.default_rng(70)
    mtx = W.draw_q5k(g, 3, 512)
    mtx.code[0, :64], mtx.code[1, 64:192] = 31, 16
    mtx.s[2, :4], mtx.m[2, :4] = [0, 63, 1, 62], [63, 0, 62, 1]
    x = W.draw_x(g, 2, 512)
    y, S = oracle.q5k_gemv(mtx.blocks(), x)
    wq = q5k_weights_from_fields(mtx)
    for n in range(2):
        for r in range(3):
            terms = [w * Fraction(float(xv)) for w, xv in zip(wq[r], x[n])]
            tot, mag = sum(terms, Fraction(0)), sum((abs(t) for t in terms), Fraction(0))
            assert abs(float(tot) - y[n, r]) <= 512 * 2.0 ** -52 * float(mag) + 1e-300, (n, r)
            assert abs(float(mag) - S[n, r]) <= 512 * 2.0 ** -52 * float(mag), (n, r)


def check_q5k_one_hot_every_position():
    """Every weight of two blocks against the fields, with distinct codes per
    position (fifth bits in every sub-block) and per-sub-block scales/mins."""
    g = np.random.default_rng(71)
    mtx = W.draw_q5k(g, 2, 512)
    mtx.code[:] = (np.arange(512)[None, :] * 11 + np.array([[0], [7]])) % 32
    mtx.s[:] = np.arange(16)[None, :] * 4 + 2
    mtx.m[:] = 60 - np.arange(16)[None, :] * 3
    wq = q5k_weights_from_fields(mtx)
    deq = oracle.q5k_dequant_rows(mtx.blocks(), 512)
    for r in range(2):
        assert [float(w) for w in wq[r]] == list(deq[r]), r
    ks = [0, 31, 32, 63, 64, 100, 200, 255, 256, 300, 511]
    y, _ = oracle.q5k_gemv(mtx.blocks(), np.eye(512, dtype=np.float32)[ks])
    for i, k in enumerate(ks):
        assert y[i, 0] == float(wq[0][k]) and y[i, 1] == float(wq[1][k]), k


ALL_CHECKS = [
    check_f16_exhaustive, check_f16_golden, check_hand_examples, check_closed_form_constant,
    check_one_hot, check_bruteforce_k32, check_dense_matvec_shapes, check_invariants,
    check_columns_independent, check_threads_identical, check_argmax, check_router,
    check_glue, check_moe, check_qwen_layer, check_f32_to_f16_numpy,
    check_quantize_act_closed_forms, check_gemv_q8act, check_q4k_bruteforce,
    check_q4k_one_hot_every_position, check_q4k_closed_form_constant, check_q6k_bruteforce,
    check_q6k_one_hot_every_position, check_q6k_closed_form_constant, check_q5k_bruteforce,
    check_q5k_one_hot_every_position,
]
