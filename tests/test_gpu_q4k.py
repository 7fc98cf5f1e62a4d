"""GPU parity of the Q4_K weights (NEXT-2): the repack layout bit-exact, the
GEMV against the fp64 oracle on the same GGUF bytes.

Tolerance (derived): the kernel evaluates each 32-weight sub-block as
fl(d s) * sum(q x) - fl(dmin m) * sum(x) in fp32 (d s and dmin m are exact:
11 x 6 bits), so its rounding error is bounded by the magnitudes of both
terms, S2 = sum_k (|d s_j q_k| + |dmin m_j|) |x_k|, not by the magnitude of
the combined weight: |y_gpu - y_ref| <= 2e-5 * S2 + 1e-6, the same relative
bound the Q8_0 path uses."""
import numpy as np
import pytest
import torch

import block_quantized_gemv_amd as q
import oracle
import workloads as W
from gpu_util import DEV, host, to_dev

pytestmark = pytest.mark.gpu


def pack4(m: W.Q4KMatrix) -> q.PackedQ4K:
    return q.PackedQ4K.from_blocks(to_dev(m.blocks().reshape(-1)), m.M, m.K)


def s2_bound(m: W.Q4KMatrix, x: np.ndarray) -> np.ndarray:
    """S2[n][r] from the drawn fields (fp64)."""
    M, K = m.q.shape
    d = np.repeat(m.d.astype(np.float64), 256, axis=1)
    dmin = np.repeat(m.dmin.astype(np.float64), 256, axis=1)
    s = np.repeat(m.s.astype(np.float64), 32, axis=1)
    mm = np.repeat(m.m.astype(np.float64), 32, axis=1)
    a = np.abs(d * s * m.q) + np.abs(dmin * mm)
    return np.abs(x.astype(np.float64)) @ a.T


def check(y, yr, S2, what):
    err = np.abs(np.asarray(y, np.float64) - yr)
    bad = np.argwhere(~(err <= 2e-5 * S2 + 1e-6))
    assert bad.size == 0, f"{what}: {bad.shape[0]} outputs out of tolerance, first {tuple(bad[0])}"


def expected_layout(m: W.Q4KMatrix):
    """The packed layout written out from its definition (q8gemv.h): qs byte b
    of sub-block c of row r = q[r, 32c + b] | q[r, 32c + 16 + b] << 4; meta =
    the block's first 16 GGUF bytes; rows padded to 64 with zeros."""
    M, K = m.q.shape
    T = (M + 63) // 64
    qpad = np.zeros((T * 64, K), np.uint8)
    qpad[:M] = m.q
    sub = qpad.reshape(T, 64, K // 32, 32)
    qs = (sub[..., :16] | (sub[..., 16:] << 4)).transpose(0, 2, 1, 3)  # [T][K/32][64][16]
    hdr = np.zeros((T * 64, K // 256, 16), np.uint8)
    hdr[:M] = m.blocks()[:, :, :16]
    meta = hdr.reshape(T, 64, K // 256, 16).transpose(0, 2, 1, 3)
    return np.ascontiguousarray(qs).reshape(-1), np.ascontiguousarray(meta).reshape(-1)


@pytest.mark.parametrize("M,K", [(1, 256), (64, 512), (65, 256), (130, 1024), (300, 4864)])
def test_q4k_repack_layout_bit_exact(M, K):
    m = W.draw_q4k(W.rng(80, M, K), M, K)
    p = pack4(m)
    eq, em = expected_layout(m)
    assert np.array_equal(host(p.qs), eq)
    assert np.array_equal(host(p.meta), em)


SHAPES = [(1, 256), (64, 256), (65, 512), (130, 1024), (300, 2048), (64, 4096), (200, 4864),
          (1000, 1024)]


@pytest.mark.parametrize("M,K", SHAPES)
@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 6, 7, 8])
def test_q4k_gemv_matches_oracle(M, K, N):
    g = W.rng(81, M * 7 + N, K)
    m = W.draw_q4k(g, M, K)
    x = W.draw_x(g, N, K)
    y = host(q.q4k_gemv(pack4(m), to_dev(x)))
    yr, _ = oracle.q4k_gemv(m.blocks(), x)
    check(y, yr, s2_bound(m, x), f"q4k {M}x{K} N={N}")


def test_q4k_one_hot_exact():
    """x = e_k gives the fp32 rounding of weight k exactly (d s q exact, one
    rounding for the min term), at positions in every sub-block of a block."""
    M, K = 130, 1024
    m = W.draw_q4k(W.rng(82), M, K)
    m.q[0, :] = 15
    m.s[1, :], m.m[1, :] = 63, 63
    m.s[2, :], m.m[2, :] = 0, 0
    p = pack4(m)
    ks = [0, 15, 16, 31, 32, 63, 64, 100, 200, 255, 256, 511, 700, 1023]
    deq = oracle.q4k_dequant_rows(m.blocks(), K)
    for i in range(0, len(ks), 4):
        sel = ks[i:i + 4]
        x = np.zeros((len(sel), K), np.float32)
        for j, k in enumerate(sel):
            x[j, k] = 1.0
        y = host(q.q4k_gemv(p, to_dev(x)))
        for j, k in enumerate(sel):
            assert np.array_equal(y[j], deq[:, k].astype(np.float32)), k


def test_q4k_repeated_calls_bitwise_identical():
    m = W.draw_q4k(W.rng(83), 4096, 4096)
    x = to_dev(W.draw_x(W.rng(84), 2, 4096))
    p = pack4(m)
    a = host(q.q4k_gemv(p, x))
    for _ in range(3):
        assert np.array_equal(host(q.q4k_gemv(p, x)), a)


def test_q4k_rejects_bad_arguments():
    m = W.draw_q4k(W.rng(85), 64, 256)
    p = pack4(m)
    x = torch.zeros((1, 256), device=DEV)
    y = torch.zeros((1, 64), device=DEV)
    bad = q.PackedQ4K(p.qs[4:], p.meta, 64, 256)  # nibbles not 16-byte aligned
    with pytest.raises(q.Q8Error):
        q.q4k_gemv(bad, x)
    rc = q.lib().q4k_gemv(q.ctypes.byref(p.desc), x.cpu().data_ptr(), y.data_ptr(), 64, 256, 1,
                          None, 0, None)
    assert rc == q.Q8_EHOSTPTR
