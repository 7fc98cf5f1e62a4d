"""GPU parity of the Q6_K weights (NEXT-2): the repack layout bit-exact, the
GEMV against the fp64 oracle on the same GGUF bytes.

Tolerance (derived): the kernel evaluates each 16-weight group as
fl(d s) * sum(code x) - 32 fl(d s) * sum(x) in fp32 (d s is exact: 11 x 8
bits), so its rounding error is bounded by both terms' magnitudes,
S2 = sum_k (|d s_g code_k| + 32 |d s_g|) |x_k|, not by the magnitude of the
combined weight: |y_gpu - y_ref| <= 2e-5 * S2 + 1e-6."""
import numpy as np
import pytest
import torch

import block_quantized_gemv_amd as q
import oracle
import workloads as W
from gpu_util import DEV, host, to_dev

pytestmark = pytest.mark.gpu


def pack6(m: W.Q6KMatrix) -> q.PackedQ6K:
    return q.PackedQ6K.from_blocks(to_dev(m.blocks().reshape(-1)), m.M, m.K)


def s2_bound(m: W.Q6KMatrix, x: np.ndarray) -> np.ndarray:
    ds = np.repeat(m.d.astype(np.float64), 256, axis=1) * np.repeat(m.sc.astype(np.float64), 16,
                                                                    axis=1)
    a = np.abs(ds * m.code) + 32 * np.abs(ds)
    return np.abs(x.astype(np.float64)) @ a.T


def check(y, yr, S2, what):
    err = np.abs(np.asarray(y, np.float64) - yr)
    bad = np.argwhere(~(err <= 2e-5 * S2 + 1e-6))
    assert bad.size == 0, f"{what}: {bad.shape[0]} outputs out of tolerance, first {tuple(bad[0])}"


def expected_layout(m: W.Q6KMatrix):
    """The packed layout written out from its definition (q8gemv.h)."""
    M, K = m.code.shape
    T = (M + 63) // 64
    c = np.zeros((T * 64, K), np.uint8)
    c[:M] = m.code
    sub = c.reshape(T, 64, K // 32, 32)
    low, high = sub & 15, sub >> 4
    ql = (low[..., :16] | (low[..., 16:] << 4)).transpose(0, 2, 1, 3)   # [T][K/32][64][16]
    hw = (high.astype(np.uint32).reshape(T, 64, K // 32, 2, 16) << (2 * np.arange(16))).sum(-1)
    qh = hw.astype(np.uint32).transpose(0, 2, 1, 3)                     # [T][K/32][64][2]
    sc = np.zeros((T * 64, K // 16), np.int8)
    sc[:M] = m.sc
    dd = np.zeros((T * 64, K // 256), np.float16)
    dd[:M] = m.d
    meta = np.zeros((T * 64, K // 128, 16), np.uint8)
    meta[:, :, 0:8] = sc.view(np.uint8).reshape(T * 64, K // 128, 8)
    meta[:, :, 8:10] = np.repeat(dd, 2, axis=1).view(np.uint8).reshape(T * 64, K // 128, 2)
    meta = meta.reshape(T, 64, K // 128, 16).transpose(0, 2, 1, 3)
    return (np.ascontiguousarray(ql).reshape(-1),
            np.ascontiguousarray(qh).view(np.uint8).reshape(-1),
            np.ascontiguousarray(meta).reshape(-1))


@pytest.mark.parametrize("M,K", [(1, 256), (64, 512), (65, 256), (130, 1024), (300, 4864)])
def test_q6k_repack_layout_bit_exact(M, K):
    m = W.draw_q6k(W.rng(86, M, K), M, K)
    p = pack6(m)
    el, eh, em = expected_layout(m)
    assert np.array_equal(host(p.ql), el)
    assert np.array_equal(host(p.qh), eh)
    assert np.array_equal(host(p.meta), em)


SHAPES = [(1, 256), (64, 256), (65, 512), (130, 1024), (300, 2048), (64, 4096), (200, 4864),
          (1000, 1024)]


@pytest.mark.parametrize("M,K", SHAPES)
@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 6, 7, 8])
def test_q6k_gemv_matches_oracle(M, K, N):
    g = W.rng(87, M * 7 + N, K)
    m = W.draw_q6k(g, M, K)
    x = W.draw_x(g, N, K)
    y = host(q.q6k_gemv(pack6(m), to_dev(x)))
    yr, _ = oracle.q6k_gemv(m.blocks(), x)
    check(y, yr, s2_bound(m, x), f"q6k {M}x{K} N={N}")


def test_q6k_one_hot_exact():
    """x = e_k gives the fp32 rounding of weight k exactly, at positions in
    every 16-weight group of a block, with extreme codes and scales."""
    M, K = 130, 1024
    m = W.draw_q6k(W.rng(88), M, K)
    m.code[0, :], m.code[1, :] = 63, 0
    m.sc[2, :], m.sc[3, :] = -128, 127
    p = pack6(m)
    ks = [0, 15, 16, 31, 32, 63, 64, 100, 127, 128, 200, 255, 256, 511, 700, 1023]
    deq = oracle.q6k_dequant_rows(m.blocks(), K)
    for i in range(0, len(ks), 4):
        sel = ks[i:i + 4]
        x = np.zeros((len(sel), K), np.float32)
        for j, k in enumerate(sel):
            x[j, k] = 1.0
        y = host(q.q6k_gemv(p, to_dev(x)))
        for j, k in enumerate(sel):
            assert np.array_equal(y[j], deq[:, k].astype(np.float32)), k


def test_q6k_rejects_bad_arguments():
    m = W.draw_q6k(W.rng(89), 64, 256)
    p = pack6(m)
    x = torch.zeros((1, 256), device=DEV)
    y = torch.zeros((1, 64), device=DEV)
    bad = q.PackedQ6K(p.ql, p.qh[4:], p.meta, 64, 256)  # high bits not 8-byte aligned
    with pytest.raises(q.Q8Error):
        q.q6k_gemv(bad, x)
    rc = q.lib().q6k_gemv(q.ctypes.byref(p.desc), x.cpu().data_ptr(), y.data_ptr(), 64, 256, 1,
                          None, 0, None)
    assert rc == q.Q8_EHOSTPTR
