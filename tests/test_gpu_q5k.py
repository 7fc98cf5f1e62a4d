"""GPU parity of the Q5_K weights (NEXT-2): the repack layout bit-exact, the
GEMV against the fp64 oracle on the same GGUF bytes.

Tolerance (derived as for Q4_K): each 32-weight sub-block is evaluated as
fl(d s) * sum(code x) - fl(dmin m) * sum(x) in fp32 with codes 0..31 (d s and
dmin m are exact: 11 x 6 bits), so the rounding error is bounded by both
terms' magnitudes, S2 = sum_k (|d s_j code_k| + |dmin m_j|) |x_k|:
|y_gpu - y_ref| <= 2e-5 * S2 + 1e-6."""
import numpy as np
import pytest
import torch

import block_quantized_gemv_amd as q
import oracle
import workloads as W
from gpu_util import DEV, host, to_dev

pytestmark = pytest.mark.gpu


def pack5(m: W.Q5KMatrix) -> q.PackedQ5K:
    return q.PackedQ5K.from_blocks(to_dev(m.blocks().reshape(-1)), m.M, m.K)


def s2_bound(m: W.Q5KMatrix, x: np.ndarray) -> np.ndarray:
    """S2[n][r] from the drawn fields (fp64)."""
    d = np.repeat(m.d.astype(np.float64), 256, axis=1)
    dmin = np.repeat(m.dmin.astype(np.float64), 256, axis=1)
    s = np.repeat(m.s.astype(np.float64), 32, axis=1)
    mm = np.repeat(m.m.astype(np.float64), 32, axis=1)
    a = np.abs(d * s * m.code) + np.abs(dmin * mm)
    return np.abs(x.astype(np.float64)) @ a.T


def check(y, yr, S2, what):
    err = np.abs(np.asarray(y, np.float64) - yr)
    bad = np.argwhere(~(err <= 2e-5 * S2 + 1e-6))
    assert bad.size == 0, f"{what}: {bad.shape[0]} outputs out of tolerance, first {tuple(bad[0])}"


def expected_layout(m: W.Q5KMatrix):
    """The packed layout written out from its definition (q8gemv.h): qs byte b
    of sub-block c of row r = low[r, 32c + b] | low[r, 32c + 16 + b] << 4; qh
    dword bit 8b + a = fifth bit of weight 4a + b, bit 8b + 4 + a that of
    weight 16 + 4a + b, the 4 dwords of a quad's sub-blocks together per row;
    meta = the block's first 16 GGUF bytes; rows padded
    to 64 with zeros."""
    M, K = m.code.shape
    T = (M + 63) // 64
    c = np.zeros((T * 64, K), np.uint8)
    c[:M] = m.code
    sub = c.reshape(T, 64, K // 32, 32)
    low, fifth = sub & 15, (sub >> 4).astype(np.uint32)
    qs = (low[..., :16] | (low[..., 16:] << 4)).transpose(0, 2, 1, 3)  # [T][K/32][64][16]
    fw = np.zeros(sub.shape[:3], np.uint32)
    for a in range(4):
        for b in range(4):
            fw |= fifth[..., 4 * a + b] << (8 * b + a)
            fw |= fifth[..., 16 + 4 * a + b] << (8 * b + 4 + a)
    qh = fw.reshape(T, 64, K // 128, 4).transpose(0, 2, 1, 3)         # [T][K/128][64][4]
    hdr = np.zeros((T * 64, K // 256, 16), np.uint8)
    hdr[:M] = m.blocks()[:, :, :16]
    meta = hdr.reshape(T, 64, K // 256, 16).transpose(0, 2, 1, 3)
    return (np.ascontiguousarray(qs).reshape(-1),
            np.ascontiguousarray(qh).view(np.uint8).reshape(-1),
            np.ascontiguousarray(meta).reshape(-1))


@pytest.mark.parametrize("M,K", [(1, 256), (64, 512), (65, 256), (130, 1024), (300, 4864)])
def test_q5k_repack_layout_bit_exact(M, K):
    m = W.draw_q5k(W.rng(93, M, K), M, K)
    p = pack5(m)
    es, eh, em = expected_layout(m)
    assert np.array_equal(host(p.qs), es)
    assert np.array_equal(host(p.qh), eh)
    assert np.array_equal(host(p.meta), em)


SHAPES = [(1, 256), (64, 256), (65, 512), (130, 1024), (300, 2048), (64, 4096), (200, 4864),
          (1000, 1024)]


@pytest.mark.parametrize("M,K", SHAPES)
@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 6, 7, 8])
def test_q5k_gemv_matches_oracle(M, K, N):
    g = W.rng(94, M * 7 + N, K)
    m = W.draw_q5k(g, M, K)
    x = W.draw_x(g, N, K)
    y = host(q.q5k_gemv(pack5(m), to_dev(x)))
    yr, _ = oracle.q5k_gemv(m.blocks(), x)
    check(y, yr, s2_bound(m, x), f"q5k {M}x{K} N={N}")


def test_q5k_one_hot_exact():
    """x = e_k gives the fp32 rounding of weight k exactly, at positions in
    every 4-weight group of both halves of sub-blocks in both block halves,
    with all-ones and all-zero fifth bits and extreme scales and mins."""
    M, K = 130, 1024
    m = W.draw_q5k(W.rng(95), M, K)
    m.code[0, :], m.code[1, :] = 31, 0
    m.code[2, :] = 16
    m.s[3, :], m.m[3, :] = 63, 0
    m.s[4, :], m.m[4, :] = 0, 63
    p = pack5(m)
    ks = [0, 3, 4, 15, 16, 19, 20, 31, 32, 63, 64, 100, 127, 128, 200, 255, 256, 511, 700, 1023]
    deq = oracle.q5k_dequant_rows(m.blocks(), K)
    for i in range(0, len(ks), 4):
        sel = ks[i:i + 4]
        x = np.zeros((len(sel), K), np.float32)
        for j, k in enumerate(sel):
            x[j, k] = 1.0
        y = host(q.q5k_gemv(p, to_dev(x)))
        for j, k in enumerate(sel):
            assert np.array_equal(y[j], deq[:, k].astype(np.float32)), k


def test_q5k_zero_codes_give_exact_zero():
    """Zero codes and zero mins give exact 0 (ragged rows, several columns)."""
    m = W.draw_q5k(W.rng(96), 70, 512)
    m.code[:], m.m[:] = 0, 0
    y = host(q.q5k_gemv(pack5(m), to_dev(W.draw_x(W.rng(97), 3, 512))))
    assert np.array_equal(y, np.zeros((3, 70), np.float32))


def test_q5k_rejects_bad_arguments():
    m = W.draw_q5k(W.rng(99), 64, 256)
    p = pack5(m)
    x = torch.zeros((1, 256), device=DEV)
    y = torch.zeros((1, 64), device=DEV)
    bad = q.PackedQ5K(p.qs, p.qh[4:], p.meta, 64, 256)  # fifth bits not 16-byte aligned
    with pytest.raises(q.Q8Error):
        q.q5k_gemv(bad, x)
    rc = q.lib().q5k_gemv(q.ctypes.byref(p.desc), x.cpu().data_ptr(), y.data_ptr(), 64, 256, 1,
                          None, 0, None)
    assert rc == q.Q8_EHOSTPTR
