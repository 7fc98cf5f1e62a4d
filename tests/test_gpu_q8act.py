"""GPU parity of the opt-in integer-activation variant: the activation
quantizer bit-exact against the oracle (codes and binary16 scales), and the
int8 x int8 GEMV within the fp32 tolerance of the oracle's fp64 result on
the same codes."""
import ctypes
import numpy as np
import pytest
import torch

import block_quantized_gemv_amd as q
import oracle
import q8tol
import workloads as W
from gpu_util import DEV, host, pack, to_dev

pytestmark = pytest.mark.gpu


def quantize(x: np.ndarray):
    qx, dx = q.q8_0_quantize_act(to_dev(x))
    return host(qx), host(dx).view(np.uint16)


@pytest.mark.parametrize("N,K", [(1, 32), (1, 896), (3, 160), (8, 1408), (8, 12288), (2, 4864)])
def test_quantize_act_bit_exact(N, K):
    x = W.draw_x(W.rng(70, N, K), N, K)
    qx, dx = quantize(x)
    eq, ed = oracle.quantize_act(x)
    assert np.array_equal(dx, ed), (N, K)
    assert np.array_equal(qx, eq), (N, K)


def test_quantize_act_special_blocks():
    """All-zero block (codes 0, scale 0), amax = 127 (d = 1, so x/d is x and
    halves round to even), negative amax, constant block, tiny and large
    magnitudes, and a block whose amax sits in its last entry."""
    K = 32 * 8
    x = np.zeros((2, K), dtype=np.float32)
    x[0, 32:64] = np.r_[127.0, np.arange(31) - 15.5].astype(np.float32)      # ties to even
    x[0, 64:96] = np.r_[-127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, np.zeros(25)]
    x[0, 96:128] = 3.0                                                          # constant
    x[0, 128:160] = np.linspace(-1e-3, 2e-3, 32, dtype=np.float32)              # tiny
    x[0, 160:192] = np.linspace(-6e4, 5e4, 32, dtype=np.float32)                # large
    x[0, 192:224] = np.r_[np.arange(31, dtype=np.float32) * 0.1, -9.0]          # amax last
    x[1] = -x[0]
    qx, dx = quantize(x)
    eq, ed = oracle.quantize_act(x)
    assert np.array_equal(dx, ed)
    assert np.array_equal(qx, eq)
    assert not qx[:, 0:32].any() and not dx[:, 0].any()
    assert list(qx[0, 65:71]) == [0, 2, 2, 0, -2, -2]                            # RNE ties


SHAPES = [(1, 32), (64, 96), (65, 160), (130, 224), (200, 1408), (896, 896), (300, 4864),
          (64, 5632), (40, 12288), (2048, 2048)]


@pytest.mark.parametrize("M,K", SHAPES)
@pytest.mark.parametrize("N", [1, 2, 3, 5, 8])
def test_gemv_q8act_matches_oracle(M, K, N):
    g = W.rng(71, M * 7 + N, K)
    m = W.draw_matrix(g, M, K)
    x = W.draw_x(g, N, K)
    qx, dx = q.q8_0_quantize_act(to_dev(x))
    y = q.q8_0_gemv_q8act(pack(m), qx, dx)
    eq, ed = oracle.quantize_act(x)
    yr, S = oracle.gemv_q8act(m.aos(), eq, ed)
    q8tol.check(host(y), yr, S, f"gemv_q8act {M}x{K} N={N}")


def test_gemv_q8act_extreme_codes_exact():
    """Weights and activation codes all -128 / 127 with power-of-two scales:
    each block's integer sum is exact and the scaled sums are exact in fp32,
    so the result equals the closed form bit for bit."""
    M, K = 130, 1408
    for qw, qa in ((-128, 127), (127, 127), (-128, -128)):
        m = W.Q8Matrix(np.full((M, K), qw, np.int8),
                       np.full((M, K // 32), np.float16(0.25)))
        qx = np.full((2, K), qa, np.int8)
        dx = np.full((2, K // 32), np.float16(0.5)).view(np.uint16)
        y = host(q.q8_0_gemv_q8act(pack(m), to_dev(qx), to_dev(dx.view(np.int16))))
        want = 0.25 * 0.5 * qw * qa * K
        assert np.array_equal(y, np.full((2, M), want, np.float32)), (qw, qa)


def test_gemv_q8act_rejects_bad_arguments():
    m = W.draw_matrix(W.rng(72), 64, 96)
    p = pack(m)
    qx = torch.zeros((1, 96), dtype=torch.int8, device=DEV)
    dx = torch.zeros((1, 3), dtype=torch.int16, device=DEV)
    shifted = torch.zeros(97, dtype=torch.int8, device=DEV)[1:].view(1, 96)  # misaligned
    with pytest.raises(q.Q8Error):
        q.q8_0_gemv_q8act(p, shifted, dx)
    # 9 columns: the binding refuses before the call, and the C entry point
    # itself refuses too
    with pytest.raises(ValueError):
        q.q8_0_gemv_q8act(p, qx.repeat(9, 1), dx.repeat(9, 1))
    q9, d9 = qx.repeat(9, 1), dx.repeat(9, 1)
    y9 = torch.zeros(9 * 64, device=DEV)
    ws = q.Workspace(1 << 20)
    wp, wb = ws.get(1 << 20)
    rc = q.lib().q8_0_gemv_q8act(ctypes.byref(p.desc), q9.data_ptr(), d9.data_ptr(),
                                 y9.data_ptr(), 64, 96, 9, wp, wb,
                                 torch.cuda.current_stream().cuda_stream)
    assert rc == q.Q8_EINVAL
    with pytest.raises(q.Q8Error):
        q.q8_0_quantize_act(torch.zeros((1, 100), device=DEV))
    with pytest.raises(q.Q8Error):
        q.q8_0_quantize_act(torch.zeros((9, 64), device=DEV))
