"""q8_0_gemv_noalloc: the GEMV without a workspace or any allocation (the
library's per-device scratch array).  Called through the C ABI, it must give
bitwise the result of q8_0_gemv (same kernels and plan) and meet the parity
bar against the fp64 oracle, on two calls in a row, the second with a
smaller input; a plan larger than the array is refused before any launch."""
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


def noalloc_c(p, x, y):
    """The entry point called directly through the C ABI (ctypes)."""
    N = 1 if x.dim() == 1 else x.shape[0]
    return q.lib().q8_0_gemv_noalloc(ctypes.byref(p.desc), x.data_ptr(), y.data_ptr(), p.M, p.K,
                                     N, torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("first,second", [((896, 4864, 4), (896, 2048, 3)),
                                          ((4096, 12288, 8), (896, 4864, 2)),
                                          ((1152, 896, 1), (130, 896, 3))])
def test_noalloc_matches_gemv_twice(first, second):
    for i, (M, K, N) in enumerate((first, second)):
        m = W.matrix(90 + i, M, K, M, K)
        x = W.activations(91 + i, N, K)
        p = pack(m)
        xd = to_dev(x)
        ws_need = q.q8_0_workspace_bytes(q.Q8_OP_GEMV, M, K, N)
        y_ref = q.q8_0_gemv(p, xd).clone()
        y = torch.full((N, M), np.nan, dtype=torch.float32, device=DEV)
        assert noalloc_c(p, xd, y) == q.Q8_OK
        torch.cuda.synchronize()
        assert torch.equal(y.reshape(-1), y_ref.reshape(-1)), (M, K, N, ws_need)
        yr, S = oracle.gemv(m.aos(), x)
        q8tol.check(host(y).reshape(N, M), yr.reshape(N, M), S.reshape(N, M),
                    f"noalloc {M}x{K} N={N}")


def test_noalloc_repeated_calls_stream_ordered():
    """Back-to-back calls of different shapes on one stream share the array:
    each must still be exact (the ticket counters are cleared per call)."""
    shapes = [(896, 4864, 3), (4096, 12288, 8), (896, 4864, 3)]
    outs = []
    ref = []
    for i, (M, K, N) in enumerate(shapes):
        m = W.matrix(95, M, K, M, K)
        x = to_dev(W.activations(96, N, K))
        p = pack(m)
        ref.append(q.q8_0_gemv(p, x).clone())
        y = torch.empty((N, M), dtype=torch.float32, device=DEV)
        assert noalloc_c(p, x, y) == q.Q8_OK
        outs.append(y)
    torch.cuda.synchronize()
    for y, r in zip(outs, ref):
        assert torch.equal(y.reshape(-1), r.reshape(-1))


def test_noalloc_refuses_plans_beyond_the_array():
    """4096 x 2^20 at N = 8 plans more partials than 8 MiB: refused on the
    host (Q8_EWORKSPACE) before anything is launched; the (fake) pointers are
    never touched."""
    M, K, N = 4096, 1 << 20, 8
    assert q.q8_0_workspace_bytes(q.Q8_OP_GEMV, M, K, N) > (8 << 20)
    qb, db = q.q8_0_packed_size(M, K)
    desc = q.q8_0_weights(256, 256, M, K, 1, qb, db, q.Q8_LAYOUT_ROWS, 0)
    rc = q.lib().q8_0_gemv_noalloc(ctypes.byref(desc), 256, 256, M, K, N, None)
    assert rc == q.Q8_EWORKSPACE
