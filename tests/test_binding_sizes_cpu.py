"""The Python binding checks every tensor's size against the weights before
anything reaches the library: the C ABI only receives raw pointers, so a
short x or y would otherwise become an out-of-bounds device access.  Host
only: with CPU tensors a correctly sized call stops at the device-tensor
check, a wrongly sized one at the size check, and nothing is launched."""
import pytest
import torch

import block_quantized_gemv_amd as q

M, K = 128, 256


def packed(M=M, K=K, n_mats=1):
    qb, db = q.q8_0_packed_size(M, K)
    return q.PackedQ8(torch.zeros(n_mats * qb, dtype=torch.uint8),
                      torch.zeros(n_mats * db, dtype=torch.uint8), M, K, n_mats)


def raises_size(call):
    with pytest.raises(ValueError) as e:
        call()
    assert "device tensor" not in str(e.value), str(e.value)


def reaches_device_check(call):
    with pytest.raises(ValueError, match="device tensor"):
        call()


def test_gemv_sizes():
    W = packed()
    raises_size(lambda: q.q8_0_gemv(W, torch.zeros(K - 1)))
    raises_size(lambda: q.q8_0_gemv(W, torch.zeros(2, K + 32)))
    raises_size(lambda: q.q8_0_gemv(W, torch.zeros(9, K)))              # N > 8
    raises_size(lambda: q.q8_0_gemv(W, torch.zeros(2, 2, K)))           # not [N, K]
    raises_size(lambda: q.q8_0_gemv(W, torch.zeros(3, K), torch.zeros(3 * M - 1)))
    reaches_device_check(lambda: q.q8_0_gemv(W, torch.zeros(3, K), torch.zeros(3, M)))
    reaches_device_check(lambda: q.q8_0_gemv(W, torch.zeros(K)))


def test_gemv_argmax_and_q8act_sizes():
    W = packed()
    raises_size(lambda: q.q8_0_gemv_argmax(W, torch.zeros(4, K), torch.zeros(4 * M),
                                           torch.zeros(3, dtype=torch.int32)))
    raises_size(lambda: q.q8_0_gemv_argmax(W, torch.zeros(4, K), torch.zeros(4 * M - 1)))
    reaches_device_check(lambda: q.q8_0_gemv_argmax(W, torch.zeros(4, K), torch.zeros(4 * M),
                                                    torch.zeros(4, dtype=torch.int32)))
    qx, dx = torch.zeros(2, K, dtype=torch.int8), torch.zeros(2, K // 32, dtype=torch.int16)
    raises_size(lambda: q.q8_0_gemv_q8act(W, qx[:, :K - 32], dx))
    raises_size(lambda: q.q8_0_gemv_q8act(W, qx, dx[:1]))
    raises_size(lambda: q.q8_0_gemv_q8act(W, qx, dx, torch.zeros(2 * M - 1)))
    reaches_device_check(lambda: q.q8_0_gemv_q8act(W, qx, dx, torch.zeros(2 * M)))


def test_fused_sizes():
    W = packed()
    f = q.make_fusion(q.Q8_PRO_RMSNORM, 0, 1e-6)
    raises_size(lambda: q.q8_0_gemv_fused(W, torch.zeros(K + 1), torch.zeros(M), f))
    raises_size(lambda: q.q8_0_gemv_fused(W, torch.zeros(K), torch.zeros(M - 1), f))
    f = q.make_fusion(q.Q8_PRO_NONE, q.Q8_EPI_SWIGLU)
    raises_size(lambda: q.q8_0_gemv_fused(W, torch.zeros(K), torch.zeros(M // 2 - 1), f))
    reaches_device_check(lambda: q.q8_0_gemv_fused(W, torch.zeros(K), torch.zeros(M // 2), f))
    f = q.make_fusion(q.Q8_PRO_NONE, q.Q8_EPI_RESIDUAL, residual=torch.zeros(M - 1))
    raises_size(lambda: q.q8_0_gemv_fused(W, torch.zeros(K), torch.zeros(M), f))
    # GQA: K = n_heads * head_dim and the value heads inside x
    f = q.make_fusion(q.Q8_PRO_GQA, 0, n_heads=4, n_kv_heads=2, head_dim=64, gqa_offset=384)
    raises_size(lambda: q.q8_0_gemv_fused(W, torch.zeros(500), torch.zeros(M), f))
    reaches_device_check(lambda: q.q8_0_gemv_fused(W, torch.zeros(512), torch.zeros(M), f))
    f = q.make_fusion(q.Q8_PRO_GQA, 0, n_heads=2, n_kv_heads=2, head_dim=64, gqa_offset=0)
    raises_size(lambda: q.q8_0_gemv_fused(W, torch.zeros(512), torch.zeros(M), f))


def test_kquant_sizes():
    for cls, fn, sizes in ((q.PackedQ4K, q.q4k_gemv, q.q4k_packed_size),
                           (q.PackedQ5K, q.q5k_gemv, q.q5k_packed_size),
                           (q.PackedQ6K, q.q6k_gemv, q.q6k_packed_size)):
        bufs = [torch.zeros(n, dtype=torch.uint8) for n in sizes(M, K)]
        W = cls(*bufs, M, K)
        raises_size(lambda: fn(W, torch.zeros(K - 32)))
        raises_size(lambda: fn(W, torch.zeros(2, K), torch.zeros(2 * M - 1)))
        reaches_device_check(lambda: fn(W, torch.zeros(2, K), torch.zeros(2 * M)))


def test_moe_sizes():
    I, H, S = 128, 256, 4
    gu = packed(2 * I, H, 8)
    dn = packed(H, I, 8)
    sh_gu, sh_dn = packed(256, H), packed(H, 128)
    ids = torch.zeros(S, dtype=torch.int32)
    mode = q.Q8_MOE_SCATTER | q.Q8_MOE_SWIGLU
    raises_size(lambda: q.q8_0_moe_gemv(gu, ids, None, torch.zeros(H + 32),
                                        torch.zeros(S * I + 128), mode, shared=sh_gu))
    raises_size(lambda: q.q8_0_moe_gemv(gu, ids, None, torch.zeros(H),
                                        torch.zeros(S * I + 127), mode, shared=sh_gu))
    reaches_device_check(lambda: q.q8_0_moe_gemv(gu, ids, None, torch.zeros(H),
                                                 torch.zeros(S * I + 128), mode, shared=sh_gu))
    w, lam = torch.zeros(S), torch.zeros(1)
    raises_size(lambda: q.q8_0_moe_gemv(dn, ids, w, torch.zeros(S * I), torch.zeros(H),
                                        q.Q8_MOE_COMBINE, shared=sh_dn, shared_gate=lam))
    raises_size(lambda: q.q8_0_moe_gemv(dn, ids, w[:3], torch.zeros(S * I + 128), torch.zeros(H),
                                        q.Q8_MOE_COMBINE, shared=sh_dn, shared_gate=lam))
    raises_size(lambda: q.q8_0_moe_gemv(dn, ids, w, torch.zeros(S * I + 128),
                                        torch.zeros(H - 1), q.Q8_MOE_COMBINE, shared=sh_dn,
                                        shared_gate=lam))
    reaches_device_check(lambda: q.q8_0_moe_gemv(dn, ids, w, torch.zeros(S * I + 128),
                                                 torch.zeros(H), q.Q8_MOE_COMBINE,
                                                 shared=sh_dn, shared_gate=lam))


def test_router_argmax_repack_sizes():
    raises_size(lambda: q.q8_0_route_topk(torch.zeros(60), 4, torch.zeros(3, dtype=torch.int32)))
    raises_size(lambda: q.q8_0_route_topk(torch.zeros(60), 4, slot_weights=torch.zeros(2)))
    reaches_device_check(lambda: q.q8_0_route_topk(torch.zeros(60), 4))
    raises_size(lambda: q.q8_0_argmax(torch.zeros(10), torch.zeros(0, dtype=torch.int32)))
    qb, db = q.q8_0_packed_size(M, K)
    aos = torch.zeros(M * (K // 32) * 34, dtype=torch.uint8)
    raises_size(lambda: q.q8_0_repack(aos[1:], M, K, torch.zeros(qb, dtype=torch.uint8),
                                      torch.zeros(db, dtype=torch.uint8)))
    raises_size(lambda: q.q8_0_repack(aos, M, K, torch.zeros(qb - 1, dtype=torch.uint8),
                                      torch.zeros(db, dtype=torch.uint8)))
    reaches_device_check(lambda: q.q8_0_repack(aos, M, K, torch.zeros(qb, dtype=torch.uint8),
                                               torch.zeros(db, dtype=torch.uint8)))
