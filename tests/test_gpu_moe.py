"""GPU mixture-of-experts FFN, stage by stage against the oracle:
router ids bit-exact, gate_up of every slot (+ shared) in one launch, SwiGLU
epilogue, and the fused down + weighted combine in one launch."""
import numpy as np
import pytest
import torch

import block_quantized_gemv_amd as q
import oracle
import q8tol
import workloads as W
from gpu_util import DEV, host, pack, to_dev

pytestmark = pytest.mark.gpu


def silu_prime(g):
    s = 1.0 / (1.0 + np.exp(-g))
    return s * (1.0 + g * (1.0 - s))


def swiglu_bound(g_ref, u_ref, Sg, Su):
    """Tolerance of h = silu(g) * u computed in fp32 from g, u that are each
    within the GEMV tolerance: first-order propagation plus the fp32
    evaluation of silu and the product (a few ulps of |h|)."""
    tg, tu = q8tol.bound(Sg), q8tol.bound(Su)
    sil = g_ref / (1.0 + np.exp(-g_ref))
    h = sil * u_ref
    return (np.abs(silu_prime(g_ref)) * np.abs(u_ref) * tg + (np.abs(sil) + 1.2 * tg) * tu
            + 0.5 * tg * tg * np.abs(u_ref) + 8 * 2.0 ** -24 * np.abs(h))


class MoE:
    def __init__(self, cfg, E, H, I, Ish, S=4, layout=q.Q8_LAYOUT_ROWS):
        self.E, self.H, self.I, self.Ish, self.S = E, H, I, Ish, S
        self.gu = W.expert_stack(cfg, W.MAT_GATE_UP, E, 2 * I, H)
        self.dn = W.expert_stack(cfg, W.MAT_DOWN, E, H, I)
        self.sgu = W.matrix(cfg, 0, W.MAT_SHARED_GU, 2 * Ish, H).aos()
        self.sdn = W.matrix(cfg, 0, W.MAT_SHARED_DOWN, H, Ish).aos()
        self.p_gu = pack(self.gu, 2 * I, H, n_mats=E, layout=layout)
        self.p_dn = pack(self.dn, H, I, n_mats=E)
        self.p_sgu = pack(self.sgu, layout=layout)
        self.p_sdn = pack(self.sdn)
        self.cfg = cfg

    def inputs(self, token):
        x = W.activations(self.cfg, 1, self.H, layer=token)[0]
        lg = W.router_logits(self.cfg, token, self.E)
        lam = W.shared_gate_logit(self.cfg, token)
        return x, lg, lam

    def scatter(self, ids, x, swiglu, shared=True):
        Mo = self.I if swiglu else 2 * self.I
        Msh = (self.Ish if swiglu else 2 * self.Ish) if shared else 0
        y = torch.full((self.S * Mo + Msh,), np.nan, dtype=torch.float32, device=DEV)
        mode = q.Q8_MOE_SCATTER | (q.Q8_MOE_SWIGLU if swiglu else 0)
        q.q8_0_moe_gemv(self.p_gu, ids, None, x, y, mode, shared=self.p_sgu if shared else None)
        return y

    def combine(self, ids, w, h, lam, shared=True):
        y = torch.full((self.H,), np.nan, dtype=torch.float32, device=DEV)
        q.q8_0_moe_gemv(self.p_dn, ids, w, h, y, q.Q8_MOE_COMBINE,
                        shared=self.p_sdn if shared else None,
                        shared_gate=lam if shared else None)
        return y


def run_stagewise(moe: MoE, token: int):
    x, lg, lam = moe.inputs(token)
    xd, lgd = to_dev(x), to_dev(lg)
    lamd = torch.tensor([lam], dtype=torch.float32, device=DEV)
    ids, w = q.q8_0_route_topk(lgd, moe.S)
    ids_r, w_r = oracle.route_topk(lg, moe.S)
    idh = host(ids)
    assert np.array_equal(idh, ids_r)
    assert np.all(np.abs(host(w).astype(np.float64) - w_r) <= 1e-6)
    I, Ish = moe.I, moe.Ish
    # gate_up of every slot + shared, one launch, raw outputs
    gu = host(moe.scatter(ids, xd, swiglu=False)).astype(np.float64)
    refs = []
    for s in range(moe.S):
        yr, S = oracle.gemv(moe.gu[idh[s]], x)
        q8tol.check(gu[s * 2 * I:(s + 1) * 2 * I], yr, S, f"scatter slot {s}")
        refs.append((yr, S))
    ysh, Ssh = oracle.gemv(moe.sgu, x)
    q8tol.check(gu[moe.S * 2 * I:], ysh, Ssh, "scatter shared")
    # SwiGLU epilogue
    h = moe.scatter(ids, xd, swiglu=True)
    hh = host(h).astype(np.float64)
    for s, (yr, S) in enumerate(refs):
        b = swiglu_bound(yr[:I], yr[I:], S[:I], S[I:])
        err = np.abs(hh[s * I:(s + 1) * I] - oracle.swiglu(yr[:I], yr[I:]))
        assert np.all(err <= b), f"swiglu slot {s}"
    b = swiglu_bound(ysh[:Ish], ysh[Ish:], Ssh[:Ish], Ssh[Ish:])
    assert np.all(np.abs(hh[moe.S * I:] - oracle.swiglu(ysh[:Ish], ysh[Ish:])) <= b)
    # combine on the GPU's own h, router weights and gate logit
    y = host(moe.combine(ids, w, h, lamd)).astype(np.float64)
    yr, Sabs = oracle.moe_combine(moe.dn, idh, host(w).astype(np.float64),
                                  hh[:moe.S * I].reshape(moe.S, I), moe.sdn, hh[moe.S * I:],
                                  oracle.sigmoid(float(lam)))
    q8tol.check(y, yr, Sabs, "combine")
    # end to end against the oracle on x (reported; rounding composes)
    ye = oracle.moe_ffn(moe.gu, moe.dn, ids_r, w_r, moe.sgu, moe.sdn, oracle.sigmoid(float(lam)), x)
    rel = float(np.max(np.abs(y - ye)) / np.max(np.abs(ye)))
    assert rel < 1e-3, rel
    return ids, w, h, y


LAYOUTS = [q.Q8_LAYOUT_ROWS, q.Q8_LAYOUT_GATE_UP_PAIRS]


@pytest.mark.parametrize("layout", LAYOUTS)
def test_moe_small_stagewise(layout):
    moe = MoE(cfg=50, E=8, H=256, I=128, Ish=192, layout=layout)
    for token in range(4):
        run_stagewise(moe, token)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_moe_qwen15_shapes_stagewise(layout):
    c = W.C5
    moe = MoE(cfg=c["cfg"], E=c["n_experts"], H=c["hidden"], I=c["inter"], Ish=c["shared_inter"],
              S=c["top_k"], layout=layout)
    for token in range(2):
        run_stagewise(moe, token)


def test_moe_fused_equals_per_slot_composition():
    """The one-launch scatter/combine equals per-slot dense GEMV calls on each
    selected expert (the fused-vs-per-slot check of the #144 PR), within the
    GEMV tolerance."""
    moe = MoE(cfg=51, E=8, H=256, I=128, Ish=192)
    x, lg, lam = moe.inputs(0)
    xd = to_dev(x)
    ids, w = q.q8_0_route_topk(to_dev(lg), moe.S)
    idh = host(ids)
    gu = host(moe.scatter(ids, xd, swiglu=False)).astype(np.float64)
    for s in range(moe.S):
        ys = host(q.q8_0_gemv(moe.p_gu.expert(int(idh[s])), xd)).astype(np.float64)
        _, S = oracle.gemv(moe.gu[idh[s]], x)
        assert np.all(np.abs(gu[s * 256:(s + 1) * 256] - ys) <= 2 * q8tol.bound(S))


def test_moe_one_hot_weights_no_shared_is_dense_ffn():
    moe = MoE(cfg=52, E=8, H=256, I=128, Ish=192)
    x, lg, _ = moe.inputs(1)
    xd = to_dev(x)
    ids, _ = q.q8_0_route_topk(to_dev(lg), moe.S)
    w = torch.tensor([1.0, 0.0, 0.0, 0.0], dtype=torch.float32, device=DEV)
    h = moe.scatter(ids, xd, swiglu=True, shared=False)
    y = host(moe.combine(ids, w, h, None, shared=False)).astype(np.float64)
    e0 = int(host(ids)[0])
    hh = host(h).astype(np.float64)
    yr, S = oracle.gemv(moe.dn[e0], hh[:128])
    q8tol.check(y, yr, S, "one-hot combine")


def test_moe_bad_expert_id_sets_status_and_zeroes_slot():
    moe = MoE(cfg=53, E=8, H=256, I=128, Ish=192)
    x, _, lam = moe.inputs(2)
    xd = to_dev(x)
    ids = torch.tensor([3, 8, -1, 5], dtype=torch.int32, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    y = torch.full((4 * 256 + 384,), np.nan, dtype=torch.float32, device=DEV)
    q.q8_0_moe_gemv(moe.p_gu, ids, None, xd, y, q.Q8_MOE_SCATTER, shared=moe.p_sgu, dev_status=st)
    yh = host(y).astype(np.float64)
    assert int(host(st)[0]) & 1
    assert np.all(yh[256:768] == 0)
    for s, e in ((0, 3), (3, 5)):
        yr, S = oracle.gemv(moe.gu[e], x)
        q8tol.check(yh[s * 256:(s + 1) * 256], yr, S, f"valid slot {s}")
    st.zero_()
    ids_ok = torch.tensor([3, 1, 2, 5], dtype=torch.int32, device=DEV)
    q.q8_0_moe_gemv(moe.p_gu, ids_ok, None, xd, y, q.Q8_MOE_SCATTER, shared=moe.p_sgu,
                    dev_status=st)
    assert int(host(st)[0]) == 0


def test_moe_repeatable():
    moe = MoE(cfg=54, E=8, H=256, I=128, Ish=192)
    x, lg, lam = moe.inputs(3)
    xd, lamd = to_dev(x), torch.tensor([lam], dtype=torch.float32, device=DEV)
    ids, w = q.q8_0_route_topk(to_dev(lg), moe.S)
    h0 = moe.scatter(ids, xd, True).clone()
    y0 = moe.combine(ids, w, h0, lamd).clone()
    for _ in range(20):
        h = moe.scatter(ids, xd, True)
        assert torch.equal(h, h0)
        assert torch.equal(moe.combine(ids, w, h, lamd), y0)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("swiglu", [False, True])
def test_moe_router_fused_into_scatter(layout, swiglu):
    """q8_0_moe_route_gemv: the router fused into the gate_up launch picks the
    oracle's experts (bit-exact, planted ties included), publishes the same
    ids and weights as q8_0_route_topk, and its products equal the unfused
    route + scatter pair bitwise (same kernel, same plan)."""
    moe = MoE(cfg=52, E=60, H=256, I=128, Ish=192, layout=layout)
    mode = q.Q8_MOE_SCATTER | (q.Q8_MOE_SWIGLU if swiglu else 0)
    Mo = moe.I if swiglu else 2 * moe.I
    Msh = moe.Ish if swiglu else 2 * moe.Ish
    for t in range(12):
        x, lg, _ = moe.inputs(t)
        if t % 3 == 0:  # ties at the top and across the k-th place
            lg[np.random.default_rng(t).integers(0, moe.E, 6)] = lg.max()
        xd, lgd = to_dev(x), to_dev(lg)
        y_f = torch.full((moe.S * Mo + Msh,), np.nan, dtype=torch.float32, device=DEV)
        _, ids_f, w_f = q.q8_0_moe_route_gemv(moe.p_gu, lgd, moe.S, xd, y_f, mode,
                                              shared=moe.p_sgu)
        ids, w = q.q8_0_route_topk(lgd, moe.S)
        y = moe.scatter(ids, xd, swiglu)
        ids_r, w_r = oracle.route_topk(lg, moe.S)
        assert np.array_equal(host(ids_f), ids_r), t
        assert np.array_equal(host(ids_f), host(ids)), t
        assert np.array_equal(host(w_f), host(w)), t
        assert np.all(np.abs(host(w_f).astype(np.float64) - w_r) <= 1e-6), t
        assert np.array_equal(host(y_f), host(y)), t


def test_moe_router_fused_qwen15_token():
    """The fused router at the Qwen1.5-MoE shapes (60 experts, top-4, shared
    expert), followed by the combine on its published ids and weights, equals
    the three-launch token bitwise."""
    c = W.C5
    moe = MoE(cfg=c["cfg"], E=c["n_experts"], H=c["hidden"], I=c["inter"], Ish=c["shared_inter"],
              S=c["top_k"])
    for t in range(3):
        x, lg, lam = moe.inputs(t)
        xd, lgd = to_dev(x), to_dev(lg)
        lamd = torch.tensor([lam], dtype=torch.float32, device=DEV)
        h_f = torch.full((moe.S * moe.I + moe.Ish,), np.nan, dtype=torch.float32, device=DEV)
        _, ids_f, w_f = q.q8_0_moe_route_gemv(moe.p_gu, lgd, moe.S, xd, h_f,
                                              q.Q8_MOE_SCATTER | q.Q8_MOE_SWIGLU,
                                              shared=moe.p_sgu)
        y_f = moe.combine(ids_f, w_f, h_f, lamd)
        ids, w = q.q8_0_route_topk(lgd, moe.S)
        h = moe.scatter(ids, xd, swiglu=True)
        y = moe.combine(ids, w, h, lamd)
        assert np.array_equal(host(h_f), host(h)), t
        assert np.array_equal(host(y_f), host(y)), t


def test_moe_router_fused_invalid_arguments():
    moe = MoE(cfg=53, E=8, H=256, I=128, Ish=192)
    lib = q.lib()
    lg = to_dev(np.zeros(8, dtype=np.float32))
    x = to_dev(np.zeros(256, dtype=np.float32))
    y = torch.zeros(4 * 256 + 384, dtype=torch.float32, device=DEV)
    ids = torch.zeros(8, dtype=torch.int32, device=DEV)
    w = torch.zeros(8, dtype=torch.float32, device=DEV)
    import ctypes
    call = lambda E, k, mode: lib.q8_0_moe_route_gemv(
        ctypes.byref(moe.p_gu.desc), lg.data_ptr(), E, ids.data_ptr(), w.data_ptr(), x.data_ptr(),
        y.data_ptr(), 256, 256, k, mode, None, None, None, 0, None)
    assert call(8, 9, q.Q8_MOE_SCATTER) == q.Q8_EINVAL      # k > E
    assert call(9, 4, q.Q8_MOE_SCATTER) == q.Q8_EINVAL      # E > experts stored
    assert call(8, 0, q.Q8_MOE_SCATTER) == q.Q8_EINVAL
    assert call(8, 4, q.Q8_MOE_COMBINE) == q.Q8_EINVAL      # scatter only
    with pytest.raises(ValueError):
        q.q8_0_moe_route_gemv(moe.p_gu, lg, 4, x, y, q.Q8_MOE_COMBINE)
