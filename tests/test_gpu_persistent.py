"""GPU persistent decode chain (q8_0_chain_*): the whole decode step in one
launch.  Every projection is checked against the oracle applied to the GPU's
own input to that projection (read back from the chain's workspace records),
the glue (RMS scale, GQA broadcast, SwiGLU, residual) in fp64 by the oracle;
the 24-layer token end to end through the argmax band; repeated runs and
graph replays must be bitwise identical; the status word must stay 0."""
import numpy as np
import pytest
import torch

import block_quantized_gemv_amd as q
import oracle
import q8tol
import workloads as W
from block_quantized_gemv_amd.decode import ChainConfig
from gpu_util import DEV, host, pack, to_dev
from test_gpu_chain import C_REL, U, make_layers, normed_bound, silu_prime

pytestmark = pytest.mark.gpu


def build(cfg: ChainConfig, n_layers: int, cfg_id: int, with_lm=True):
    aos, packed = make_layers(cfg_id, cfg, n_layers)
    lm = W.matrix(cfg_id, 0, W.MAT_LM_HEAD, cfg.vocab, cfg.hidden) if with_lm else None
    pc = q.PersistentChain(packed, pack(lm) if with_lm else None, cfg.hidden, cfg.n_heads,
                           cfg.n_kv_heads, cfg.head_dim, cfg.intermediate, cfg.eps)
    h0 = W.activations(cfg_id, 1, cfg.hidden)[0]
    return aos, lm, pc, h0


def outputs(pc: q.PersistentChain, cfg: ChainConfig):
    logits = torch.full((max(pc.vocab, 1),), np.nan, dtype=torch.float32, device=DEV)
    tok = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    h_out = torch.full((cfg.hidden,), np.nan, dtype=torch.float32, device=DEV)
    return logits, tok, h_out


def check_stagewise(aos, lm, pc, h0, cfg: ChainConfig, logits, tok, h_out, lm_rows=None):
    n_layers = len(aos)
    H, I = cfg.hidden, cfg.intermediate
    voff = (cfg.n_heads + cfg.n_kv_heads) * cfg.head_dim
    hin = h0.astype(np.float64)
    for l in range(n_layers):
        qkv = host(pc.read(l, q.Q8_CHAIN_QKV)).astype(np.float64)
        yr, S = oracle.gemv(aos[l]["qkv"], oracle.rmsnorm(hin, cfg.eps))
        assert np.all(np.abs(qkv - yr) <= normed_bound(S, yr)), f"layer {l} qkv"
        h1 = host(pc.read(l, q.Q8_CHAIN_H_ATTN)).astype(np.float64)
        att = oracle.gqa_position0(qkv[voff:voff + cfg.n_kv_heads * cfg.head_dim], cfg.n_heads,
                                   cfg.n_kv_heads, cfg.head_dim)
        t, S = oracle.gemv(aos[l]["wo"], att)
        yr = hin + t
        assert np.all(np.abs(h1 - yr) <= q8tol.bound(S) + 2 * U * np.abs(yr)), f"layer {l} wo"
        s = host(pc.read(l, q.Q8_CHAIN_SWIGLU)).astype(np.float64)
        gu, S = oracle.gemv(aos[l]["gate_up"], oracle.rmsnorm(h1, cfg.eps))
        g, u = gu[:I], gu[I:]
        tg, tu = normed_bound(S[:I], g), normed_bound(S[I:], u)
        sil = g / (1 + np.exp(-g))
        b = (np.abs(silu_prime(g)) * np.abs(u) * tg + (np.abs(sil) + 1.2 * tg) * tu
             + 0.5 * tg * tg * np.abs(u) + 8 * U * np.abs(sil * u))
        assert np.all(np.abs(s - oracle.swiglu(g, u)) <= b), f"layer {l} swiglu"
        h2 = host(pc.read(l, q.Q8_CHAIN_H_OUT)).astype(np.float64)
        t, S = oracle.gemv(aos[l]["down"], s)
        yr = h1 + t
        assert np.all(np.abs(h2 - yr) <= q8tol.bound(S) + 2 * U * np.abs(yr)), f"layer {l} down"
        hin = h2
    if n_layers:
        assert np.array_equal(host(h_out), hin.astype(np.float32)), "h_out is the last record"
    if lm is None:
        return
    lg = host(logits)
    pick = int(host(tok)[0])
    assert pick == int(np.argmax(lg)), "next_token is the lowest index of the largest logit"
    # every logit unless a sample size is given
    rows = (np.arange(cfg.vocab) if lm_rows is None else
            np.unique(np.concatenate([np.random.default_rng(0).integers(0, cfg.vocab, lm_rows),
                                      [0, cfg.vocab - 1, pick]])))
    yr, S = oracle.gemv(lm.aos()[rows], oracle.rmsnorm(hin, cfg.eps))
    assert np.all(np.abs(lg[rows].astype(np.float64) - yr) <= normed_bound(S, yr)), "lm_head"


def run(pc, h0, logits, tok, h_out):
    pc.run(to_dev(h0), logits if pc.vocab else None, tok if pc.vocab else None, h_out)
    torch.cuda.synchronize()


def test_persistent_two_layers_stagewise():
    cfg = ChainConfig(vocab=4096)
    aos, lm, pc, h0 = build(cfg, 2, 2)
    print(f"plan: grid {pc.plan.grid}, lds {pc.plan.lds_bytes}, ws {pc.plan.ws_bytes}")
    logits, tok, h_out = outputs(pc, cfg)
    run(pc, h0, logits, tok, h_out)
    check_stagewise(aos, lm, pc, h0, cfg, logits, tok, h_out)
    assert pc.status() == 0


def test_persistent_small_ragged_config():
    """hidden 128, 4 heads over 2 KV heads of 32, intermediate 192, vocab 1000
    (a ragged last LM tile), 3 layers."""
    cfg = ChainConfig(hidden=128, n_heads=4, n_kv_heads=2, head_dim=32, intermediate=192,
                      vocab=1000)
    aos, lm, pc, h0 = build(cfg, 3, 60)
    logits, tok, h_out = outputs(pc, cfg)
    run(pc, h0, logits, tok, h_out)
    check_stagewise(aos, lm, pc, h0, cfg, logits, tok, h_out, lm_rows=1000)
    assert pc.status() == 0


def test_persistent_wide_heads():
    """4 query heads over 4 KV heads of 128 (no grouping, 512 value rows),
    hidden 512, intermediate 512, 2 layers."""
    cfg = ChainConfig(hidden=512, n_heads=4, n_kv_heads=4, head_dim=128, intermediate=512,
                      vocab=2000)
    aos, lm, pc, h0 = build(cfg, 2, 63)
    logits, tok, h_out = outputs(pc, cfg)
    run(pc, h0, logits, tok, h_out)
    check_stagewise(aos, lm, pc, h0, cfg, logits, tok, h_out, lm_rows=2000)
    assert pc.status() == 0


def test_persistent_lm_head_only_and_no_lm_head():
    cfg = ChainConfig(vocab=3000)
    aos, lm, pc, h0 = build(cfg, 0, 61)
    logits, tok, h_out = outputs(pc, cfg)
    run(pc, h0, logits, tok, h_out)
    check_stagewise(aos, lm, pc, h0, cfg, logits, tok, h_out)
    cfg2 = ChainConfig(vocab=0)
    aos, lm, pc, h0 = build(cfg2, 2, 62, with_lm=False)
    logits, tok, h_out = outputs(pc, cfg2)
    run(pc, h0, logits, tok, h_out)
    check_stagewise(aos, lm, pc, h0, cfg2, logits, tok, h_out)
    assert pc.status() == 0


def test_persistent_24_layers_end_to_end():
    """The full Qwen2.5-0.5B-shaped step in one launch; per-layer parity of
    the first and last layers, the pick against the fp64 oracle chain."""
    cfg = ChainConfig()
    aos, lm, pc, h0 = build(cfg, 24, 2)
    logits, tok, h_out = outputs(pc, cfg)
    run(pc, h0, logits, tok, h_out)
    check_stagewise(aos, lm, pc, h0, cfg, logits, tok, h_out)
    pick = int(host(tok)[0])
    h = h0.astype(np.float64)
    for l in range(24):
        h = oracle.qwen_layer(aos[l]["qkv"], aos[l]["wo"], aos[l]["gate_up"], aos[l]["down"], h,
                              cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.eps)
    yr, S = oracle.gemv(lm.aos(), oracle.rmsnorm(h, cfg.eps))
    order = np.argsort(-yr)
    gap = yr[order[0]] - yr[order[1]]
    allowance = 1e-3 * np.abs(yr[order[0]])
    print(f"oracle top-2 gap {gap:.4g}, allowance {allowance:.4g}, pick {pick}, oracle {order[0]}")
    if gap > allowance:
        assert pick == order[0]
    else:
        assert yr[pick] >= yr[order[0]] - allowance
    hg = host(h_out).astype(np.float64)
    assert np.max(np.abs(hg - h)) <= 1e-3 * np.max(np.abs(h))
    assert pc.status() == 0


def test_persistent_repeatable_and_graph_replay():
    cfg = ChainConfig(vocab=4096)
    aos, lm, pc, h0 = build(cfg, 2, 70)
    logits, tok, h_out = outputs(pc, cfg)
    x = to_dev(h0)
    pc.run(x, logits, tok, h_out)
    torch.cuda.synchronize()
    ref = (logits.clone(), tok.clone(), h_out.clone(), pc.read(1, q.Q8_CHAIN_SWIGLU).clone())
    for _ in range(5):
        logits.fill_(0)
        h_out.fill_(0)
        pc.run(x, logits, tok, h_out)
        torch.cuda.synchronize()
        assert torch.equal(logits, ref[0]) and torch.equal(tok, ref[1])
        assert torch.equal(h_out, ref[2])
        assert torch.equal(pc.read(1, q.Q8_CHAIN_SWIGLU), ref[3])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        pc.run(x, logits, tok, h_out, stream=s)
    for _ in range(3):
        logits.fill_(0)
        tok.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(logits, ref[0]) and torch.equal(tok, ref[1])
        pc.run(x, logits, tok, h_out)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(logits, ref[0])
    x.copy_(to_dev(W.activations(71, 1, cfg.hidden)[0]))
    g.replay()
    torch.cuda.synchronize()
    new = logits.clone()
    assert not torch.equal(new, ref[0])
    pc.run(x, logits, tok, h_out)
    torch.cuda.synchronize()
    assert torch.equal(logits, new)
    assert pc.status() == 0


def test_persistent_expired_wait_marks_step_invalid():
    """A host-set spin limit of one round makes the kernel's own bounded waits
    give up (the data of other workgroups is not there yet): the step must say
    so (next_token == -1, sticky status bit 1) and exit normally; the next step
    with the default limit is valid again and bitwise equal to a clean run."""
    cfg = ChainConfig(vocab=4096)
    aos, lm, pc, h0 = build(cfg, 2, 72)
    logits, tok, h_out = outputs(pc, cfg)
    x = to_dev(h0)
    pc.run(x, logits, tok, h_out, check=True)
    torch.cuda.synchronize()
    ref_tok, ref_logits = int(host(tok)[0]), logits.clone()
    assert ref_tok >= 0 and pc.status() == 0
    pc.plan.spin_limit = 1
    pc.run(x, logits, tok, h_out)
    torch.cuda.synchronize()
    assert int(host(tok)[0]) == -1
    assert pc.status() & 2
    with pytest.raises(q.ChainStepError):
        pc.run(x, logits, tok, h_out, check=True)
    pc.plan.spin_limit = 0
    pc.run(x, logits, tok, h_out, check=True)
    torch.cuda.synchronize()
    assert int(host(tok)[0]) == ref_tok
    assert torch.equal(logits, ref_logits)


def test_persistent_coherent_mode_bitwise_equal():
    """Q8_CHAIN_COHERENT (every hand-off through device-scope stores) changes
    only where the hand-offs are visible, never the arithmetic."""
    cfg = ChainConfig(vocab=4096)
    aos, lm, pc, h0 = build(cfg, 3, 73)
    logits, tok, h_out = outputs(pc, cfg)
    x = to_dev(h0)
    pc.run(x, logits, tok, h_out, check=True)
    torch.cuda.synchronize()
    ref = (logits.clone(), tok.clone(), h_out.clone(), pc.read(2, q.Q8_CHAIN_SWIGLU).clone())
    flags = pc.plan.flags
    pc.plan.flags = flags | q.Q8_CHAIN_COHERENT
    pc.run(x, logits, tok, h_out, check=True)
    torch.cuda.synchronize()
    pc.plan.flags = flags
    assert torch.equal(logits, ref[0]) and torch.equal(tok, ref[1])
    assert torch.equal(h_out, ref[2]) and torch.equal(pc.read(2, q.Q8_CHAIN_SWIGLU), ref[3])
    check_stagewise(aos, lm, pc, h0, cfg, logits, tok, h_out)


def test_persistent_stamped_run_equals_plain_and_orders_its_stamps():
    """q8_0_chain_run_stamped: the same outputs bit for bit as q8_0_chain_run,
    and per workgroup the stage-start stamps of every recorded layer are
    nonzero and in stage order (A < B < C < D < next A)."""
    cfg = ChainConfig(vocab=4096)
    n_layers = 3
    aos, lm, pc, h0 = build(cfg, n_layers, 72)
    logits, tok, h_out = outputs(pc, cfg)
    x = to_dev(h0)
    pc.run(x, logits, tok, h_out)
    torch.cuda.synchronize()
    ref = (logits.clone(), tok.clone(), h_out.clone())
    G, Wd = pc.plan.grid, q.Q8_CHAIN_STAMP_WORDS
    stamps = torch.zeros(G * Wd, dtype=torch.int64, device=DEV)
    logits.fill_(0)
    pc.run(x, logits, tok, h_out, stamps=stamps)
    torch.cuda.synchronize()
    assert torch.equal(logits, ref[0]) and torch.equal(tok, ref[1]) and torch.equal(h_out, ref[2])
    t = host(stamps).reshape(G, Wd)
    P = q.Q8_CHAIN_STAMP_POINTS
    lay = t[:, :q.Q8_CHAIN_STAMP_LAYERS * P].reshape(G, q.Q8_CHAIN_STAMP_LAYERS, P)
    for l in range(n_layers):
        starts = lay[:, l, [0, 2, 4, 7]]
        assert np.all(starts > 0), l
        assert np.all(np.diff(starts, axis=1) > 0), l
        if l + 1 < n_layers:
            assert np.all(lay[:, l + 1, 0] > lay[:, l, 7]), l
    assert np.all(lay[:, n_layers:, :] == 0)  # nothing recorded past the last layer
    kern = t[:, q.Q8_CHAIN_STAMP_LAYERS * P:]
    assert np.all(kern[:, 0] > 0) and np.all(kern[:, 3] >= kern[:, 1]) and np.all(kern[:, 1] > 0)
    assert pc.status() == 0
