"""Benchmark: the Q8_0 decode matmul chain of a Qwen2.5-0.5B-shaped decoder on
one MI355X, and every kernel of the path on its own workload.

A step is one decode token through the whole hot path: 24 layers of Q8_0
GEMVs (qkv 1152x896 behind the RMSNorm, wo 896x896 behind the GQA broadcast
with the residual add, gate_up 9728x896 behind the RMSNorm with the SwiGLU,
down 896x4864 with the residual add), then the LM head 151936x896 behind the
final RMSNorm and the argmax.  By default the step is ONE launch of the
persistent decode-chain kernel (q8_0_chain_run); `--path graph` times the
97-launch chain of q8_0_gemv_fused calls replayed from a HIP graph instead.
Weights are synthetic and seeded (quants uniform in [-127, 127], scales
|N(0,1)|*0.01 in binary16, h0 ~ N(0,1)); 527 MB of weights per step exceed
the 256 MB Infinity Cache, so every step streams them from HBM.

Prints one JSON line:
  value        algorithmic HBM GB/s of the step (1.0625 B/weight + x + y per
               GEMV) over the timed region; tok/s alongside; the timed steps
               are also split into rounds (median / min / p90 per step)
  roofline     the step's kernel: algorithmic bytes per launch / average
               launch duration, from HIP events on the launch stream
  rows         every kernel of the path on its own workload, timed three ways:
               M1  dependent calls replayed from a HIP graph, each on a
                   different weight copy (the copies in rotation exceed 768 MB,
                   three times the Infinity Cache, so every call streams cold)
               M2  the same calls in 4 independent graph branches, so launches
                   overlap: steady-state streaming throughput of the shape
               M3  the decode step as 97 dependent graph-replayed launches
               each over rounds (median / min / p90 of the per-call time), plus
               the on-box read reference (q8_stream_read)
  cpu_baseline the fp64 oracle on this host: 1 thread and all threads, and a
               BLAS-backed numpy matvec, on a bounded sample

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--path persistent|graph]
                       [--only SUBSTR[,SUBSTR...]] [--no-rows] [--no-cpu-baseline] [--stages RUNS]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
COLD_BYTES = 768e6     # weight copies in rotation per row: 3x the 256 MB Infinity Cache
ROUNDS = 7             # timing rounds per row


def gemv_bytes(M, K, N=1):
    return 1.0625 * M * K + 4 * K * N + 4 * M * N


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=24)
    ap.add_argument("--path", choices=("persistent", "graph"), default="persistent",
                    help="persistent: one q8_0_chain_run launch per step; graph: 97 "
                         "q8_0_gemv_fused launches replayed from a HIP graph")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="wall-clock budget of the oracle CPU baseline (split over its legs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the per-kernel measurements of every workload")
    ap.add_argument("--only", default="",
                    help="comma-separated substrings: run only the rows whose description "
                         "contains one of them (no decode step, no CPU baseline); for profiling")
    ap.add_argument("--stages", type=int, default=0, metavar="RUNS",
                    help="only time the persistent step with stage timestamps "
                         "(q8_0_chain_run_stamped) over RUNS steps and print the per-stage "
                         "breakdown of a layer")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes 5 times (the reference "
                         "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE) and exit")
    return ap.parse_args()


SHAPES = {"qkv": (1152, 896), "wo": (896, 896), "gate_up": (9728, 896), "down": (896, 4864)}


def spread(xs):
    """median / min / p90 of a list of per-round values."""
    a = np.sort(np.asarray(xs, dtype=np.float64))
    p90 = a[min(len(a) - 1, int(math.ceil(0.9 * len(a))) - 1)]
    return float(np.median(a)), float(a[0]), float(p90)


def build_weights(n_layers, log):
    """Seeded synthetic weights of every layer and the LM head, repacked on
    the device.  gate_up uses the gate/up pairs layout the chain kernels
    expect; the others the plain row layout."""
    import torch
    import block_quantized_gemv_amd as q
    import workloads as W
    from block_quantized_gemv_amd.decode import ChainConfig

    cfg = ChainConfig()
    dev = torch.device("cuda", 0)
    mats = {"qkv": W.MAT_QKV, "wo": W.MAT_WO, "gate_up": W.MAT_GATE_UP, "down": W.MAT_DOWN}
    layers, sample_aos = [], {}
    t0 = time.time()
    for l in range(n_layers):
        L = {}
        for name, mat in mats.items():
            M, K = SHAPES[name]
            aos = W.matrix(W.C2["cfg"], l, mat, M, K).aos()
            if l == 0:
                sample_aos[name] = aos
            layout = q.Q8_LAYOUT_GATE_UP_PAIRS if name == "gate_up" else q.Q8_LAYOUT_ROWS
            L[name] = q.PackedQ8.from_aos(torch.from_numpy(aos.reshape(-1)).to(dev), M, K,
                                          layout=layout)
        layers.append(L)
    lm = W.matrix(W.C2["cfg"], 0, W.MAT_LM_HEAD, cfg.vocab, cfg.hidden).aos()
    sample_aos["lm_head_rows"] = lm[:16384].copy()
    lm_p = q.PackedQ8.from_aos(torch.from_numpy(lm.reshape(-1)).to(dev), cfg.vocab, cfg.hidden)
    del lm
    h0 = torch.from_numpy(W.activations(W.C2["cfg"], 1, cfg.hidden)[0]).to(dev)
    torch.cuda.synchronize()
    log(f"weights generated and repacked in {time.time() - t0:.1f} s")
    step_bytes = n_layers * sum(gemv_bytes(M, K) for (M, K) in SHAPES.values())
    step_bytes += gemv_bytes(cfg.vocab, cfg.hidden)
    return cfg, layers, lm_p, h0, step_bytes, sample_aos


def time_launches(launch, steps, warmup, stream, rounds=ROUNDS):
    """Average time of one `launch()` over `steps` back-to-back launches, from
    HIP events recorded on the stream the kernels run on; events between
    groups of steps also give per-round averages."""
    import torch
    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    r = max(1, min(rounds, steps))
    cuts = [steps * i // r for i in range(r + 1)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(r + 1)]
    ev[0].record(stream)
    for i in range(r):
        for _ in range(cuts[i + 1] - cuts[i]):
            launch()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    total = ev[0].elapsed_time(ev[-1]) * 1e-3 / steps
    per_round = [ev[i].elapsed_time(ev[i + 1]) * 1e-3 / (cuts[i + 1] - cuts[i]) for i in range(r)]
    return total, per_round


def time_persistent(cfg, layers, lm_p, h0, steps, warmup, stream, log):
    import torch
    import block_quantized_gemv_amd as q
    pc = q.PersistentChain(layers, lm_p, cfg.hidden, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim,
                           cfg.intermediate, cfg.eps)
    dev = h0.device
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device=dev)
    tok = torch.empty(1, dtype=torch.int32, device=dev)
    h_out = torch.empty(cfg.hidden, dtype=torch.float32, device=dev)
    log(f"persistent chain: grid {pc.plan.grid} x {pc.plan.threads} threads, "
        f"LDS {pc.plan.lds_bytes} B, workspace {pc.plan.ws_bytes} B, flags {pc.plan.flags}")
    s, rounds = time_launches(lambda: pc.run(h0, logits, tok, h_out, stream=stream), steps,
                              warmup, stream)
    status = pc.status()
    token = int(tok.cpu()[0])
    if status != 0 or token < 0:
        raise RuntimeError(f"persistent chain reported status {status}, token {token}")
    return s, rounds, 1, "q8::chain_kernel", token


def time_graph(cfg, layers, lm_p, h0, steps, warmup, stream, log):
    from block_quantized_gemv_amd.decode import DecodeChain
    chain = DecodeChain(cfg, layers, lm_p)
    chain.h0.copy_(h0)
    g = chain.capture()
    s, rounds = time_launches(g.replay, steps, warmup, stream)
    return s, rounds, 4 * len(layers) + 1, "q8::gemv_kernel<1>", int(chain.next_token.cpu()[0])


def graph_rounds(enqueue, n_calls, branches=1, rounds=ROUNDS):
    """Seconds per call of `enqueue(i, stream)` (i < n_calls), captured once
    into a HIP graph and replayed `rounds` times; HIP events on the replay
    stream bracket each replay, so host launch overhead is excluded and each
    call's dispatch is included.  With branches > 1 the calls are dealt to
    that many independent graph branches (forked from and joined to the
    capture stream), so their launches may overlap."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(min(n_calls, 2)):
            enqueue(i, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    bs = [torch.cuda.Stream() for _ in range(branches)] if branches > 1 else []
    with torch.cuda.graph(g, stream=side):
        if branches == 1:
            for i in range(n_calls):
                enqueue(i, side)
        else:
            for b in bs:
                b.wait_stream(side)
            for k, b in enumerate(bs):
                with torch.cuda.stream(b):
                    for i in range(k, n_calls, branches):
                        enqueue(i, b)
            for b in bs:
                side.wait_stream(b)
    g.replay()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    out = []
    for _ in range(rounds):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        g.replay()
        e1.record(st)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) * 1e-3 / n_calls)
    del g
    return out


def copies_for(nbytes):
    """Weight copies to rotate over so that more than COLD_BYTES are in
    rotation (every call then reads its weights cold from HBM)."""
    return max(2, int(math.ceil(COLD_BYTES / nbytes)) + 1)


def rand_packed(M, K, n_mats, gen):
    """Seeded packed Q8_0 weights drawn on the device with the workload's
    distributions (quants uniform in [-127, 127], scales |N(0,1)|*0.01 in
    binary16); only for shapes with no padding (M % 64 == 0, K % 128 == 0)."""
    import torch
    import block_quantized_gemv_amd as q
    assert M % 64 == 0 and K % 128 == 0
    qb, db = q.q8_0_packed_size(M, K)
    dev = torch.device("cuda", 0)
    qs = torch.randint(-127, 128, (n_mats * qb,), dtype=torch.int8, device=dev, generator=gen)
    d = (torch.randn(n_mats * db // 2, device=dev, generator=gen).abs() * 0.01).half()
    return q.PackedQ8(qs.view(torch.uint8), d.view(torch.uint8), M, K, n_mats)


def rand_packed_q4k(M, K, n_mats, gen):
    """Seeded packed Q4_K weights drawn on the device: every nibble and every
    6-bit scale/min uniform (random bytes), d = |N(0,1)|*0.001 and
    dmin = |N(0,1)|*0.004 in binary16.  Returns one tensor pair holding n_mats
    packed matrices back to back (M % 64 == 0, K % 256 == 0)."""
    import torch
    import block_quantized_gemv_amd as q
    assert M % 64 == 0 and K % 256 == 0
    qb, mb = q.q4k_packed_size(M, K)
    dev = torch.device("cuda", 0)
    qs = torch.randint(0, 256, (n_mats * qb,), dtype=torch.uint8, device=dev, generator=gen)
    meta = torch.randint(0, 256, (n_mats * mb // 16, 16), dtype=torch.uint8, device=dev,
                         generator=gen)
    hdr = torch.randn(n_mats * mb // 16, 2, device=dev, generator=gen).abs()
    hdr = (hdr * torch.tensor([0.001, 0.004], device=dev)).half()
    meta[:, 0:4] = hdr.view(torch.uint8).view(-1, 4)
    return qs, meta.view(-1), qb, mb


def rand_packed_q5k(M, K, n_mats, gen):
    """Seeded packed Q5_K weights drawn on the device: nibbles, fifth bits and
    6-bit scales/mins uniform (random bytes), d = |N(0,1)|*0.0005 and
    dmin = |N(0,1)|*0.004 in binary16.  Returns qs, qh, meta tensors holding
    n_mats packed matrices back to back and their per-matrix byte counts
    (M % 64 == 0, K % 256 == 0)."""
    import torch
    import block_quantized_gemv_amd as q
    assert M % 64 == 0 and K % 256 == 0
    a, b, c = q.q5k_packed_size(M, K)
    dev = torch.device("cuda", 0)
    qs = torch.randint(0, 256, (n_mats * a,), dtype=torch.uint8, device=dev, generator=gen)
    qh = torch.randint(0, 256, (n_mats * b,), dtype=torch.uint8, device=dev, generator=gen)
    meta = torch.randint(0, 256, (n_mats * c // 16, 16), dtype=torch.uint8, device=dev,
                         generator=gen)
    hdr = torch.randn(n_mats * c // 16, 2, device=dev, generator=gen).abs()
    hdr = (hdr * torch.tensor([0.0005, 0.004], device=dev)).half()
    meta[:, 0:4] = hdr.view(torch.uint8).view(-1, 4)
    return qs, qh, meta.view(-1), (a, b, c)


def rand_packed_q6k(M, K, n_mats, gen):
    """Seeded packed Q6_K weights drawn on the device: every 6-bit code and
    int8 scale uniform (random bytes), d = |N(0,1)|*0.0002 in binary16.
    Returns ql, qh, meta tensors holding n_mats packed matrices back to back
    and their per-matrix byte counts (M % 64 == 0, K % 256 == 0)."""
    import torch
    import block_quantized_gemv_amd as q
    assert M % 64 == 0 and K % 256 == 0
    a, b, c = q.q6k_packed_size(M, K)
    dev = torch.device("cuda", 0)
    ql = torch.randint(0, 256, (n_mats * a,), dtype=torch.uint8, device=dev, generator=gen)
    qh = torch.randint(0, 256, (n_mats * b,), dtype=torch.uint8, device=dev, generator=gen)
    meta = torch.zeros(n_mats * c // 16, 16, dtype=torch.uint8, device=dev)
    meta[:, 0:8] = torch.randint(0, 256, (n_mats * c // 16, 8), dtype=torch.uint8, device=dev,
                                 generator=gen)
    d = (torch.randn(n_mats * c // 16, device=dev, generator=gen).abs() * 0.0002).half()
    meta[:, 8:10] = d.view(torch.uint8).view(-1, 2)
    return ql, qh, meta.view(-1), (a, b, c)


def measure_rows(log, only=()):
    """Every kernel of the path on its own workload, timed as M1 (dependent
    graph-replayed calls on rotating cold weight copies) and, for the
    0.5B-layer shapes and the LM head, M2 (the same calls in 4 independent
    graph branches): C1 896x896; the 0.5B layer shapes; lm_head with the fused
    RMSNorm/argmax and the standalone argmax; the 9B-class shapes at N = 1, 2,
    4, 8; the integer-activation variant; Q4_K, Q5_K and Q6_K weights on the
    9B shapes; the verify-chunk LM head with one argmax per column; the
    Qwen1.5-MoE-shaped FFN (router, scatter + SwiGLU, combine).  The on-box
    read reference (q8_stream_read) comes first."""
    import torch
    import block_quantized_gemv_amd as q
    import workloads as W
    dev = torch.device("cuda", 0)
    gen = torch.Generator(device=dev).manual_seed(1234)
    rows = []
    want = lambda what: not only or any(s in what for s in only)

    def rec(row, what, mode, secs, nbytes, **extra):
        med, mn, p90 = spread(secs)
        r = {"row": row, "what": what, "mode": mode, "us": round(med * 1e6, 3),
             "us_min": round(mn * 1e6, 3), "us_p90": round(p90 * 1e6, 3), "rounds": len(secs)}
        if nbytes:
            gbs = nbytes / med / 1e9
            r.update(GBs=round(gbs, 1), frac=round(gbs / PEAK_HBM_GBS, 4))
        r.update(extra)
        rows.append(r)
        log(f"{row} {mode} {what}: {med * 1e6:.2f} us (min {mn * 1e6:.2f}, p90 {p90 * 1e6:.2f})"
            + (f", {r['GBs']} GB/s" if nbytes else ""))

    # ---- the read reference: 16-byte non-temporal loads, 2 GiB and cold 145 MB
    if want("q8_stream_read"):
        out = torch.zeros(8192, dtype=torch.int32, device=dev)
        big = torch.empty(1 << 31, dtype=torch.uint8, device=dev).fill_(1)
        st = torch.cuda.current_stream()
        for grid in (2048, 4096):
            _, secs = time_launches(lambda: q.q8_stream_read(big, out, grid), 10, 2, st)
            rec("hbm", f"q8_stream_read 2 GiB (grid {grid} x 256)", "M1", secs, big.numel(),
                copies=1)
        del big
        lmb = 151936 * 896 * 17 // 16
        n = copies_for(lmb)
        bufs = torch.empty(n * lmb, dtype=torch.uint8, device=dev).fill_(1)
        views = [bufs[i * lmb:(i + 1) * lmb] for i in range(n)]
        secs = graph_rounds(lambda i, s: q.q8_stream_read(views[i % n], out, 4096, stream=s), n)
        rec("hbm", "q8_stream_read 145 MB (lm_head bytes), rotating cold copies", "M1", secs,
            lmb, copies=n)
        secs = graph_rounds(lambda i, s: q.q8_stream_read(views[i % n][:16], out, 1, stream=s),
                            n)
        rec("hbm", "q8_stream_read 16 B, one workgroup: the dependent-launch floor", "M1", secs,
            0)
        del bufs, views
        torch.cuda.empty_cache()

    def gemv_row(row, M, K, N, what, epi=None, m2=False):
        if not want(what):
            return
        n = copies_for(1.0625 * M * K)
        Wm = rand_packed(M, K, n, gen)
        qb, db = q.q8_0_packed_size(M, K)
        views = [q.PackedQ8(Wm.qs[i * qb:(i + 1) * qb], Wm.d[i * db:(i + 1) * db], M, K)
                 for i in range(n)]
        x = torch.randn(N, K, device=dev, generator=gen)
        nb = 4 if m2 else 1
        ys = [torch.empty(N, M, device=dev) for _ in range(nb)]
        if epi is None:
            op = q.Q8_OP_GEMV
            wss = [q.Workspace(q.q8_0_workspace_bytes(op, M, K, N)) for _ in range(nb)]
            call = lambda i, s: q.q8_0_gemv(views[i % n], x, ys[i % nb], wss[i % nb], stream=s)
            nbytes = gemv_bytes(M, K, N)
        elif epi in ("q8act", "q8act+quant"):
            # integer activations: codes + binary16 scales replace the fp32 vector
            qx, dx = q.q8_0_quantize_act(x)
            ws = q.Workspace(q.q8_0_workspace_bytes(q.Q8_OP_GEMV, M, K, N))
            if epi == "q8act":
                call = lambda i, s: q.q8_0_gemv_q8act(views[i % n], qx, dx, ys[0], ws, stream=s)
            else:
                def call(i, s):
                    q.q8_0_quantize_act(x, qx, dx, stream=s)
                    q.q8_0_gemv_q8act(views[i % n], qx, dx, ys[0], ws, stream=s)
            nbytes = 1.0625 * M * K + 1.0625 * K * N + 4 * M * N
        elif epi == "col_argmax":
            am = torch.empty(N, dtype=torch.int32, device=dev)
            ws = q.Workspace(q.q8_0_workspace_bytes(q.Q8_OP_GEMV_ARGMAX, M, K, N))
            call = lambda i, s: q.q8_0_gemv_argmax(views[i % n], x, ys[0], am, ws, stream=s)
            nbytes = gemv_bytes(M, K, N)
        else:
            tok = torch.empty(1, dtype=torch.int32, device=dev)
            fus = q.make_fusion(q.Q8_PRO_RMSNORM, q.Q8_EPI_ARGMAX, 1e-6, argmax_out=tok)
            ws = q.Workspace(q.q8_0_workspace_bytes(q.Q8_OP_GEMV_FUSED, M, K, q.Q8_EPI_ARGMAX))
            call = lambda i, s: q.q8_0_gemv_fused(views[i % n], x[0], ys[0][0], fus, ws,
                                                  stream=s)
            nbytes = gemv_bytes(M, K, N)
        rec(row, what, "M1", graph_rounds(call, n), nbytes, copies=n)
        if m2:
            rec(row, what, "M2", graph_rounds(call, n, branches=nb), nbytes, copies=n,
                branches=nb)
        del views, Wm
        torch.cuda.empty_cache()

    gemv_row("a2", 896, 896, 1, "C1 gemv 896x896", m2=True)
    for name, (M, K) in SHAPES.items():
        gemv_row("a2", M, K, 1, f"C2 {name} {M}x{K}", m2=True)
    gemv_row("a2", 151936, 896, 1, "C3 lm_head 151936x896", m2=True)
    gemv_row("a4", 151936, 896, 1, "C3 lm_head 151936x896 + RMSNorm + argmax", epi="argmax")
    if want("argmax over"):
        nl = 151936
        n = copies_for(4 * nl)
        vs = torch.randn(n, nl, device=dev, generator=gen)
        out = torch.empty(1, dtype=torch.int32, device=dev)
        ws = q.Workspace(q.q8_0_workspace_bytes(q.Q8_OP_ARGMAX, nl, 0, 0))
        rec("a4", "argmax over 151936 fp32 logits", "M1",
            graph_rounds(lambda i, s: q.q8_0_argmax(vs[i % n], out, ws, stream=s), n), 4 * nl,
            copies=n)
        del vs
        torch.cuda.empty_cache()
    for N in (1, 2, 4, 8):
        gemv_row("a3" if N > 1 else "a2", 24576, 4096, N, f"C4 gate_up 24576x4096 N={N}")
        gemv_row("a3" if N > 1 else "a2", 4096, 12288, N, f"C4 down 4096x12288 N={N}")
    for N in (1, 8):
        gemv_row("f3", 24576, 4096, N, f"C4 gate_up 24576x4096 N={N}, int8 activations",
                 epi="q8act")
    gemv_row("f3", 24576, 4096, 8, "C4 gate_up 24576x4096 N=8, quantize + int8 activations",
             epi="q8act+quant")

    def kquant_rows(tag, bpw, shapes, draw, make, fn, op):
        for (M, K) in shapes:
            for N in (1, 8):
                what = f"C4-shaped {M}x{K} {tag} N={N}"
                if not want(what):
                    continue
                n = copies_for(bpw * M * K)
                bufs, sizes = draw(M, K, n)
                views = [make([b[i * s:(i + 1) * s] for b, s in zip(bufs, sizes)], M, K)
                         for i in range(n)]
                x = torch.randn(N, K, device=dev, generator=gen)
                y = torch.empty(N, M, device=dev)
                ws = q.Workspace(q.q8_0_workspace_bytes(op, M, K, N))
                rec("n2", what, "M1",
                    graph_rounds(lambda i, s: fn(views[i % n], x, y, ws, stream=s), n),
                    bpw * M * K + 4 * K * N + 4 * M * N, copies=n)
                del views, bufs
                torch.cuda.empty_cache()

    def d4(M, K, n):
        qs, meta, qb, mb = rand_packed_q4k(M, K, n, gen)
        return (qs, meta), (qb, mb)

    def d5(M, K, n):
        qs, qh, meta, s = rand_packed_q5k(M, K, n, gen)
        return (qs, qh, meta), s

    def d6(M, K, n):
        ql, qh, meta, s = rand_packed_q6k(M, K, n, gen)
        return (ql, qh, meta), s

    c4 = ((24576, 4096), (4096, 12288))
    kquant_rows("Q4_K", 0.5625, c4, d4, lambda b, M, K: q.PackedQ4K(*b, M, K), q.q4k_gemv,
                q.Q8_OP_Q4K_GEMV)
    kquant_rows("Q5_K", 176 / 256, c4, d5, lambda b, M, K: q.PackedQ5K(*b, M, K), q.q5k_gemv,
                q.Q8_OP_Q5K_GEMV)
    kquant_rows("Q6_K", 210 / 256, c4, d6, lambda b, M, K: q.PackedQ6K(*b, M, K), q.q6k_gemv,
                q.Q8_OP_Q6K_GEMV)
    for N in (2, 8):
        gemv_row("f4", 151936, 896, N, f"lm_head 151936x896 N={N} + argmax per column (2 launches)",
                 epi="col_argmax")

    # Qwen1.5-MoE-shaped FFN, one token per call, routing from seeded N(0,1) logits
    if want("C5"):
        E, H, I, Ish, S, T = 60, 2048, 1408, 5632, 4, 32
        NSH = copies_for(gemv_bytes(2 * Ish, H) + gemv_bytes(H, Ish))
        gu, dn = rand_packed(2 * I, H, E, gen), rand_packed(H, I, E, gen)
        sgu = [rand_packed(2 * Ish, H, 1, gen) for _ in range(NSH)]
        sdn = [rand_packed(H, Ish, 1, gen) for _ in range(NSH)]
        logits = torch.from_numpy(np.stack([W.router_logits(5, t, E) for t in range(T)])).to(dev)
        lam = torch.randn(T, device=dev, generator=gen)
        x = torch.randn(T, H, device=dev, generator=gen)
        ids = torch.empty(T, S, dtype=torch.int32, device=dev)
        w = torch.empty(T, S, device=dev)
        h = torch.empty(T, S * I + Ish, device=dev)
        y = torch.empty(T, H, device=dev)
        mode_s = q.Q8_MOE_SCATTER | q.Q8_MOE_SWIGLU
        ws1 = q.Workspace(q.q8_0_workspace_bytes(q.Q8_OP_MOE_SCATTER, 2 * I, H, S, 2 * Ish, H,
                                                 mode_s))
        ws2 = q.Workspace(q.q8_0_workspace_bytes(q.Q8_OP_MOE_COMBINE, H, I, S, H, Ish,
                                                 q.Q8_MOE_COMBINE))
        route = lambda t, s: q.q8_0_route_topk(logits[t % T], S, ids[t % T], w[t % T], stream=s)
        scatter = lambda t, s: q.q8_0_moe_gemv(gu, ids[t % T], None, x[t % T], h[t % T], mode_s,
                                               shared=sgu[t % NSH], workspace=ws1, stream=s)
        combine = lambda t, s: q.q8_0_moe_gemv(dn, ids[t % T], w[t % T], h[t % T], y[t % T],
                                               q.Q8_MOE_COMBINE, shared=sdn[t % NSH],
                                               shared_gate=lam[t % T:t % T + 1], workspace=ws2,
                                               stream=s)
        for t in range(T):
            route(t, torch.cuda.current_stream())
        torch.cuda.synchronize()
        nt = max(T, NSH)
        bs = S * gemv_bytes(2 * I, H) + gemv_bytes(2 * Ish, H)
        bc = S * gemv_bytes(H, I) + gemv_bytes(H, Ish)
        rec("a5", "C5 router top-4 of 60", "M1", graph_rounds(route, nt), 0)
        rec("a6", "C5 scatter: 4 slots gate_up 2816x2048 + shared 11264x2048 + SwiGLU", "M1",
            graph_rounds(scatter, nt), bs, copies=NSH)
        rec("a8", "C5 combine: 4 slots down 2048x1408 + shared 2048x5632, weighted", "M1",
            graph_rounds(combine, nt), bc, copies=NSH)
        rec("a5-a8", "C5 MoE FFN token: router + scatter + combine (3 launches)", "M1",
            graph_rounds(lambda t, s: (route(t, s), scatter(t, s), combine(t, s)), nt), bs + bc,
            copies=NSH)
        # the router fused into the scatter launch; the combine reads the ids
        # and weights that launch publishes
        route_scatter = lambda t, s: q.q8_0_moe_route_gemv(
            gu, logits[t % T], S, x[t % T], h[t % T], mode_s, shared=sgu[t % NSH],
            expert_ids=ids[t % T], slot_weights=w[t % T], workspace=ws1, stream=s)
        rec("a5+a6", "C5 router fused into the scatter launch", "M1",
            graph_rounds(route_scatter, nt), bs, copies=NSH)
        rec("a5-a8", "C5 MoE FFN token: fused router + scatter, combine (2 launches)", "M1",
            graph_rounds(lambda t, s: (route_scatter(t, s), combine(t, s)), nt), bs + bc,
            copies=NSH)
        del gu, dn, sgu, sdn
        torch.cuda.empty_cache()
    return rows


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(sample_aos, seconds, log):
    """The oracle as it stands on this host's cores, over a bounded sample of
    the same workload (layer 0's four GEMVs plus 16384 LM-head rows),
    repeated until each leg's time budget is spent: one thread, then every
    thread of this process's affinity set; then a BLAS-backed numpy fp64
    matvec on the same sample dequantised once beforehand.  Each leg is
    reported in the metric's unit over the same algorithmic bytes."""
    import oracle
    import workloads as W
    T = oracle.default_threads()
    x = {name: W.draw_x(W.rng(999, i), 1, a.shape[1] * 32)[0]
         for i, (name, a) in enumerate(sample_aos.items())}
    bytes_pass = sum(gemv_bytes(a.shape[0], a.shape[1] * 32) for a in sample_aos.values())

    def leg(fn, budget):
        passes, t0 = 0, time.perf_counter()
        while True:
            fn()
            passes += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return bytes_pass * passes / el / 1e9, passes, el

    one = leg(lambda: [oracle.gemv(a, x[k], threads=1) for k, a in sample_aos.items()],
              0.4 * seconds)
    many = leg(lambda: [oracle.gemv(a, x[k], threads=T) for k, a in sample_aos.items()],
               0.3 * seconds)
    # numpy: dequantise each sample matrix to fp64 once (binary16 scale times
    # int8 quant), then time only the dense matvecs
    dense = {}
    for k, a in sample_aos.items():
        blk = np.ascontiguousarray(a, dtype=np.uint8)
        d = blk[:, :, 0:2].copy().view(np.float16)[:, :, 0].astype(np.float64)
        qv = blk[:, :, 2:34].view(np.int8).astype(np.float64)
        dense[k] = (qv * d[:, :, None]).reshape(a.shape[0], -1)
    xs = {k: v.astype(np.float64) for k, v in x.items()}
    nump = leg(lambda: [dense[k] @ xs[k] for k in dense], 0.3 * seconds)
    model = cpu_model()
    log(f"oracle: 1 thread {one[0]:.3f} GB/s, {T} threads {many[0]:.3f} GB/s; "
        f"numpy {nump[0]:.3f} GB/s on {model}")
    return {"value": round(many[0], 4), "unit": "GB/s", "cores": T, "kind": "oracle",
            "sample": (f"fp64 C oracle, layer-0 qkv/wo/gate_up/down + 16384 lm_head rows, "
                       f"{many[1]} passes in {many[2]:.1f} s on {T} threads"),
            "cpu_model": model,
            "one_thread": {"value": round(one[0], 4), "passes": one[1],
                           "seconds": round(one[2], 2)},
            "numpy_blas": {"value": round(nump[0], 4), "passes": nump[1],
                           "seconds": round(nump[2], 2),
                           "note": "numpy fp64 dense matvec on the dequantised sample "
                                   "(BLAS-backed second reference)"},
            "tok_per_s_equiv": round(many[0] * 1e9 / 527386624, 4)}


def source_hash(files):
    h = hashlib.sha256()
    for name in files:
        with open(os.path.join(ROOT, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, each scaled by what the counter reads
    for a plain copy of known size), when it was taken on the kernel's current
    sources; else None."""
    name = {"q8::chain_kernel": "chain_kernel_counters.json"}.get(kernel)
    if name is None:
        return None
    try:
        with open(os.path.join(ROOT, "profiles", name)) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel") != kernel or c.get("kernel_source_hash") != source_hash(
            c.get("kernel_sources", [])):
        return None
    return c.get("hbm_bytes_per_launch")


def context_rows(cfg, layers, lm_p, h0, steps, stream, log):
    """The decode step split and timed other ways, same weights: the 24
    layers alone as one persistent launch (no LM head), so the LM head's share
    is the difference; and the step as 97 dependent launches replayed from a
    HIP graph (M3)."""
    import torch
    import block_quantized_gemv_amd as q
    rows = []
    lay_bytes = len(layers) * sum(gemv_bytes(M, K) for (M, K) in SHAPES.values())
    pc = q.PersistentChain(layers, None, cfg.hidden, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim,
                           cfg.intermediate, cfg.eps)
    h_out = torch.empty(cfg.hidden, dtype=torch.float32, device=h0.device)
    s, rounds = time_launches(lambda: pc.run(h0, h_out=h_out, stream=stream), steps,
                              max(5, steps // 10), stream)
    if pc.status() != 0:
        raise RuntimeError(f"layers-only chain reported status {pc.status()}")
    med, mn, p90 = spread(rounds)
    rows.append({"row": "a7", "what": f"persistent chain, {len(layers)} layers, no LM head",
                 "mode": "M3", "us": round(s * 1e6, 2), "us_min": round(mn * 1e6, 2),
                 "us_p90": round(p90 * 1e6, 2), "us_median": round(med * 1e6, 2),
                 "rounds": len(rounds), "GBs": round(lay_bytes / s / 1e9, 1),
                 "us_per_layer": round(s * 1e6 / max(1, len(layers)), 3)})
    log(f"layers only: {s * 1e6:.1f} us ({s * 1e6 / max(1, len(layers)):.2f} us/layer)")
    del pc
    s, rounds, launches, _, tok = time_graph(cfg, layers, lm_p, h0, steps, max(5, steps // 10),
                                             stream, log)
    med, mn, p90 = spread(rounds)
    step_bytes = lay_bytes + gemv_bytes(cfg.vocab, cfg.hidden)
    rows.append({"row": "a7", "what": f"decode step as {launches} graph-replayed launches",
                 "mode": "M3", "us": round(s * 1e6, 2), "us_min": round(mn * 1e6, 2),
                 "us_p90": round(p90 * 1e6, 2), "us_median": round(med * 1e6, 2),
                 "rounds": len(rounds), "GBs": round(step_bytes / s / 1e9, 1), "token": tok})
    log(f"graph path: {s * 1e6:.1f} us/step, token {tok}")
    return rows


STAGE_POINTS = ("A start", "value/query/key task stored", "B start", "wo task stored",
                "C start", "last gate-up task stored (first wave)",
                "first gate-up task stored (last wave)", "D start", "down partial stored",
                "8 partials received", "h2 rows stored", "next h staged",
                "value/query/key weights in registers", "gate-up weights in registers",
                "value/query/key dot product done", "gate-up dot product done")


def stage_breakdown(cfg, layers, lm_p, h0, runs, log):
    """The persistent step with stage timestamps: for every stamped point of a
    layer, the median over workgroups of its time after that layer's stage-A
    barrier, averaged over the middle layers and over `runs` steps; plus the
    LM head's share and the stamped step time (HIP events)."""
    import torch
    import block_quantized_gemv_amd as q
    pc = q.PersistentChain(layers, lm_p, cfg.hidden, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim,
                           cfg.intermediate, cfg.eps)
    dev = h0.device
    G, Wd = pc.plan.grid, q.Q8_CHAIN_STAMP_WORDS
    LP, KP = q.Q8_CHAIN_STAMP_LAYERS, q.Q8_CHAIN_STAMP_POINTS
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device=dev)
    tok = torch.empty(1, dtype=torch.int32, device=dev)
    stamps = torch.zeros(G * Wd, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()
    plain, _ = time_launches(lambda: pc.run(h0, logits, tok, stream=stream), 50, 10, stream)
    stamped, _ = time_launches(lambda: pc.run(h0, logits, tok, stream=stream, stamps=stamps), 50,
                               10, stream)
    L = min(len(layers), LP)
    mids = range(1, max(2, L - 1))
    acc = np.zeros((runs, KP))
    lm = np.zeros((runs, 3))
    for r in range(runs):
        stamps.zero_()
        pc.run(h0, logits, tok, stream=stream, stamps=stamps)
        torch.cuda.synchronize()
        t = stamps.cpu().numpy().reshape(G, Wd).astype(np.float64) * 0.01  # us
        lay = t[:, :LP * KP].reshape(G, LP, KP)
        for k in range(KP):
            vals = []
            for l in mids:
                base = lay[:, l, 0]
                have = lay[:, l, k] > 0
                vals.append(np.median(lay[have, l, k] - base[have]) if have.any() else np.nan)
            acc[r, k] = np.nanmean(vals)
        kern = t[:, LP * KP:]
        lm[r] = [np.median(kern[:, 1] - kern[:, 0]), np.median(kern[:, 3] - kern[:, 1]),
                 np.median(kern[:, 1] - lay[:, L - 1, 0])]
    if int(tok.cpu()[0]) < 0 or pc.status() != 0:
        raise RuntimeError("stamped step reported an invalid token")
    med = np.median(acc, axis=0)
    period = np.median([np.median(lay[:, l + 1, 0] - lay[:, l, 0]) for l in mids])
    out = {"step_us": round(plain * 1e6, 2), "stamped_step_us": round(stamped * 1e6, 2),
           "layer_period_us": round(float(period), 3),
           "points_us_after_A": {STAGE_POINTS[k]: round(float(med[k]), 3) for k in range(KP)},
           "layers_us": round(float(np.median(lm[:, 0])), 2),
           "lm_head_us": round(float(np.median(lm[:, 1])), 2),
           "last_layer_to_lm_us": round(float(np.median(lm[:, 2])), 2),
           "layers_averaged": f"{mids.start}..{mids.stop - 1}", "runs": runs}
    log(f"stamped step {out['stamped_step_us']} us (plain {out['step_us']} us); "
        f"layer period {out['layer_period_us']} us")
    for name, v in out["points_us_after_A"].items():
        log(f"  {v:7.2f} us  {name}")
    return out


def main():
    args = parse()
    log = lambda m: print(f"[bench] {m}", file=sys.stderr, flush=True)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by output rows; see the design notes)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        a = torch.empty(args.calibrate_copy, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"copied {args.calibrate_copy} bytes 5 times")
        return
    if args.only:
        rows = measure_rows(log, tuple(s for s in args.only.split(",") if s))
        print(json.dumps({"rows": rows}), flush=True)
        return
    cfg, layers, lm_p, h0, step_bytes, sample_aos = build_weights(args.layers, log)
    if args.stages:
        print(json.dumps({"stages": stage_breakdown(cfg, layers, lm_p, h0, args.stages, log)}),
              flush=True)
        return
    stream = torch.cuda.current_stream()
    timer = time_persistent if args.path == "persistent" else time_graph
    sec, rounds, launches, kernel, tok = timer(cfg, layers, lm_p, h0, args.steps, args.warmup,
                                               stream, log)
    ms = sec * 1e3
    gbs = step_bytes / sec / 1e9
    med, mn, p90 = spread(rounds)
    log(f"{args.path}: {args.steps} steps, {ms * 1e3:.1f} us/step (rounds: median "
        f"{med * 1e6:.1f}, min {mn * 1e6:.1f}, p90 {p90 * 1e6:.1f}), {1e3 / ms:.1f} tok/s, "
        f"{gbs:.1f} GB/s, token {tok}")
    per_launch_bytes = step_bytes / launches
    per_launch_s = sec / launches
    achieved = per_launch_bytes / per_launch_s / 1e9
    traffic = committed_traffic(kernel)
    workload = ("Qwen2.5-0.5B-shaped Q8_0 decode matmul chain, N=1: 24 layers x (qkv 1152x896, "
                "wo 896x896, gate_up 9728x896 + SwiGLU, down 896x4864) + lm_head 151936x896 + "
                "argmax, glue fused, " + ("one persistent launch per token"
                                          if args.path == "persistent" else
                                          "97 launches replayed from a HIP graph"))
    out = {
        "metric": "Q8_0 GEMV achieved HBM GB/s (% of MI355X peak) + decode matmul-chain tok/s",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "tok_per_s": round(1e3 / ms, 2),
        "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
        "step_rounds_us": {"median": round(med * 1e6, 2), "min": round(mn * 1e6, 2),
                           "p90": round(p90 * 1e6, 2), "rounds": len(rounds)},
        "config": {"workload": workload, "path": args.path,
                   "layers": args.layers, "launches_per_step": launches,
                   "bytes_per_step": int(step_bytes), "weights": "q8_0 (1.0625 B/weight)",
                   "activations": "fp32"},
        "roofline": {"bound": "hbm", "kernel": kernel,
                     "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic,
                     "bytes_per_launch": int(per_launch_bytes),
                     "avg_launch_us": round(per_launch_s * 1e6, 3)},
        "context": None,
        "rows": None,
        "cpu_baseline": None,
    }
    if not args.no_rows and args.path == "persistent":
        out["context"] = context_rows(cfg, layers, lm_p, h0, max(20, args.steps // 2), stream,
                                      log)
    del layers, lm_p
    torch.cuda.empty_cache()
    if not args.no_rows:
        out["rows"] = measure_rows(log)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(sample_aos, args.cpu_seconds, log)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
