"""Benchmark: the Q8_0 decode matmul chain of a Qwen2.5-0.5B-shaped decoder on
one MI355X.

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
               GEMV) over the timed region; tok/s alongside
  roofline     the step's kernel: algorithmic bytes per launch / average
               launch duration, from HIP events on the launch stream
  rows         every kernel of the path on its own workload (C1..C5 shapes),
               graph-timed over rotating cold weight copies (>1 GB)
  cpu_baseline the fp64 oracle timed on this host on a bounded sample

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--path persistent|graph]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E


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
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-clock budget of the oracle CPU baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the per-kernel measurements of every workload")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes 5 times (the reference "
                         "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE) and exit")
    return ap.parse_args()


SHAPES = {"qkv": (1152, 896), "wo": (896, 896), "gate_up": (9728, 896), "down": (896, 4864)}


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


def time_launches(launch, steps, warmup, stream):
    """Average time of one `launch()` over `steps` back-to-back launches,
    from HIP events recorded on the stream the kernels run on."""
    import torch
    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / steps


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
        f"LDS {pc.plan.lds_bytes} B, workspace {pc.plan.ws_bytes} B")
    s = time_launches(lambda: pc.run(h0, logits, tok, h_out, stream=stream), steps, warmup,
                      stream)
    status = pc.status()
    if status != 0:
        raise RuntimeError(f"persistent chain reported status {status}")
    return s, 1, "q8::chain_kernel", int(tok.cpu()[0])


def time_graph(cfg, layers, lm_p, h0, steps, warmup, stream, log):
    from block_quantized_gemv_amd.decode import DecodeChain
    chain = DecodeChain(cfg, layers, lm_p)
    chain.h0.copy_(h0)
    g = chain.capture()
    s = time_launches(g.replay, steps, warmup, stream)
    return s, 4 * len(layers) + 1, "q8::gemv_kernel<1>", int(chain.next_token.cpu()[0])


def graph_time(enqueue, n_calls, replays=5):
    """Seconds per call of `enqueue(i)` (i < n_calls), captured once into a
    HIP graph and replayed; HIP events on the replay stream bracket the
    replays, so host launch overhead is excluded and each call's dispatch
    latency (about 1.6 us per graph node) is included."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(min(n_calls, 2)):
            enqueue(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for i in range(n_calls):
            enqueue(i)
    g.replay()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(replays):
        g.replay()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / replays / n_calls


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


def measure_rows(log, cold_bytes=1.2e9):
    """Every kernel of the path on its own workload, graph-timed over rotating
    cold weight copies (more than `cold_bytes` in rotation, beyond the 256 MB
    Infinity Cache): C1 896x896; the 0.5B layer shapes; lm_head with the fused
    RMSNorm/argmax and the standalone argmax; the 9B-class shapes at N = 1, 2,
    4, 8; the integer-activation variant on the 9B gate_up shape; Q4_K,
    Q5_K and Q6_K weights on the 9B shapes; the
    verify-chunk LM head with one argmax per column; the
    Qwen1.5-MoE-shaped FFN (router, scatter + SwiGLU, combine)."""
    import torch
    import block_quantized_gemv_amd as q
    import workloads as W
    dev = torch.device("cuda", 0)
    gen = torch.Generator(device=dev).manual_seed(1234)
    rows = []

    def rec(row, what, sec, nbytes):
        r = {"row": row, "what": what, "us": round(sec * 1e6, 2)}
        if nbytes:
            gbs = nbytes / sec / 1e9
            r.update(GBs=round(gbs, 1), frac=round(gbs / PEAK_HBM_GBS, 4))
        rows.append(r)
        log(f"{row} {what}: {sec * 1e6:.2f} us" + (f", {r['GBs']} GB/s" if nbytes else ""))

    def gemv_row(row, M, K, N, what, epi=None):
        n = max(2, min(64, int(cold_bytes // (1.0625 * M * K)) + 1))
        Wm = rand_packed(M, K, n, gen)
        qb, db = q.q8_0_packed_size(M, K)
        views = [q.PackedQ8(Wm.qs[i * qb:(i + 1) * qb], Wm.d[i * db:(i + 1) * db], M, K)
                 for i in range(n)]
        x = torch.randn(N, K, device=dev, generator=gen)
        y = torch.empty(N, M, device=dev)
        if epi is None:
            ws = q.Workspace(q.q8_0_workspace_bytes(q.Q8_OP_GEMV, M, K, N))
            sec = graph_time(lambda i: q.q8_0_gemv(views[i % n], x, y, ws), n)
        elif epi in ("q8act", "q8act+quant"):
            # integer activations: codes + binary16 scales replace the fp32 vector
            qx, dx = q.q8_0_quantize_act(x)
            ws = q.Workspace(q.q8_0_workspace_bytes(q.Q8_OP_GEMV, M, K, N))
            if epi == "q8act":
                call = lambda i: q.q8_0_gemv_q8act(views[i % n], qx, dx, y, ws)
            else:
                def call(i):
                    q.q8_0_quantize_act(x, qx, dx)
                    q.q8_0_gemv_q8act(views[i % n], qx, dx, y, ws)
            sec = graph_time(call, n)
            rec(row, what, sec, 1.0625 * M * K + 1.0625 * K * N + 4 * M * N)
            del views, Wm
            torch.cuda.empty_cache()
            return
        elif epi == "col_argmax":
            am = torch.empty(N, dtype=torch.int32, device=dev)
            ws = q.Workspace(q.q8_0_workspace_bytes(q.Q8_OP_GEMV_ARGMAX, M, K, N))
            sec = graph_time(lambda i: q.q8_0_gemv_argmax(views[i % n], x, y, am, ws), n)
        else:
            tok = torch.empty(1, dtype=torch.int32, device=dev)
            fus = q.make_fusion(q.Q8_PRO_RMSNORM, q.Q8_EPI_ARGMAX, 1e-6, argmax_out=tok)
            ws = q.Workspace(q.q8_0_workspace_bytes(q.Q8_OP_GEMV_FUSED, M, K, q.Q8_EPI_ARGMAX))
            sec = graph_time(lambda i: q.q8_0_gemv_fused(views[i % n], x[0], y[0], fus, ws), n)
        rec(row, what, sec, gemv_bytes(M, K, N))
        del views, Wm
        torch.cuda.empty_cache()

    # context: what plain torch kernels reach on this device (read-reduce, copy)
    big = torch.empty(1 << 29, dtype=torch.float32, device=dev).uniform_(generator=gen)
    dst = torch.empty_like(big)
    sink = torch.empty((), device=dev)
    st = torch.cuda.current_stream()
    rec("hbm", "torch sum over 2 GiB fp32 (read)",
        time_launches(lambda: torch.sum(big, dim=0, out=sink), 5, 2, st), big.numel() * 4)
    rec("hbm", "torch copy of 2 GiB (read + write)",
        time_launches(lambda: dst.copy_(big), 5, 2, st), big.numel() * 8)
    del big, dst
    torch.cuda.empty_cache()
    gemv_row("a2", 896, 896, 1, "C1 gemv 896x896")
    for name, (M, K) in SHAPES.items():
        gemv_row("a2", M, K, 1, f"C2 {name} {M}x{K}")
    gemv_row("a2", 151936, 896, 1, "C3 lm_head 151936x896")
    gemv_row("a4", 151936, 896, 1, "C3 lm_head 151936x896 + RMSNorm + argmax", epi="argmax")
    v = torch.randn(151936, device=dev, generator=gen)
    out = torch.empty(1, dtype=torch.int32, device=dev)
    ws = q.Workspace(q.q8_0_workspace_bytes(q.Q8_OP_ARGMAX, v.numel(), 0, 0))
    rec("a4", "argmax over 151936 fp32 logits", graph_time(lambda i: q.q8_0_argmax(v, out, ws), 32),
        4 * v.numel())
    for N in (1, 2, 4, 8):
        gemv_row("a3" if N > 1 else "a2", 24576, 4096, N, f"C4 gate_up 24576x4096 N={N}")
        gemv_row("a3" if N > 1 else "a2", 4096, 12288, N, f"C4 down 4096x12288 N={N}")
    for N in (1, 8):
        gemv_row("f3", 24576, 4096, N, f"C4 gate_up 24576x4096 N={N}, int8 activations",
                 epi="q8act")
    gemv_row("f3", 24576, 4096, 8, "C4 gate_up 24576x4096 N=8, quantize + int8 activations",
             epi="q8act+quant")
    # Q4_K weights (NEXT-2) on the same 9B-class shapes
    for (M, K) in ((24576, 4096), (4096, 12288)):
        for N in (1, 8):
            n = max(2, min(64, int(cold_bytes // (0.5625 * M * K)) + 1))
            qs, meta, qb, mb = rand_packed_q4k(M, K, n, gen)
            views = [q.PackedQ4K(qs[i * qb:(i + 1) * qb], meta[i * mb:(i + 1) * mb], M, K)
                     for i in range(n)]
            x = torch.randn(N, K, device=dev, generator=gen)
            y = torch.empty(N, M, device=dev)
            ws = q.Workspace(q.q8_0_workspace_bytes(q.Q8_OP_Q4K_GEMV, M, K, N))
            sec = graph_time(lambda i: q.q4k_gemv(views[i % n], x, y, ws), n)
            rec("n2", f"C4-shaped {M}x{K} Q4_K N={N}", sec,
                0.5625 * M * K + 4 * K * N + 4 * M * N)
            del views, qs, meta
            torch.cuda.empty_cache()
    # Q5_K weights (NEXT-2); algorithmic bytes are GGUF's 176 per 256 weights
    for (M, K) in ((24576, 4096), (4096, 12288)):
        for N in (1, 8):
            n = max(2, min(64, int(cold_bytes // (0.6875 * M * K)) + 1))
            qs, qh, meta, (a, b, c) = rand_packed_q5k(M, K, n, gen)
            views = [q.PackedQ5K(qs[i * a:(i + 1) * a], qh[i * b:(i + 1) * b],
                                 meta[i * c:(i + 1) * c], M, K) for i in range(n)]
            x = torch.randn(N, K, device=dev, generator=gen)
            y = torch.empty(N, M, device=dev)
            ws = q.Workspace(q.q8_0_workspace_bytes(q.Q8_OP_Q5K_GEMV, M, K, N))
            sec = graph_time(lambda i: q.q5k_gemv(views[i % n], x, y, ws), n)
            rec("n2", f"C4-shaped {M}x{K} Q5_K N={N}", sec,
                176 / 256 * M * K + 4 * K * N + 4 * M * N)
            del views, qs, qh, meta
            torch.cuda.empty_cache()
    # Q6_K weights (NEXT-2); algorithmic bytes are GGUF's 210 per 256 weights
    for (M, K) in ((4096, 12288), (24576, 4096)):
        for N in (1, 8):
            n = max(2, min(64, int(cold_bytes // (0.875 * M * K)) + 1))
            ql, qh, meta, (a, b, c) = rand_packed_q6k(M, K, n, gen)
            views = [q.PackedQ6K(ql[i * a:(i + 1) * a], qh[i * b:(i + 1) * b],
                                 meta[i * c:(i + 1) * c], M, K) for i in range(n)]
            x = torch.randn(N, K, device=dev, generator=gen)
            y = torch.empty(N, M, device=dev)
            ws = q.Workspace(q.q8_0_workspace_bytes(q.Q8_OP_Q6K_GEMV, M, K, N))
            sec = graph_time(lambda i: q.q6k_gemv(views[i % n], x, y, ws), n)
            rec("n2", f"C4-shaped {M}x{K} Q6_K N={N}", sec,
                210 / 256 * M * K + 4 * K * N + 4 * M * N)
            del views, ql, qh, meta
            torch.cuda.empty_cache()
    for N in (2, 8):
        gemv_row("f4", 151936, 896, N, f"lm_head 151936x896 N={N} + argmax per column (2 launches)",
                 epi="col_argmax")

    # Qwen1.5-MoE-shaped FFN, one token per call, routing from seeded N(0,1) logits
    E, H, I, Ish, S, T, NSH = 60, 2048, 1408, 5632, 4, 32, 8
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
    ws1 = q.Workspace(q.q8_0_workspace_bytes(q.Q8_OP_MOE_SCATTER, 2 * I, H, S, 2 * Ish, H, mode_s))
    ws2 = q.Workspace(q.q8_0_workspace_bytes(q.Q8_OP_MOE_COMBINE, H, I, S, H, Ish, q.Q8_MOE_COMBINE))
    route = lambda t: q.q8_0_route_topk(logits[t], S, ids[t], w[t])
    scatter = lambda t: q.q8_0_moe_gemv(gu, ids[t], None, x[t], h[t], mode_s, shared=sgu[t % NSH],
                                        workspace=ws1)
    combine = lambda t: q.q8_0_moe_gemv(dn, ids[t], w[t], h[t], y[t], q.Q8_MOE_COMBINE,
                                        shared=sdn[t % NSH], shared_gate=lam[t:t + 1],
                                        workspace=ws2)
    for t in range(T):
        route(t)
    torch.cuda.synchronize()
    bs = S * gemv_bytes(2 * I, H) + gemv_bytes(2 * Ish, H)
    bc = S * gemv_bytes(H, I) + gemv_bytes(H, Ish)
    rec("a5", "C5 router top-4 of 60", graph_time(route, T), 0)
    rec("a6", "C5 scatter: 4 slots gate_up 2816x2048 + shared 11264x2048 + SwiGLU",
        graph_time(scatter, T), bs)
    rec("a8", "C5 combine: 4 slots down 2048x1408 + shared 2048x5632, weighted",
        graph_time(combine, T), bc)
    rec("a5-a8", "C5 MoE FFN token: router + scatter + combine",
        graph_time(lambda t: (route(t), scatter(t), combine(t)), T), bs + bc)
    del gu, dn, sgu, sdn
    torch.cuda.empty_cache()
    return rows


def cpu_baseline(sample_aos, cfg, seconds, log):
    """The oracle as it stands, on this host's cores, over a bounded sample of
    the same workload: layer 0's four GEMVs plus 16384 LM-head rows, repeated
    until the time budget is spent.  Reported in the metric's unit."""
    import oracle
    import workloads as W
    threads = oracle.default_threads()
    x = {name: W.draw_x(W.rng(999, i), 1, a.shape[1] * 32)[0]
         for i, (name, a) in enumerate(sample_aos.items())}
    bytes_pass = sum(gemv_bytes(a.shape[0], a.shape[1] * 32) for a in sample_aos.values())
    passes, t0 = 0, time.perf_counter()
    while True:
        for name, a in sample_aos.items():
            oracle.gemv(a, x[name], threads=threads)
        passes += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    gbs = bytes_pass * passes / el / 1e9
    log(f"oracle: {passes} passes in {el:.1f} s on {threads} threads -> {gbs:.3f} GB/s")
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": (f"fp64 C oracle, layer-0 qkv/wo/gate_up/down + 16384 lm_head rows, "
                       f"{passes} passes in {el:.1f} s"),
            "tok_per_s_equiv": round(gbs * 1e9 / 527386624, 4)}


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
    cfg, layers, lm_p, h0, step_bytes, sample_aos = build_weights(args.layers, log)
    stream = torch.cuda.current_stream()
    timer = time_persistent if args.path == "persistent" else time_graph
    sec, launches, kernel, tok = timer(cfg, layers, lm_p, h0, args.steps, args.warmup, stream,
                                       log)
    ms = sec * 1e3
    gbs = step_bytes / sec / 1e9
    log(f"{args.path}: {args.steps} steps, {ms * 1e3:.1f} us/step, {1e3 / ms:.1f} tok/s, "
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
        "rows": None,
        "cpu_baseline": None,
    }
    del layers, lm_p
    if not args.no_rows:
        out["rows"] = measure_rows(log)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(sample_aos, cfg, args.cpu_seconds, log)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
