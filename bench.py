"""Benchmark: the Q8_0 decode matmul chain of a Qwen2.5-0.5B-shaped decoder on
one MI355X.

A step is one decode token through the whole hot path: 24 layers of fused
Q8_0 GEMVs (qkv 1152x896 with the RMSNorm prologue, wo 896x896 with the GQA
prologue and residual epilogue, gate_up 9728x896 with RMSNorm and SwiGLU,
down 896x4864 with the residual epilogue), then the LM head 151936x896 with
the RMSNorm prologue and the argmax epilogue: 97 launches, captured once in a
HIP graph and replayed.  Weights are synthetic and seeded (quants uniform in
[-127, 127], scales |N(0,1)|*0.01 in binary16, h0 ~ N(0,1)); 527 MB of
weights per step exceed the 256 MB Infinity Cache, so replays stream from HBM.

Prints one JSON line:
  value        algorithmic HBM GB/s of the step (1.0625 B/weight + x + y per
               GEMV) over the timed region; tok/s alongside
  roofline     the GEMV kernel (the only kernel of the step): algorithmic bytes
               per launch / average launch duration over the timed region
  cpu_baseline the fp64 oracle timed on this host on a bounded sample

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
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
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-clock budget of the oracle CPU baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes 5 times (the reference "
                         "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE) and exit")
    return ap.parse_args()


def build_chain(n_layers, log):
    import torch
    import block_quantized_gemv_amd as q
    import workloads as W
    from block_quantized_gemv_amd.decode import ChainConfig, DecodeChain

    cfg = ChainConfig()
    dev = torch.device("cuda", 0)
    shapes = {W.MAT_QKV: ("qkv", cfg.qkv_rows, cfg.hidden), W.MAT_WO: ("wo", cfg.hidden, cfg.hidden),
              W.MAT_GATE_UP: ("gate_up", 2 * cfg.intermediate, cfg.hidden),
              W.MAT_DOWN: ("down", cfg.hidden, cfg.intermediate)}
    layers, sample_aos = [], {}
    t0 = time.time()
    for l in range(n_layers):
        L = {}
        for mat, (name, M, K) in shapes.items():
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
    torch.cuda.synchronize()
    log(f"weights generated and repacked in {time.time() - t0:.1f} s")
    chain = DecodeChain(cfg, layers, lm_p)
    chain.h0.copy_(torch.from_numpy(W.activations(W.C2["cfg"], 1, cfg.hidden)[0]).to(dev))
    step_bytes = n_layers * sum(gemv_bytes(M, K) for (_, M, K) in shapes.values())
    step_bytes += gemv_bytes(cfg.vocab, cfg.hidden)
    launches = 4 * n_layers + 1
    return chain, cfg, step_bytes, launches, sample_aos


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


def kernel_source_hash():
    h = hashlib.sha256()
    for name in sorted(os.listdir(os.path.join(ROOT, "block_quantized_gemv_amd", "csrc"))):
        with open(os.path.join(ROOT, "block_quantized_gemv_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def committed_traffic(launches):
    """HBM bytes per launch from the committed rocprofv3 counter summary, when
    it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "chain_counters.json")
    try:
        with open(path) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_hash") != kernel_source_hash():
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
    chain, cfg, step_bytes, launches, sample_aos = build_chain(args.layers, log)
    stream = torch.cuda.current_stream()
    g = chain.capture()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    gbs = step_bytes / (ms * 1e-3) / 1e9
    log(f"{args.steps} steps: {ms * 1e3:.1f} us/step, {1e3 / ms:.1f} tok/s, {gbs:.1f} GB/s")
    per_launch_bytes = step_bytes / launches
    per_launch_s = ms * 1e-3 / launches
    achieved = per_launch_bytes / per_launch_s / 1e9
    traffic = committed_traffic(launches)
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
        "config": {"workload": "Qwen2.5-0.5B-shaped Q8_0 decode matmul chain, N=1: 24 layers x "
                               "(qkv 1152x896, wo 896x896, gate_up 9728x896 + SwiGLU, down "
                               "896x4864) + lm_head 151936x896 + argmax, glue fused, HIP graph",
                   "layers": args.layers, "launches_per_step": launches,
                   "bytes_per_step": int(step_bytes), "weights": "q8_0 (1.0625 B/weight)",
                   "activations": "fp32"},
        "roofline": {"bound": "hbm", "kernel": "q8::gemv_kernel<1>",
                     "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic,
                     "bytes_per_launch": int(per_launch_bytes),
                     "avg_launch_us": round(per_launch_s * 1e6, 3)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(sample_aos, cfg, args.cpu_seconds, log)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
