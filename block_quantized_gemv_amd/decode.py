"""Decode matmul chain of a Qwen2-style decoder on the Q8_0 GEMV library.

One decode step at position 0 ("augur" README, "Features": decoder block
order norm, attention, residual, norm, MLP, residual; final norm and LM head;
greedy pick), with every non-matmul step folded into the GEMVs through
q8_0_gemv_fused, so a step is 4 launches per layer plus one for the LM head:

    qkv  = Wqkv . rmsnorm(h)                       prologue RMSNORM
    h    = h + Wo . gqa(v)                         prologue GQA, epilogue RESIDUAL
    s    = swiglu(Wgu . rmsnorm(h))                prologue RMSNORM, epilogue SWIGLU
    h    = h + Wdown . s                           epilogue RESIDUAL
    ...  x n_layers
    logits = Wlm . rmsnorm(h); next = argmax       prologue RMSNORM, epilogue ARGMAX

Layer 0 reads the input hidden state h0 and writes h (its wo call uses h0 as
the residual), so a captured step needs no copy node.  Norm weights are 1
and there are no biases; with a single key the attention softmax weight is
1, so each query head outputs its key/value head's value vector.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import (PackedQ8, Q8_EPI_ARGMAX, Q8_EPI_RESIDUAL, Q8_EPI_SWIGLU, Q8_OP_GEMV_FUSED,
               Q8_PRO_GQA, Q8_PRO_RMSNORM, Q8Error, lib, make_fusion, q8_0_workspace_bytes)


@dataclass
class ChainConfig:
    hidden: int = 896
    n_heads: int = 14
    n_kv_heads: int = 2
    head_dim: int = 64
    intermediate: int = 4864
    vocab: int = 151936
    eps: float = 1e-6

    @property
    def qkv_rows(self) -> int:
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim


class DecodeChain:
    """Preallocated buffers and pre-built call arguments for one decode step.

    layers: list of dicts with PackedQ8 entries "qkv", "wo", "gate_up", "down".
    """

    def __init__(self, cfg: ChainConfig, layers: list, lm_head: PackedQ8, device=None):
        self.cfg, self.layers, self.lm_head = cfg, layers, lm_head
        dev = device or lm_head.qs.device
        f32 = dict(dtype=torch.float32, device=dev)
        self.h = torch.empty(cfg.hidden, **f32)
        self.qkv = torch.empty(cfg.qkv_rows, **f32)
        self.s = torch.empty(cfg.intermediate, **f32)
        self.logits = torch.empty(cfg.vocab, **f32)
        self.next_token = torch.zeros(1, dtype=torch.int32, device=dev)
        need = 0
        for L in layers:
            need = max(need,
                       q8_0_workspace_bytes(Q8_OP_GEMV_FUSED, L["qkv"].M, L["qkv"].K, 0),
                       q8_0_workspace_bytes(Q8_OP_GEMV_FUSED, L["wo"].M, L["wo"].K,
                                            Q8_EPI_RESIDUAL),
                       q8_0_workspace_bytes(Q8_OP_GEMV_FUSED, L["gate_up"].M, L["gate_up"].K,
                                            Q8_EPI_SWIGLU),
                       q8_0_workspace_bytes(Q8_OP_GEMV_FUSED, L["down"].M, L["down"].K,
                                            Q8_EPI_RESIDUAL))
        need = max(need, q8_0_workspace_bytes(Q8_OP_GEMV_FUSED, lm_head.M, lm_head.K,
                                              Q8_EPI_ARGMAX))
        # calls are stream-ordered and each leaves its counters at zero, so one
        # zero-filled workspace serves the whole chain
        self.ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
        self.h0 = torch.empty(cfg.hidden, **f32)
        self._calls = None

    def _build_calls(self):
        c = self.cfg
        f_norm = make_fusion(prologue=Q8_PRO_RMSNORM, eps=c.eps)
        f_o0 = make_fusion(prologue=Q8_PRO_GQA, epilogue=Q8_EPI_RESIDUAL, n_heads=c.n_heads,
                           n_kv_heads=c.n_kv_heads, head_dim=c.head_dim,
                           gqa_offset=(c.n_heads + c.n_kv_heads) * c.head_dim, residual=self.h0)
        f_o = make_fusion(prologue=Q8_PRO_GQA, epilogue=Q8_EPI_RESIDUAL, n_heads=c.n_heads,
                          n_kv_heads=c.n_kv_heads, head_dim=c.head_dim,
                          gqa_offset=(c.n_heads + c.n_kv_heads) * c.head_dim, residual=self.h)
        f_gu = make_fusion(prologue=Q8_PRO_RMSNORM, epilogue=Q8_EPI_SWIGLU, eps=c.eps)
        f_dn = make_fusion(epilogue=Q8_EPI_RESIDUAL, residual=self.h)
        f_lm = make_fusion(prologue=Q8_PRO_RMSNORM, epilogue=Q8_EPI_ARGMAX, eps=c.eps,
                           argmax_out=self.next_token)
        self._fusions = [f_norm, f_o0, f_o, f_gu, f_dn, f_lm]
        h, h0, qkv, s = self.h.data_ptr(), self.h0.data_ptr(), self.qkv.data_ptr(), self.s.data_ptr()
        calls = []
        for i, L in enumerate(self.layers):
            calls.append((L["qkv"], h0 if i == 0 else h, qkv, f_norm))
            calls.append((L["wo"], qkv, h, f_o0 if i == 0 else f_o))
            calls.append((L["gate_up"], h, s, f_gu))
            calls.append((L["down"], s, h, f_dn))
        calls.append((self.lm_head, h0 if not self.layers else h, self.logits.data_ptr(), f_lm))
        self._calls = [(ctypes.byref(W.desc), x, y, W.M, W.K, ctypes.byref(f)) for (W, x, y, f) in
                       calls]

    def enqueue(self, stream=None) -> None:
        """Enqueue one decode step reading self.h0; results in self.h,
        self.logits and self.next_token."""
        if self._calls is None:
            self._build_calls()
        s = (stream or torch.cuda.current_stream()).cuda_stream
        L = lib()
        ws, wsb = self.ws.data_ptr(), self.ws.numel()
        for (w, x, y, M, K, f) in self._calls:
            rc = L.q8_0_gemv_fused(w, x, y, M, K, f, ws, wsb, s)
            if rc:
                raise Q8Error("q8_0_gemv_fused", rc)

    def run_layer_calls(self, stream=None):
        """Yield after each call (for stage-wise checks): (index, call kind)."""
        if self._calls is None:
            self._build_calls()
        s = (stream or torch.cuda.current_stream()).cuda_stream
        L = lib()
        kinds = ["qkv", "wo", "gate_up", "down"] * len(self.layers) + ["lm_head"]
        for i, ((w, x, y, M, K, f), kind) in enumerate(zip(self._calls, kinds)):
            rc = L.q8_0_gemv_fused(w, x, y, M, K, f, self.ws.data_ptr(), self.ws.numel(), s)
            if rc:
                raise Q8Error("q8_0_gemv_fused", rc)
            yield i, kind

    def capture(self) -> torch.cuda.CUDAGraph:
        """Capture one step into a HIP graph (all buffers are fixed)."""
        if self._calls is None:
            self._build_calls()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.enqueue(side)  # warm-up outside the capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            self.enqueue()
        return g
