"""Seeded synthetic inputs for the Q8_0 decode path.

This module is shared by the CPU oracle tests, the GPU parity tests and the
benchmark.  It draws numbers and lays them out in the GGUF Q8_0 block format;
it performs none of the method's arithmetic (no dequantisation, no dot
products), so neither side of a parity comparison borrows anything from the
other through it.

Block format (GGUF Q8_0, as named on the cogni-ml page, section "Qwen 3.5
Native Metal" / cuda_q8_gemv_probe "raw GGUF Q8_0 block layout"): each block
covers 32 consecutive weights of one row and is 34 bytes: a little-endian
IEEE binary16 scale d followed by 32 signed 8-bit quants.  Blocks of a row are
consecutive, rows are consecutive.

Value distributions (of the benchmarked and tested workloads):
  quants  discrete uniform in [-127, 127], both ends inclusive
  scales  |N(0,1)| * 0.01, rounded to binary16 (round-to-nearest-even)
  x       N(0,1) in float32, shape [N][K]
Generator: numpy PCG64 seeded by SeedSequence([cfg, layer, mat]).
"""
from __future__ import annotations

import dataclasses

import numpy as np

QK = 32           # weights per block
BLOCK_BYTES = 34  # 2-byte scale + 32 quants

# Matrix ids inside a configuration's seed sequence.
MAT_QKV, MAT_WO, MAT_GATE_UP, MAT_DOWN, MAT_LM_HEAD = 0, 1, 2, 3, 4
MAT_X = 100
MAT_ROUTER = 101
MAT_SHARED_GATE = 102
MAT_SHARED_GU, MAT_SHARED_DOWN = 103, 104


def rng(cfg: int, layer: int = 0, mat: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg, layer, mat])))


@dataclasses.dataclass
class Q8Matrix:
    """A Q8_0 matrix as drawn: quants [M][K] int8, scales [M][K/32] float16."""
    qs: np.ndarray
    d: np.ndarray

    @property
    def M(self) -> int:
        return self.qs.shape[0]

    @property
    def K(self) -> int:
        return self.qs.shape[1]

    def aos(self) -> np.ndarray:
        """GGUF array-of-blocks bytes, shape [M, K/32, 34] uint8."""
        return encode_aos(self.qs, self.d)


def encode_aos(qs: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Lay quants and binary16 scales out as GGUF 34-byte blocks."""
    qs = np.ascontiguousarray(qs, dtype=np.int8)
    d = np.ascontiguousarray(d, dtype=np.float16)
    M, K = qs.shape
    if K % QK:
        raise ValueError("K must be a multiple of 32")
    B = K // QK
    if d.shape != (M, B):
        raise ValueError("scale shape must be [M, K/32]")
    out = np.empty((M, B, BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = d.view(np.uint8).reshape(M, B, 2)  # little-endian host
    out[:, :, 2:] = qs.view(np.uint8).reshape(M, B, QK)
    return out


def draw_matrix(g: np.random.Generator, M: int, K: int) -> Q8Matrix:
    """Quants first, then scales, from one generator (fixed draw order)."""
    qs = g.integers(-127, 128, size=(M, K), dtype=np.int8)
    d = (np.abs(g.standard_normal((M, K // QK))) * 0.01).astype(np.float16)
    return Q8Matrix(qs, d)


# --------------------------------------------------------------------------
# Q4_K (GGUF k-quant, named on the cogni-ml page, "Qwen 3.5 Native Metal" /
# cuda_q4k_gemv_probe: d, dmin, 12-byte packed scales/mins, 128-byte packed
# nibbles).  A 144-byte block holds 256 weights of one row as 8 sub-blocks of
# 32, each with a 6-bit scale s and a 6-bit min m.  The byte arrangement (the
# GGUF one):
#   [0:2] d, [2:4] dmin (binary16, little-endian)
#   [4:16] sc: for j < 4, sc[j] low 6 bits = s_j, sc[j+4] low 6 bits = m_j;
#          for j >= 4, sc[j+4] = (s_j & 15) | (m_j & 15) << 4, and the top
#          two bits of sc[j-4] and sc[j] hold s_j >> 4 and m_j >> 4
#   [16:144] qs: weight k's 4-bit quant in byte 32 (k // 64) + k % 32, low
#          nibble when k % 64 < 32, high nibble otherwise.
# Value distributions: quants uniform 0..15, s and m uniform 0..63,
# d = |N(0,1)| * 0.001 and dmin = |N(0,1)| * 0.004 as binary16.
# --------------------------------------------------------------------------
QKK = 256
Q4K_BYTES = 144


@dataclasses.dataclass
class Q4KMatrix:
    """A Q4_K matrix as drawn: quants [M][K] 0..15, sub-block scales and mins
    [M][K/32] 0..63, super-block d and dmin [M][K/256] float16."""
    q: np.ndarray
    s: np.ndarray
    m: np.ndarray
    d: np.ndarray
    dmin: np.ndarray

    @property
    def M(self) -> int:
        return self.q.shape[0]

    @property
    def K(self) -> int:
        return self.q.shape[1]

    def blocks(self) -> np.ndarray:
        """GGUF Q4_K bytes, shape [M, K/256, 144] uint8."""
        M, K = self.q.shape
        if K % QKK:
            raise ValueError("K must be a multiple of 256")
        B = K // QKK
        out = np.zeros((M, B, Q4K_BYTES), dtype=np.uint8)
        out[:, :, 0:2] = np.ascontiguousarray(self.d, np.float16).view(np.uint8).reshape(M, B, 2)
        out[:, :, 2:4] = np.ascontiguousarray(self.dmin, np.float16).view(np.uint8).reshape(M, B, 2)
        s = self.s.astype(np.uint8).reshape(M, B, 8)
        m = self.m.astype(np.uint8).reshape(M, B, 8)
        sc = np.zeros((M, B, 12), dtype=np.uint8)
        sc[:, :, 0:4] = (s[:, :, 0:4] & 63) | ((s[:, :, 4:8] >> 4) << 6)
        sc[:, :, 4:8] = (m[:, :, 0:4] & 63) | ((m[:, :, 4:8] >> 4) << 6)
        sc[:, :, 8:12] = (s[:, :, 4:8] & 15) | ((m[:, :, 4:8] & 15) << 4)
        out[:, :, 4:16] = sc
        q = self.q.astype(np.uint8).reshape(M, B, 4, 2, 32)  # [group][half][32]
        out[:, :, 16:] = (q[:, :, :, 0, :] | (q[:, :, :, 1, :] << 4)).reshape(M, B, 128)
        return out


def draw_q4k(g: np.random.Generator, M: int, K: int) -> Q4KMatrix:
    """Quants, then scales, mins, d, dmin, from one generator."""
    q = g.integers(0, 16, size=(M, K), dtype=np.uint8)
    s = g.integers(0, 64, size=(M, K // 32), dtype=np.uint8)
    m = g.integers(0, 64, size=(M, K // 32), dtype=np.uint8)
    d = (np.abs(g.standard_normal((M, K // QKK))) * 0.001).astype(np.float16)
    dmin = (np.abs(g.standard_normal((M, K // QKK))) * 0.004).astype(np.float16)
    return Q4KMatrix(q, s, m, d, dmin)


# --------------------------------------------------------------------------
# Q5_K (GGUF k-quant, named on the cogni-ml page, cuda_q5k_gemv_probe).  A
# 176-byte block: the Q4_K header (d, dmin, 12 scale/min bytes), then qh[32]
# holding the fifth bit of weight k at bit k // 32 of qh[k % 32], then the
# 128 nibble bytes of the low 4 bits placed as in Q4_K.  Codes 0..31,
# weight = d * s * code - dmin * m.  Distributions: codes uniform 0..31, s
# and m uniform 0..63, d = |N(0,1)| * 0.0005, dmin = |N(0,1)| * 0.004.
# --------------------------------------------------------------------------
Q5K_BYTES = 176


@dataclasses.dataclass
class Q5KMatrix:
    """A Q5_K matrix as drawn: 5-bit codes [M][K], scales and mins [M][K/32],
    d and dmin [M][K/256] float16."""
    code: np.ndarray
    s: np.ndarray
    m: np.ndarray
    d: np.ndarray
    dmin: np.ndarray

    @property
    def M(self) -> int:
        return self.code.shape[0]

    @property
    def K(self) -> int:
        return self.code.shape[1]

    def blocks(self) -> np.ndarray:
        """GGUF Q5_K bytes, shape [M, K/256, 176] uint8."""
        M, K = self.code.shape
        B = K // QKK
        low = (self.code & 15).astype(np.uint8)
        q4 = Q4KMatrix(low, self.s, self.m, self.d, self.dmin).blocks()
        out = np.zeros((M, B, Q5K_BYTES), dtype=np.uint8)
        out[:, :, 0:16] = q4[:, :, 0:16]
        out[:, :, 48:176] = q4[:, :, 16:144]
        fifth = (self.code >> 4).astype(np.uint8).reshape(M, B, 8, 32)  # [j][l]
        out[:, :, 16:48] = (fifth << np.arange(8, dtype=np.uint8)[None, None, :, None]).sum(
            axis=2).astype(np.uint8)
        return out


def draw_q5k(g: np.random.Generator, M: int, K: int) -> Q5KMatrix:
    """Codes, then scales, mins, d, dmin, from one generator."""
    code = g.integers(0, 32, size=(M, K), dtype=np.uint8)
    s = g.integers(0, 64, size=(M, K // 32), dtype=np.uint8)
    m = g.integers(0, 64, size=(M, K // 32), dtype=np.uint8)
    d = (np.abs(g.standard_normal((M, K // QKK))) * 0.0005).astype(np.float16)
    dmin = (np.abs(g.standard_normal((M, K // QKK))) * 0.004).astype(np.float16)
    return Q5KMatrix(code, s, m, d, dmin)


# --------------------------------------------------------------------------
# Q6_K (GGUF k-quant, named on the cogni-ml page, cuda_q6k_gemv_probe: ql, qh,
# signed scales, d).  A 210-byte block holds 256 weights of one row: [0:128]
# ql (low 4 bits), [128:192] qh (high 2 bits), [192:208] 16 int8 scales (one
# per 16 weights), [208:210] d (binary16).  Weight k = 128 h + 32 a + l: low
# bits in ql[64 h + 32 (a % 2) + l] (low nibble for a < 2, else high), high
# bits at bits 2a..2a+1 of qh[32 h + l]; q = low + 16 high - 32.
# Value distributions: 6-bit codes uniform 0..63, scales uniform -128..127,
# d = |N(0,1)| * 0.0002 as binary16.
# --------------------------------------------------------------------------
Q6K_BYTES = 210


@dataclasses.dataclass
class Q6KMatrix:
    """A Q6_K matrix as drawn: 6-bit codes [M][K] 0..63 (weight = d * scale *
    (code - 32)), int8 scales [M][K/16], d [M][K/256] float16."""
    code: np.ndarray
    sc: np.ndarray
    d: np.ndarray

    @property
    def M(self) -> int:
        return self.code.shape[0]

    @property
    def K(self) -> int:
        return self.code.shape[1]

    def blocks(self) -> np.ndarray:
        """GGUF Q6_K bytes, shape [M, K/256, 210] uint8."""
        M, K = self.code.shape
        if K % QKK:
            raise ValueError("K must be a multiple of 256")
        B = K // QKK
        c = self.code.astype(np.uint8).reshape(M, B, 2, 4, 32)  # [h][a][l]
        low, high = c & 15, c >> 4
        out = np.zeros((M, B, Q6K_BYTES), dtype=np.uint8)
        ql = np.zeros((M, B, 2, 2, 32), dtype=np.uint8)  # [h][a % 2][l]
        ql[:, :, :, 0, :] = low[:, :, :, 0, :] | (low[:, :, :, 2, :] << 4)
        ql[:, :, :, 1, :] = low[:, :, :, 1, :] | (low[:, :, :, 3, :] << 4)
        out[:, :, 0:128] = ql.reshape(M, B, 128)
        qh = (high[:, :, :, 0, :] | (high[:, :, :, 1, :] << 2) | (high[:, :, :, 2, :] << 4) |
              (high[:, :, :, 3, :] << 6))
        out[:, :, 128:192] = qh.reshape(M, B, 64)
        out[:, :, 192:208] = np.ascontiguousarray(self.sc, np.int8).view(np.uint8).reshape(M, B, 16)
        out[:, :, 208:210] = np.ascontiguousarray(self.d, np.float16).view(np.uint8).reshape(M, B, 2)
        return out


def draw_q6k(g: np.random.Generator, M: int, K: int) -> Q6KMatrix:
    """Codes, then scales, then d, from one generator."""
    code = g.integers(0, 64, size=(M, K), dtype=np.uint8)
    sc = g.integers(-128, 128, size=(M, K // 16), dtype=np.int8)
    d = (np.abs(g.standard_normal((M, K // QKK))) * 0.0002).astype(np.float16)
    return Q6KMatrix(code, sc, d)


def draw_x(g: np.random.Generator, N: int, K: int) -> np.ndarray:
    return g.standard_normal((N, K)).astype(np.float32)


def matrix(cfg: int, layer: int, mat: int, M: int, K: int) -> Q8Matrix:
    return draw_matrix(rng(cfg, layer, mat), M, K)


def activations(cfg: int, N: int, K: int, layer: int = 0) -> np.ndarray:
    return draw_x(rng(cfg, layer, MAT_X), N, K)


# --------------------------------------------------------------------------
# Workload shapes
# --------------------------------------------------------------------------

# Single GEMV, 896 x 896, N = 1.
C1 = dict(cfg=1, M=896, K=896, N=1)

# Qwen2.5-0.5B-shaped decoder layer: hidden 896, 14 q heads / 2 kv heads of
# 64, intermediate 4864, 24 layers, vocabulary 151936.
QWEN05 = dict(hidden=896, n_heads=14, n_kv_heads=2, head_dim=64,
              intermediate=4864, n_layers=24, vocab=151936, eps=1e-6)
C2 = dict(cfg=2, **QWEN05)
C2_SHAPES = {  # mat id -> (M, K)
    MAT_QKV: (1152, 896),
    MAT_WO: (896, 896),
    MAT_GATE_UP: (9728, 896),
    MAT_DOWN: (896, 4864),
}
C3 = dict(cfg=3, M=151936, K=896, N=1)

# Small-batch verify chunk on 9B-class shapes.
C4 = dict(cfg=4, hidden=4096, intermediate=12288, Ns=(2, 4, 8))
C4_SHAPES = {MAT_GATE_UP: (24576, 4096), MAT_DOWN: (4096, 12288)}

# Qwen1.5-MoE-A2.7B-shaped FFN: 60 routed experts (top-4), expert
# intermediate 1408, shared expert intermediate 5632, hidden 2048.
C5 = dict(cfg=5, hidden=2048, n_experts=60, top_k=4, inter=1408, shared_inter=5632)


def layer_matrices(cfg: int, layer: int, shapes: dict) -> dict:
    return {mat: matrix(cfg, layer, mat, M, K) for mat, (M, K) in shapes.items()}


def expert_stack(cfg: int, mat: int, n_experts: int, M: int, K: int) -> np.ndarray:
    """AoS bytes of n_experts matrices, shape [E, M, K/32, 34]; expert e uses
    seed layer index e."""
    out = np.empty((n_experts, M, K // QK, BLOCK_BYTES), dtype=np.uint8)
    for e in range(n_experts):
        out[e] = matrix(cfg, e, mat, M, K).aos()
    return out


def router_logits(cfg: int, token: int, n_experts: int) -> np.ndarray:
    return rng(cfg, token, MAT_ROUTER).standard_normal(n_experts).astype(np.float32)


def shared_gate_logit(cfg: int, token: int) -> np.float32:
    return np.float32(rng(cfg, token, MAT_SHARED_GATE).standard_normal())
