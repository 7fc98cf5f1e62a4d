"""Helpers for the GPU parity tests: upload seeded inputs, repack through the
C ABI, and compare against the oracle."""
import numpy as np
import torch

import block_quantized_gemv_amd as q
import workloads as W

DEV = torch.device("cuda", 0)


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def pack(m_or_aos, M=None, K=None, n_mats=1, layout=q.Q8_LAYOUT_ROWS) -> q.PackedQ8:
    """Upload AoS bytes (a Q8Matrix or a uint8 array) and repack on device."""
    aos = m_or_aos.aos() if isinstance(m_or_aos, W.Q8Matrix) else m_or_aos
    aos = np.ascontiguousarray(aos, dtype=np.uint8)
    if M is None:
        M, K = aos.shape[-3], aos.shape[-2] * 32
    return q.PackedQ8.from_aos(to_dev(aos.reshape(-1)), M, K, n_mats, layout=layout)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def expected_packed(qs: np.ndarray, d: np.ndarray, layout=q.Q8_LAYOUT_ROWS):
    """The packed layout written out from its definition in include/q8gemv.h
    (independent of the repack kernel): quants [T][K/16][64][16], scales
    [T][G][64][4]; with the gate/up pairs layout, packed row 64t+i holds
    matrix row 32t+i (i < 32) or M/2+32t+i-32."""
    M, K = qs.shape
    if layout == q.Q8_LAYOUT_GATE_UP_PAIRS:
        t = np.arange(M) // 64
        i = np.arange(M) % 64
        src = np.where(i < 32, 32 * t + i, M // 2 + 32 * t + i - 32)
        qs, d = qs[src], d[src]
    T = -(-M // 64)
    nb = K // 32
    G = -(-nb // 4)
    qpad = np.zeros((T * 64, K), dtype=np.int8)
    qpad[:M] = qs
    eq = qpad.reshape(T, 64, K // 16, 16).transpose(0, 2, 1, 3).copy()
    dpad = np.zeros((T * 64, G * 4), dtype=np.uint16)
    dpad[:M, :nb] = d.view(np.uint16)
    ed = dpad.reshape(T, 64, G, 4).transpose(0, 2, 1, 3).copy()
    return eq.view(np.uint8).reshape(-1), ed.view(np.uint8).reshape(-1)
