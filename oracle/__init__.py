"""ctypes wrapper around the fp64 CPU oracle (q8_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg.  The HIP library never imports or links it, and
it imports nothing from the HIP package.

All arrays cross as numpy arrays; results come back as float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q8_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GCC_CMD = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", _LIB, _SRC, "-lm", "-lpthread"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        subprocess.run(GCC_CMD, check=True)
    return _LIB


_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_D = ctypes.c_double


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        # Q8_ORACLE_LIB points the wrapper at another build of the same source
        # (the mutation test uses it to load deliberately broken copies).
        path = os.environ.get("Q8_ORACLE_LIB")
        if not path:
            path = build()
        L = ctypes.CDLL(path)
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f64.restype = _D
        L.oracle_f16_decode.argtypes = [_P, _I64, _P]
        L.oracle_dequant_row.argtypes = [_P, _I64, _I64, _P]
        L.oracle_q8_0_gemv.argtypes = [_P, _I64, _I64, _P, _I64, _P, _P, ctypes.c_int]
        L.oracle_q8_0_gemv.restype = ctypes.c_int
        L.oracle_q8_0_gemv_f64.argtypes = [_P, _I64, _I64, _P, _I64, _P, _P, ctypes.c_int]
        L.oracle_q8_0_gemv_f64.restype = ctypes.c_int
        L.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_f16.restype = ctypes.c_uint16
        L.oracle_quantize_act.argtypes = [_P, _I64, _I64, _P, _P]
        L.oracle_quantize_act.restype = ctypes.c_int
        L.oracle_q8_0_gemv_q8act.argtypes = [_P, _I64, _I64, _P, _P, _I64, _P, _P]
        L.oracle_q8_0_gemv_q8act.restype = ctypes.c_int
        L.oracle_q4k_dequant_row.argtypes = [_P, _I64, _I64, _P]
        L.oracle_q4k_gemv.argtypes = [_P, _I64, _I64, _P, _I64, _P, _P]
        L.oracle_q4k_gemv.restype = ctypes.c_int
        L.oracle_q5k_dequant_row.argtypes = [_P, _I64, _I64, _P]
        L.oracle_q5k_gemv.argtypes = [_P, _I64, _I64, _P, _I64, _P, _P]
        L.oracle_q5k_gemv.restype = ctypes.c_int
        L.oracle_q6k_dequant_row.argtypes = [_P, _I64, _I64, _P]
        L.oracle_q6k_gemv.argtypes = [_P, _I64, _I64, _P, _I64, _P, _P]
        L.oracle_q6k_gemv.restype = ctypes.c_int
        L.oracle_argmax_f32.argtypes = [_P, _I64]
        L.oracle_argmax_f32.restype = _I64
        L.oracle_argmax_f64.argtypes = [_P, _I64]
        L.oracle_argmax_f64.restype = _I64
        L.oracle_route_topk.argtypes = [_P, _I32, _I32, _P, _P]
        L.oracle_route_topk.restype = ctypes.c_int
        L.oracle_silu.argtypes = [_D]
        L.oracle_silu.restype = _D
        L.oracle_sigmoid.argtypes = [_D]
        L.oracle_sigmoid.restype = _D
        L.oracle_swiglu.argtypes = [_P, _P, _I64, _P]
        L.oracle_rmsnorm.argtypes = [_P, _I64, _D, _P]
        L.oracle_gqa_position0.argtypes = [_P, _I32, _I32, _I32, _P]
        L.oracle_gqa_position0.restype = ctypes.c_int
        L.oracle_moe_combine.argtypes = [_P, _I32, _I64, _I64, _P, _P, _I32, _P, _P, _I64, _P,
                                         _D, _P, _P, ctypes.c_int]
        L.oracle_moe_combine.restype = ctypes.c_int
        L.oracle_moe_ffn.argtypes = [_P, _P, _I32, _I64, _I64, _P, _P, _I32, _P, _P, _I64, _D,
                                     _P, _P, ctypes.c_int]
        L.oracle_moe_ffn.restype = ctypes.c_int
        L.oracle_qwen_layer.argtypes = [_P, _P, _P, _P, _I64, _I32, _I32, _I32, _I64, _D, _P,
                                        ctypes.c_int]
        L.oracle_qwen_layer.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# ---------------------------------------------------------------------------
def f16_to_f64(bits) -> np.ndarray:
    b = _c(bits, np.uint16).ravel()
    out = np.empty(b.size, dtype=np.float64)
    lib().oracle_f16_decode(_ptr(b), b.size, _ptr(out))
    return out.reshape(np.shape(bits))


def dequant(aos: np.ndarray) -> np.ndarray:
    """Dequantised matrix [M][K] (float64) from AoS bytes [M, K/32, 34]."""
    aos = _c(aos, np.uint8)
    M, B = aos.shape[0], aos.shape[1]
    K = B * 32
    out = np.empty((M, K), dtype=np.float64)
    for r in range(M):
        lib().oracle_dequant_row(_ptr(aos), K, r, _ptr(out[r]))
    return out


def gemv(aos: np.ndarray, x: np.ndarray, threads: int = 0):
    """y[N][M], S[N][M] for the Q8_0 matrix in AoS bytes [M, K/32, 34] and
    activations x [N][K] (float32 -> widened exactly; float64 accepted)."""
    aos = _c(aos, np.uint8)
    M, B = aos.shape[0], aos.shape[1]
    K = B * 32
    x = np.asarray(x)
    squeeze = x.ndim == 1
    x2 = x.reshape(-1, K)
    N = x2.shape[0]
    y = np.empty((N, M), dtype=np.float64)
    S = np.empty((N, M), dtype=np.float64)
    thr = threads or default_threads()
    if x2.dtype == np.float64:
        xx = _c(x2, np.float64)
        rc = lib().oracle_q8_0_gemv_f64(_ptr(aos), M, K, _ptr(xx), N, _ptr(y), _ptr(S), thr)
    else:
        xx = _c(x2, np.float32)
        rc = lib().oracle_q8_0_gemv(_ptr(aos), M, K, _ptr(xx), N, _ptr(y), _ptr(S), thr)
    if rc:
        raise ValueError(f"oracle_q8_0_gemv failed ({rc})")
    if squeeze:
        return y[0], S[0]
    return y, S


def f32_to_f16(v: float) -> int:
    """binary16 bits of an fp32 value, round to nearest even."""
    return int(lib().oracle_f32_to_f16(ctypes.c_float(float(v))))


def quantize_act(x: np.ndarray):
    """Integer-activation variant: x [N][K] fp32 -> (qx int8 [N][K], dx
    binary16 bits [N][K/32]); see oracle_quantize_act."""
    x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float32)
    N, K = x.shape
    qx = np.zeros((N, K), dtype=np.int8)
    dx = np.zeros((N, K // 32), dtype=np.uint16)
    rc = lib().oracle_quantize_act(_ptr(x), N, K, _ptr(qx), _ptr(dx))
    if rc:
        raise ValueError(f"oracle_quantize_act: {rc}")
    return qx, dx


def gemv_q8act(aos: np.ndarray, qx: np.ndarray, dx: np.ndarray):
    """y [N][M] of the integer-activation variant and its magnitude sums S."""
    aos = _c(aos, np.uint8)
    M, nb = aos.shape[0], aos.shape[1]
    K = nb * 32
    qx = np.ascontiguousarray(np.atleast_2d(qx), dtype=np.int8)
    dx = np.ascontiguousarray(np.atleast_2d(dx), dtype=np.uint16)
    N = qx.shape[0]
    y = np.zeros((N, M))
    S = np.zeros((N, M))
    rc = lib().oracle_q8_0_gemv_q8act(_ptr(aos), M, K, _ptr(qx), _ptr(dx), N, _ptr(y), _ptr(S))
    if rc:
        raise ValueError(f"oracle_q8_0_gemv_q8act: {rc}")
    return y, S


def q4k_dequant_rows(blocks: np.ndarray, K: int) -> np.ndarray:
    """Dequantised fp64 rows of a Q4_K matrix (blocks: uint8 [M][K/256][144])."""
    blocks = _c(blocks, np.uint8)
    M = blocks.shape[0]
    out = np.zeros((M, K))
    for r in range(M):
        lib().oracle_q4k_dequant_row(_ptr(blocks), K, r, _ptr(out[r]))
    return out


def q4k_gemv(blocks: np.ndarray, x: np.ndarray):
    """y [N][M] and magnitude sums S of a Q4_K matrix times fp32 x [N][K]."""
    blocks = _c(blocks, np.uint8)
    M, K = blocks.shape[0], blocks.shape[1] * 256
    x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float32)
    N = x.shape[0]
    y = np.zeros((N, M))
    S = np.zeros((N, M))
    rc = lib().oracle_q4k_gemv(_ptr(blocks), M, K, _ptr(x), N, _ptr(y), _ptr(S))
    if rc:
        raise ValueError(f"oracle_q4k_gemv: {rc}")
    return y, S


def q5k_dequant_rows(blocks: np.ndarray, K: int) -> np.ndarray:
    """Dequantised fp64 rows of a Q5_K matrix (blocks: uint8 [M][K/256][176])."""
    blocks = _c(blocks, np.uint8)
    M = blocks.shape[0]
    out = np.zeros((M, K))
    for r in range(M):
        lib().oracle_q5k_dequant_row(_ptr(blocks), K, r, _ptr(out[r]))
    return out


def q5k_gemv(blocks: np.ndarray, x: np.ndarray):
    """y [N][M] and magnitude sums S of a Q5_K matrix times fp32 x [N][K]."""
    blocks = _c(blocks, np.uint8)
    M, K = blocks.shape[0], blocks.shape[1] * 256
    x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float32)
    N = x.shape[0]
    y = np.zeros((N, M))
    S = np.zeros((N, M))
    rc = lib().oracle_q5k_gemv(_ptr(blocks), M, K, _ptr(x), N, _ptr(y), _ptr(S))
    if rc:
        raise ValueError(f"oracle_q5k_gemv: {rc}")
    return y, S


def q6k_dequant_rows(blocks: np.ndarray, K: int) -> np.ndarray:
    """Dequantised fp64 rows of a Q6_K matrix (blocks: uint8 [M][K/256][210])."""
    blocks = _c(blocks, np.uint8)
    M = blocks.shape[0]
    out = np.zeros((M, K))
    for r in range(M):
        lib().oracle_q6k_dequant_row(_ptr(blocks), K, r, _ptr(out[r]))
    return out


def q6k_gemv(blocks: np.ndarray, x: np.ndarray):
    """y [N][M] and magnitude sums S of a Q6_K matrix times fp32 x [N][K]."""
    blocks = _c(blocks, np.uint8)
    M, K = blocks.shape[0], blocks.shape[1] * 256
    x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float32)
    N = x.shape[0]
    y = np.zeros((N, M))
    S = np.zeros((N, M))
    rc = lib().oracle_q6k_gemv(_ptr(blocks), M, K, _ptr(x), N, _ptr(y), _ptr(S))
    if rc:
        raise ValueError(f"oracle_q6k_gemv: {rc}")
    return y, S


def argmax(v: np.ndarray) -> int:
    v = np.ascontiguousarray(v)
    if v.dtype == np.float64:
        return int(lib().oracle_argmax_f64(_ptr(v), v.size))
    v = _c(v, np.float32)
    return int(lib().oracle_argmax_f32(_ptr(v), v.size))


def route_topk(logits: np.ndarray, k: int):
    logits = _c(logits, np.float32)
    ids = np.empty(k, dtype=np.int32)
    w = np.empty(k, dtype=np.float64)
    rc = lib().oracle_route_topk(_ptr(logits), logits.size, k, _ptr(ids), _ptr(w))
    if rc:
        raise ValueError("oracle_route_topk: bad arguments")
    return ids, w


def silu(z: float) -> float:
    return lib().oracle_silu(float(z))


def sigmoid(z: float) -> float:
    return lib().oracle_sigmoid(float(z))


def swiglu(g, u) -> np.ndarray:
    g = _c(g, np.float64)
    u = _c(u, np.float64)
    h = np.empty(g.size, dtype=np.float64)
    lib().oracle_swiglu(_ptr(g), _ptr(u), g.size, _ptr(h))
    return h


def rmsnorm(x, eps: float) -> np.ndarray:
    x = _c(x, np.float64)
    out = np.empty(x.size, dtype=np.float64)
    lib().oracle_rmsnorm(_ptr(x), x.size, float(eps), _ptr(out))
    return out


def gqa_position0(v, n_heads: int, n_kv_heads: int, head_dim: int) -> np.ndarray:
    v = _c(v, np.float64)
    out = np.empty(n_heads * head_dim, dtype=np.float64)
    if lib().oracle_gqa_position0(_ptr(v), n_heads, n_kv_heads, head_dim, _ptr(out)):
        raise ValueError("bad GQA shape")
    return out


def moe_combine(dn_stack, ids, w, h_routed, sh_dn, h_sh, gamma, threads: int = 0):
    """Down projections of the selected experts and the shared expert, folded
    in slot order then shared: returns (y [H], Sabs [H])."""
    dn_stack = _c(dn_stack, np.uint8)
    E, H, B = dn_stack.shape[0], dn_stack.shape[1], dn_stack.shape[2]
    I = B * 32
    ids = _c(ids, np.int32)
    w = _c(w, np.float64)
    hr = _c(h_routed, np.float64)
    S = ids.size
    y = np.empty(H, dtype=np.float64)
    Sabs = np.empty(H, dtype=np.float64)
    if sh_dn is not None:
        sh = _c(sh_dn, np.uint8)
        Ish = sh.shape[1] * 32
        hs = _c(h_sh, np.float64)
        shp, hsp = _ptr(sh), _ptr(hs)
    else:
        Ish, shp, hsp = 0, None, None
    rc = lib().oracle_moe_combine(_ptr(dn_stack), E, H, I, _ptr(ids), _ptr(w), S, _ptr(hr),
                                  shp, Ish, hsp, float(gamma), _ptr(y), _ptr(Sabs),
                                  threads or default_threads())
    if rc:
        raise ValueError(f"oracle_moe_combine failed ({rc})")
    return y, Sabs


def moe_ffn(gu_stack, dn_stack, ids, w, sh_gu, sh_dn, gamma, x, threads: int = 0):
    gu_stack = _c(gu_stack, np.uint8)
    dn_stack = _c(dn_stack, np.uint8)
    E, I2, B = gu_stack.shape[0], gu_stack.shape[1], gu_stack.shape[2]
    H = B * 32
    I = I2 // 2
    ids = _c(ids, np.int32)
    w = _c(w, np.float64)
    x = _c(x, np.float32)
    y = np.empty(H, dtype=np.float64)
    if sh_gu is not None:
        sg = _c(sh_gu, np.uint8)
        sd = _c(sh_dn, np.uint8)
        Ish = sg.shape[0] // 2
        sgp, sdp = _ptr(sg), _ptr(sd)
    else:
        Ish, sgp, sdp = 0, None, None
    rc = lib().oracle_moe_ffn(_ptr(gu_stack), _ptr(dn_stack), E, H, I, _ptr(ids), _ptr(w),
                              ids.size, sgp, sdp, Ish, float(gamma), _ptr(x), _ptr(y),
                              threads or default_threads())
    if rc:
        raise ValueError(f"oracle_moe_ffn failed ({rc})")
    return y


def qwen_layer(qkv_aos, wo_aos, gu_aos, down_aos, h, n_heads, n_kv_heads, head_dim, eps,
               threads: int = 0) -> np.ndarray:
    qkv_aos, wo_aos = _c(qkv_aos, np.uint8), _c(wo_aos, np.uint8)
    gu_aos, down_aos = _c(gu_aos, np.uint8), _c(down_aos, np.uint8)
    hidden = wo_aos.shape[0]
    inter = gu_aos.shape[0] // 2
    hh = np.array(h, dtype=np.float64, copy=True)
    rc = lib().oracle_qwen_layer(_ptr(qkv_aos), _ptr(wo_aos), _ptr(gu_aos), _ptr(down_aos),
                                 hidden, n_heads, n_kv_heads, head_dim, inter, float(eps),
                                 _ptr(hh), threads or default_threads())
    if rc:
        raise ValueError(f"oracle_qwen_layer failed ({rc})")
    return hh
