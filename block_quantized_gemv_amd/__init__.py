"""Python binding of the Q8_0 decode GEMV library (libq8gemv.so).

Thin ctypes marshalling over the C ABI declared in include/q8gemv.h; the
functions keep the C names.  PyTorch provides device memory and the current
stream only: every step of the computation runs in the library's HIP kernels.
There is no fallback path: if the shared library is missing, importing a
function raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libq8gemv.so")

Q8_OK, Q8_EINVAL, Q8_ENULL, Q8_EALIGN, Q8_EHOSTPTR, Q8_EWORKSPACE, Q8_ELAUNCH = 0, -1, -2, -3, -4, -5, -6
Q8_MAX_N = 8
Q8_MAX_K = 1 << 20
Q8_MAX_SLOTS = 8
Q8_TILE_ROWS = 64
Q8_PRO_NONE, Q8_PRO_RMSNORM, Q8_PRO_GQA = 0, 1, 2
Q8_EPI_RESIDUAL, Q8_EPI_SWIGLU, Q8_EPI_ARGMAX = 1, 2, 4
Q8_MOE_SCATTER, Q8_MOE_COMBINE, Q8_MOE_SWIGLU = 1, 2, 4
Q8_OP_GEMV, Q8_OP_GEMV_FUSED, Q8_OP_ARGMAX, Q8_OP_MOE_SCATTER, Q8_OP_MOE_COMBINE = 1, 2, 3, 4, 5
Q8_OP_GEMV_ARGMAX = 6
Q8_OP_Q4K_GEMV = 7
Q8_OP_Q6K_GEMV = 8
Q8_OP_Q5K_GEMV = 9

Q8_LAYOUT_ROWS, Q8_LAYOUT_GATE_UP_PAIRS = 0, 1
Q8_CHAIN_COHERENT = 1
Q8_CHAIN_QKV, Q8_CHAIN_H_ATTN, Q8_CHAIN_SWIGLU, Q8_CHAIN_H_OUT = 0, 1, 2, 3
Q8_CHAIN_STAMP_LAYERS, Q8_CHAIN_STAMP_POINTS, Q8_CHAIN_STAMP_KERNEL = 32, 16, 4
Q8_CHAIN_STAMP_WORDS = Q8_CHAIN_STAMP_LAYERS * Q8_CHAIN_STAMP_POINTS + Q8_CHAIN_STAMP_KERNEL

EXPORTS = ("q8_0_packed_size", "q8_0_repack", "q8_0_repack_layout", "q8_0_repack_host",
           "q8_0_repack_staging_bytes", "q8_0_gemv", "q8_0_gemv_fused",
           "q8_0_gemv_argmax", "q8_0_quantize_act", "q8_0_gemv_q8act", "q8_0_argmax",
           "q8_0_route_topk", "q8_0_moe_gemv", "q8_0_workspace_bytes", "q8_0_gemv_plan",
           "q8_0_strerror", "q8_0_version", "q8_0_chain_workspace_bytes", "q8_0_chain_prepare",
           "q8_0_chain_run", "q8_0_chain_read", "q8_0_chain_status", "q4k_packed_size",
           "q4k_repack", "q4k_gemv", "q5k_packed_size", "q5k_repack", "q5k_gemv",
           "q6k_packed_size", "q6k_repack", "q6k_gemv", "q8_0_gemv_noalloc",
           "q8_stream_read", "q8_0_moe_route_gemv", "q8_0_chain_run_stamped")


class Q8Error(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn}: {strerror(code)} ({code})")


class q8_0_weights(ctypes.Structure):
    _fields_ = [("qs", ctypes.c_void_p), ("d", ctypes.c_void_p), ("M", ctypes.c_int64),
                ("K", ctypes.c_int64), ("n_mats", ctypes.c_int64),
                ("qs_stride", ctypes.c_int64), ("d_stride", ctypes.c_int64),
                ("layout", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class q8_0_fusion(ctypes.Structure):
    _fields_ = [("prologue", ctypes.c_int32), ("epilogue", ctypes.c_int32),
                ("eps", ctypes.c_float), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("gqa_offset", ctypes.c_int64), ("residual", ctypes.c_void_p),
                ("argmax_out", ctypes.c_void_p)]


class q8_0_chain_desc(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("eps", ctypes.c_float),
                ("qkv", ctypes.POINTER(q8_0_weights)), ("wo", ctypes.POINTER(q8_0_weights)),
                ("gate_up", ctypes.POINTER(q8_0_weights)), ("down", ctypes.POINTER(q8_0_weights)),
                ("lm_head", ctypes.POINTER(q8_0_weights))]


class q8_0_chain_plan(ctypes.Structure):
    _fields_ = [("grid", ctypes.c_int32), ("threads", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32), ("n_layers", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("intermediate", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("eps", ctypes.c_float), ("flags", ctypes.c_uint32),
                ("ws_bytes", ctypes.c_int64), ("off", ctypes.c_int64 * 4),
                ("layer_stride", ctypes.c_int64), ("am_off", ctypes.c_int64),
                ("lm_qs", ctypes.c_void_p), ("lm_d", ctypes.c_void_p),
                ("len", ctypes.c_int32 * 4), ("spin_limit", ctypes.c_uint32),
                ("groups", ctypes.c_int32), ("off_v", ctypes.c_int64),
                ("off_p", ctypes.c_int64), ("group_words_v", ctypes.c_int32),
                ("group_words_h", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded shared library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_quantized_gemv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        PW = ctypes.POINTER(q8_0_weights)
        L.q8_0_packed_size.argtypes = [I64, I64, ctypes.POINTER(SZ), ctypes.POINTER(SZ)]
        L.q8_0_repack.argtypes = [P, I64, I64, P, P, P]
        L.q8_0_repack_layout.argtypes = [P, I64, I64, I32, P, P, P]
        L.q8_0_repack_host.argtypes = [P, I64, I64, I32, P, P, P, SZ, P]
        L.q8_0_repack_staging_bytes.argtypes = [I64, I64]
        L.q8_0_repack_staging_bytes.restype = SZ
        L.q8_0_gemv.argtypes = [PW, P, P, I64, I64, I64, P, SZ, P]
        L.q8_0_gemv_noalloc.argtypes = [PW, P, P, I64, I64, I64, P]
        L.q8_stream_read.argtypes = [P, I64, P, I32, P]
        L.q8_0_gemv_fused.argtypes = [PW, P, P, I64, I64, ctypes.POINTER(q8_0_fusion), P, SZ, P]
        L.q8_0_gemv_argmax.argtypes = [PW, P, P, I64, I64, I64, P, P, SZ, P]
        L.q8_0_quantize_act.argtypes = [P, I64, I64, P, P, P]
        L.q8_0_gemv_q8act.argtypes = [PW, P, P, P, I64, I64, I64, P, SZ, P]
        L.q4k_packed_size.argtypes = [I64, I64, ctypes.POINTER(SZ), ctypes.POINTER(SZ)]
        L.q4k_repack.argtypes = [P, I64, I64, P, P, P]
        L.q4k_gemv.argtypes = [ctypes.POINTER(q4k_weights), P, P, I64, I64, I64, P, SZ, P]
        L.q5k_packed_size.argtypes = [I64, I64, ctypes.POINTER(SZ), ctypes.POINTER(SZ),
                                      ctypes.POINTER(SZ)]
        L.q5k_repack.argtypes = [P, I64, I64, P, P, P, P]
        L.q5k_gemv.argtypes = [ctypes.POINTER(q5k_weights), P, P, I64, I64, I64, P, SZ, P]
        L.q6k_packed_size.argtypes = [I64, I64, ctypes.POINTER(SZ), ctypes.POINTER(SZ),
                                      ctypes.POINTER(SZ)]
        L.q6k_repack.argtypes = [P, I64, I64, P, P, P, P]
        L.q6k_gemv.argtypes = [ctypes.POINTER(q6k_weights), P, P, I64, I64, I64, P, SZ, P]
        L.q8_0_argmax.argtypes = [P, I64, P, P, SZ, P]
        L.q8_0_route_topk.argtypes = [P, I32, I32, P, P, P]
        L.q8_0_moe_gemv.argtypes = [PW, P, P, P, P, I64, I64, I32, I32, PW, P, P, P, SZ, P]
        L.q8_0_moe_route_gemv.argtypes = [PW, P, I32, P, P, P, P, I64, I64, I32, I32, PW, P, P,
                                          SZ, P]
        L.q8_0_workspace_bytes.argtypes = [I32, I64, I64, I64, I64, I64, I32]
        L.q8_0_workspace_bytes.restype = SZ
        L.q8_0_gemv_plan.argtypes = [I64, I64, I64, I32, ctypes.POINTER(I32)]
        L.q8_0_strerror.argtypes = [ctypes.c_int]
        L.q8_0_strerror.restype = ctypes.c_char_p
        L.q8_0_version.argtypes = []
        PD, PP = ctypes.POINTER(q8_0_chain_desc), ctypes.POINTER(q8_0_chain_plan)
        L.q8_0_chain_workspace_bytes.argtypes = [PD]
        L.q8_0_chain_workspace_bytes.restype = SZ
        L.q8_0_chain_prepare.argtypes = [PD, P, SZ, PP, P]
        L.q8_0_chain_run.argtypes = [PP, P, P, P, P, P, P]
        L.q8_0_chain_run_stamped.argtypes = [PP, P, P, P, P, P, P, P]
        L.q8_0_chain_read.argtypes = [PP, P, I32, I32, P, P]
        L.q8_0_chain_status.argtypes = [P, P, P]
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().q8_0_strerror(code).decode()


def _check(fn: str, rc: int) -> None:
    if rc != Q8_OK:
        raise Q8Error(fn, rc)


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ncols(x: torch.Tensor, K: int, name: str = "x") -> int:
    """Columns N of an activation tensor holding N vectors of K entries ([K]
    or [N, K]); raises ValueError before anything reaches the library."""
    N = 1 if x.dim() == 1 else x.shape[0]
    if x.dim() > 2 or x.numel() != N * K:
        raise ValueError(f"{name} has shape {tuple(x.shape)}; expected [{K}] or [N, {K}]")
    if not 1 <= N <= Q8_MAX_N:
        raise ValueError(f"{name} has {N} columns; 1..{Q8_MAX_N} are supported")
    return N


def _room(t: torch.Tensor, n: int, name: str) -> None:
    if t.numel() < n:
        raise ValueError(f"{name} has {t.numel()} entries; the call writes {n}")


def _need(t: torch.Tensor, dtype, name: str) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ---------------------------------------------------------------------------
# Workspace: zero-filled once, grown on demand (growing allocates, so size it
# before capturing a graph).  Calls on different streams need distinct ones.
# ---------------------------------------------------------------------------
class Workspace:
    def __init__(self, nbytes: int = 0, device=None):
        self.buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8,
                               device=device or torch.device("cuda"))

    def get(self, nbytes: int) -> tuple[int, int]:
        if nbytes == 0:
            return 0, 0
        if self.buf.numel() < nbytes:
            self.buf = torch.zeros(nbytes, dtype=torch.uint8, device=self.buf.device)
        return self.buf.data_ptr(), self.buf.numel()


_default_ws: dict = {}


def default_workspace(device=None) -> Workspace:
    dev = torch.device(device) if device is not None else torch.device("cuda",
                                                                       torch.cuda.current_device())
    if dev not in _default_ws:
        _default_ws[dev] = Workspace(1 << 20, dev)
    return _default_ws[dev]


def q8_0_workspace_bytes(op: int, M: int, K: int, N: int, M2: int = 0, K2: int = 0,
                         flags: int = 0) -> int:
    return int(lib().q8_0_workspace_bytes(op, M, K, N, M2, K2, flags))


def q8_0_gemv_plan(M: int, K: int, N: int = 1, epilogue: int = 0) -> dict:
    out = (ctypes.c_int32 * 4)()
    _check("q8_0_gemv_plan", lib().q8_0_gemv_plan(M, K, N, epilogue, out))
    return {"workgroups": out[0], "waves_per_wg": out[1], "units_per_tile": out[2],
            "wgs_per_tile": out[3]}


def q8_0_version() -> int:
    return lib().q8_0_version()


# ---------------------------------------------------------------------------
# Packed weights
# ---------------------------------------------------------------------------
def q8_0_packed_size(M: int, K: int) -> tuple[int, int]:
    qb, db = ctypes.c_size_t(), ctypes.c_size_t()
    _check("q8_0_packed_size", lib().q8_0_packed_size(M, K, ctypes.byref(qb), ctypes.byref(db)))
    return qb.value, db.value


class q4k_weights(ctypes.Structure):
    _fields_ = [("qs", ctypes.c_void_p), ("meta", ctypes.c_void_p), ("M", ctypes.c_int64),
                ("K", ctypes.c_int64)]


class PackedQ4K:
    """Packed device Q4_K weights of one matrix (see q4k_repack in q8gemv.h)."""

    def __init__(self, qs: torch.Tensor, meta: torch.Tensor, M: int, K: int):
        self.qs, self.meta, self.M, self.K = qs, meta, M, K
        self.desc = q4k_weights(qs.data_ptr(), meta.data_ptr(), M, K)

    @classmethod
    def from_blocks(cls, blocks: torch.Tensor, M: int, K: int, stream=None) -> "PackedQ4K":
        """Repack GGUF Q4_K blocks (uint8 device tensor of M*(K/256)*144 bytes)."""
        _need(blocks, torch.uint8, "blocks")
        if blocks.numel() != M * (K // 256) * 144:
            raise ValueError(f"blocks has {blocks.numel()} bytes, expected {M * (K // 256) * 144}")
        qb, mb = q4k_packed_size(M, K)
        qs = torch.empty(qb, dtype=torch.uint8, device=blocks.device)
        meta = torch.empty(mb, dtype=torch.uint8, device=blocks.device)
        _check("q4k_repack", lib().q4k_repack(blocks.data_ptr(), M, K, qs.data_ptr(),
                                              meta.data_ptr(), _stream(stream)))
        return cls(qs, meta, M, K)


def q4k_packed_size(M: int, K: int) -> tuple[int, int]:
    qb, mb = ctypes.c_size_t(), ctypes.c_size_t()
    _check("q4k_packed_size", lib().q4k_packed_size(M, K, ctypes.byref(qb), ctypes.byref(mb)))
    return qb.value, mb.value


def q4k_gemv(W: PackedQ4K, x: torch.Tensor, y: torch.Tensor | None = None, workspace=None,
             stream=None) -> torch.Tensor:
    """y[N][M] = x[N][K] @ W^T for packed Q4_K weights W (x float32)."""
    N = _ncols(x, W.K)
    if y is not None:
        _room(y, N * W.M, "y")
    _need(x, torch.float32, "x")
    if y is None:
        y = torch.empty((W.M,) if x.dim() == 1 else (N, W.M), dtype=torch.float32,
                        device=x.device)
    _need(y, torch.float32, "y")
    wsp, wsb = _ws(workspace, q8_0_workspace_bytes(Q8_OP_Q4K_GEMV, W.M, W.K, N), x.device)
    _check("q4k_gemv", lib().q4k_gemv(ctypes.byref(W.desc), x.data_ptr(), y.data_ptr(), W.M,
                                      W.K, N, wsp, wsb, _stream(stream)))
    return y


class q5k_weights(ctypes.Structure):
    _fields_ = [("qs", ctypes.c_void_p), ("qh", ctypes.c_void_p), ("meta", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("K", ctypes.c_int64)]


class PackedQ5K:
    """Packed device Q5_K weights of one matrix (see q5k_repack in q8gemv.h)."""

    def __init__(self, qs: torch.Tensor, qh: torch.Tensor, meta: torch.Tensor, M: int, K: int):
        self.qs, self.qh, self.meta, self.M, self.K = qs, qh, meta, M, K
        self.desc = q5k_weights(qs.data_ptr(), qh.data_ptr(), meta.data_ptr(), M, K)

    @classmethod
    def from_blocks(cls, blocks: torch.Tensor, M: int, K: int, stream=None) -> "PackedQ5K":
        """Repack GGUF Q5_K blocks (uint8 device tensor of M*(K/256)*176 bytes)."""
        _need(blocks, torch.uint8, "blocks")
        if blocks.numel() != M * (K // 256) * 176:
            raise ValueError(f"blocks has {blocks.numel()} bytes, expected {M * (K // 256) * 176}")
        a, b, c = q5k_packed_size(M, K)
        qs = torch.empty(a, dtype=torch.uint8, device=blocks.device)
        qh = torch.empty(b, dtype=torch.uint8, device=blocks.device)
        meta = torch.empty(c, dtype=torch.uint8, device=blocks.device)
        _check("q5k_repack", lib().q5k_repack(blocks.data_ptr(), M, K, qs.data_ptr(),
                                              qh.data_ptr(), meta.data_ptr(), _stream(stream)))
        return cls(qs, qh, meta, M, K)


def q5k_packed_size(M: int, K: int) -> tuple[int, int, int]:
    a, b, c = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check("q5k_packed_size", lib().q5k_packed_size(M, K, ctypes.byref(a), ctypes.byref(b),
                                                    ctypes.byref(c)))
    return a.value, b.value, c.value


def q5k_gemv(W: PackedQ5K, x: torch.Tensor, y: torch.Tensor | None = None, workspace=None,
             stream=None) -> torch.Tensor:
    """y[N][M] = x[N][K] @ W^T for packed Q5_K weights W (x float32)."""
    N = _ncols(x, W.K)
    if y is not None:
        _room(y, N * W.M, "y")
    _need(x, torch.float32, "x")
    if y is None:
        y = torch.empty((W.M,) if x.dim() == 1 else (N, W.M), dtype=torch.float32,
                        device=x.device)
    _need(y, torch.float32, "y")
    wsp, wsb = _ws(workspace, q8_0_workspace_bytes(Q8_OP_Q5K_GEMV, W.M, W.K, N), x.device)
    _check("q5k_gemv", lib().q5k_gemv(ctypes.byref(W.desc), x.data_ptr(), y.data_ptr(), W.M,
                                      W.K, N, wsp, wsb, _stream(stream)))
    return y


class q6k_weights(ctypes.Structure):
    _fields_ = [("ql", ctypes.c_void_p), ("qh", ctypes.c_void_p), ("meta", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("K", ctypes.c_int64)]


class PackedQ6K:
    """Packed device Q6_K weights of one matrix (see q6k_repack in q8gemv.h)."""

    def __init__(self, ql: torch.Tensor, qh: torch.Tensor, meta: torch.Tensor, M: int, K: int):
        self.ql, self.qh, self.meta, self.M, self.K = ql, qh, meta, M, K
        self.desc = q6k_weights(ql.data_ptr(), qh.data_ptr(), meta.data_ptr(), M, K)

    @classmethod
    def from_blocks(cls, blocks: torch.Tensor, M: int, K: int, stream=None) -> "PackedQ6K":
        """Repack GGUF Q6_K blocks (uint8 device tensor of M*(K/256)*210 bytes)."""
        _need(blocks, torch.uint8, "blocks")
        if blocks.numel() != M * (K // 256) * 210:
            raise ValueError(f"blocks has {blocks.numel()} bytes, expected {M * (K // 256) * 210}")
        a, b, c = q6k_packed_size(M, K)
        ql = torch.empty(a, dtype=torch.uint8, device=blocks.device)
        qh = torch.empty(b, dtype=torch.uint8, device=blocks.device)
        meta = torch.empty(c, dtype=torch.uint8, device=blocks.device)
        _check("q6k_repack", lib().q6k_repack(blocks.data_ptr(), M, K, ql.data_ptr(),
                                              qh.data_ptr(), meta.data_ptr(), _stream(stream)))
        return cls(ql, qh, meta, M, K)


def q6k_packed_size(M: int, K: int) -> tuple[int, int, int]:
    a, b, c = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check("q6k_packed_size", lib().q6k_packed_size(M, K, ctypes.byref(a), ctypes.byref(b),
                                                    ctypes.byref(c)))
    return a.value, b.value, c.value


def q6k_gemv(W: PackedQ6K, x: torch.Tensor, y: torch.Tensor | None = None, workspace=None,
             stream=None) -> torch.Tensor:
    """y[N][M] = x[N][K] @ W^T for packed Q6_K weights W (x float32)."""
    N = _ncols(x, W.K)
    if y is not None:
        _room(y, N * W.M, "y")
    _need(x, torch.float32, "x")
    if y is None:
        y = torch.empty((W.M,) if x.dim() == 1 else (N, W.M), dtype=torch.float32,
                        device=x.device)
    _need(y, torch.float32, "y")
    wsp, wsb = _ws(workspace, q8_0_workspace_bytes(Q8_OP_Q6K_GEMV, W.M, W.K, N), x.device)
    _check("q6k_gemv", lib().q6k_gemv(ctypes.byref(W.desc), x.data_ptr(), y.data_ptr(), W.M,
                                      W.K, N, wsp, wsb, _stream(stream)))
    return y


class PackedQ8:
    """Packed device weights of one matrix or a stack of n_mats matrices."""

    def __init__(self, qs: torch.Tensor, d: torch.Tensor, M: int, K: int, n_mats: int = 1,
                 layout: int = Q8_LAYOUT_ROWS):
        qb, db = q8_0_packed_size(M, K)
        self.qs, self.d, self.M, self.K, self.n_mats = qs, d, M, K, n_mats
        self.qs_bytes, self.d_bytes, self.layout = qb, db, layout
        self.desc = q8_0_weights(qs.data_ptr(), d.data_ptr(), M, K, n_mats, qb, db, layout, 0)

    @classmethod
    def empty(cls, M: int, K: int, n_mats: int = 1, device=None,
              layout: int = Q8_LAYOUT_ROWS) -> "PackedQ8":
        qb, db = q8_0_packed_size(M, K)
        dev = device or torch.device("cuda")
        qs = torch.empty(n_mats * qb, dtype=torch.uint8, device=dev)
        d = torch.empty(n_mats * db, dtype=torch.uint8, device=dev)
        return cls(qs, d, M, K, n_mats, layout)

    @classmethod
    def from_aos(cls, aos: torch.Tensor, M: int, K: int, n_mats: int = 1, stream=None,
                 layout: int = Q8_LAYOUT_ROWS) -> "PackedQ8":
        """Repack GGUF Q8_0 blocks (uint8 device tensor of n_mats*M*(K/32)*34
        bytes), one matrix at a time, in the given row layout."""
        _need(aos, torch.uint8, "aos")
        per = M * (K // 32) * 34
        if aos.numel() != n_mats * per:
            raise ValueError(f"aos has {aos.numel()} bytes, expected {n_mats * per}")
        p = cls.empty(M, K, n_mats, aos.device, layout)
        for e in range(n_mats):
            q8_0_repack(aos[e * per:(e + 1) * per], M, K, p.qs[e * p.qs_bytes:],
                        p.d[e * p.d_bytes:], stream, layout)
        return p

    def expert(self, e: int) -> "PackedQ8":
        return PackedQ8(self.qs[e * self.qs_bytes:(e + 1) * self.qs_bytes],
                        self.d[e * self.d_bytes:(e + 1) * self.d_bytes], self.M, self.K, 1,
                        self.layout)


def q8_0_repack(aos: torch.Tensor, M: int, K: int, qs: torch.Tensor, d: torch.Tensor,
                stream=None, layout: int = Q8_LAYOUT_ROWS) -> None:
    if aos.numel() != M * (K // 32) * 34:
        raise ValueError(f"aos has {aos.numel()} bytes, expected {M * (K // 32) * 34}")
    qb, db = q8_0_packed_size(M, K)
    _room(qs, qb, "qs")
    _room(d, db, "d")
    _need(aos, torch.uint8, "aos")
    if layout == Q8_LAYOUT_ROWS:
        rc = lib().q8_0_repack(aos.data_ptr(), M, K, qs.data_ptr(), d.data_ptr(), _stream(stream))
        _check("q8_0_repack", rc)
    else:
        rc = lib().q8_0_repack_layout(aos.data_ptr(), M, K, layout, qs.data_ptr(), d.data_ptr(),
                                      _stream(stream))
        _check("q8_0_repack_layout", rc)


def q8_0_repack_staging_bytes(M: int, K: int) -> int:
    """Smallest device staging buffer q8_0_repack_host accepts (one 64-row
    tile of 34-byte blocks)."""
    return int(lib().q8_0_repack_staging_bytes(M, K))


def q8_0_repack_host(aos, M: int, K: int, qs: torch.Tensor, d: torch.Tensor,
                     staging: torch.Tensor, stream=None, layout: int = Q8_LAYOUT_ROWS) -> None:
    """Repack GGUF Q8_0 blocks held in host memory (a contiguous uint8 numpy
    array or CPU tensor of M*(K/32)*34 bytes) through the device buffer
    `staging`, band by band.  Synchronises the stream before returning, so the
    host array may be freed afterwards."""
    if isinstance(aos, torch.Tensor):
        if aos.is_cuda or aos.dtype != torch.uint8 or not aos.is_contiguous():
            raise ValueError("aos must be a contiguous uint8 host array")
        ptr, n = aos.data_ptr(), aos.numel()
    else:
        if aos.dtype != np.uint8 or not aos.flags["C_CONTIGUOUS"]:
            raise ValueError("aos must be a contiguous uint8 host array")
        ptr, n = aos.ctypes.data, aos.size
    if n != M * (K // 32) * 34:
        raise ValueError(f"aos has {n} bytes, expected {M * (K // 32) * 34}")
    qb, db = q8_0_packed_size(M, K)
    _room(qs, qb, "qs")
    _room(d, db, "d")
    _need(staging, torch.uint8, "staging")
    st = stream if stream is not None else torch.cuda.current_stream()
    rc = lib().q8_0_repack_host(ptr, M, K, layout, qs.data_ptr(), d.data_ptr(),
                                staging.data_ptr(), staging.numel(), _stream(st))
    _check("q8_0_repack_host", rc)
    st.synchronize()


# ---------------------------------------------------------------------------
# GEMV family
# ---------------------------------------------------------------------------
def _ws(ws, nbytes: int, device) -> tuple[int, int]:
    if nbytes == 0:
        return 0, 0
    if ws is None:
        ws = default_workspace(device)
    if isinstance(ws, Workspace):
        return ws.get(nbytes)
    return ws.data_ptr(), ws.numel() * ws.element_size()


def q8_0_gemv(W: PackedQ8, x: torch.Tensor, y: torch.Tensor | None = None, workspace=None,
              stream=None) -> torch.Tensor:
    """y[N][M] = x[N][K] @ W^T for packed Q8_0 weights W (x float32)."""
    N = _ncols(x, W.K)
    if y is not None:
        _room(y, N * W.M, "y")
    _need(x, torch.float32, "x")
    if y is None:
        y = torch.empty((W.M,) if x.dim() == 1 else (N, W.M), dtype=torch.float32,
                        device=x.device)
    _need(y, torch.float32, "y")
    wsp, wsb = _ws(workspace, q8_0_workspace_bytes(Q8_OP_GEMV, W.M, W.K, N), x.device)
    _check("q8_0_gemv", lib().q8_0_gemv(ctypes.byref(W.desc), x.data_ptr(), y.data_ptr(), W.M,
                                        W.K, N, wsp, wsb, _stream(stream)))
    return y


def q8_0_gemv_noalloc(W: PackedQ8, x: torch.Tensor, y: torch.Tensor, stream=None) -> torch.Tensor:
    """q8_0_gemv with no workspace and no allocation (the library's own
    per-device scratch array); y must be given."""
    N = _ncols(x, W.K)
    _room(y, N * W.M, "y")
    _need(x, torch.float32, "x")
    _need(y, torch.float32, "y")
    _check("q8_0_gemv_noalloc", lib().q8_0_gemv_noalloc(ctypes.byref(W.desc), x.data_ptr(),
                                                        y.data_ptr(), W.M, W.K, N,
                                                        _stream(stream)))
    return y


def q8_stream_read(buf: torch.Tensor, out: torch.Tensor, grid: int = 4096, stream=None) -> None:
    """The streaming read reference kernel over all of buf's bytes (see
    q8_stream_read in include/q8gemv.h); out: device int32 [>= grid], one XOR
    word per workgroup."""
    if not buf.is_cuda or not out.is_cuda:
        raise ValueError("buf and out must be device tensors")
    _room(out, grid, "out")
    _need(out, torch.int32, "out")
    _check("q8_stream_read", lib().q8_stream_read(buf.data_ptr(),
                                                  buf.numel() * buf.element_size(),
                                                  out.data_ptr(), grid, _stream(stream)))


def make_fusion(prologue: int = Q8_PRO_NONE, epilogue: int = 0, eps: float = 0.0,
                n_heads: int = 0, n_kv_heads: int = 0, head_dim: int = 0, gqa_offset: int = 0,
                residual: torch.Tensor | None = None,
                argmax_out: torch.Tensor | None = None) -> q8_0_fusion:
    f = q8_0_fusion(prologue, epilogue, eps, n_heads, n_kv_heads, head_dim, gqa_offset,
                    residual.data_ptr() if residual is not None else None,
                    argmax_out.data_ptr() if argmax_out is not None else None)
    # sizes of the tensors behind the raw pointers, checked by q8_0_gemv_fused
    f.residual_numel = residual.numel() if residual is not None else None
    f.argmax_numel = argmax_out.numel() if argmax_out is not None else None
    return f


def q8_0_gemv_fused(W: PackedQ8, x: torch.Tensor, y: torch.Tensor, fusion: q8_0_fusion,
                    workspace=None, stream=None) -> torch.Tensor:
    if fusion.prologue == Q8_PRO_GQA:
        need = fusion.gqa_offset + fusion.n_kv_heads * fusion.head_dim
        if fusion.n_heads * fusion.head_dim != W.K or x.numel() < need:
            raise ValueError(f"GQA prologue reads x[{fusion.gqa_offset}:{need}] of a vector "
                             f"of {x.numel()}, with n_heads*head_dim == K ({W.K})")
    elif x.numel() != W.K:
        raise ValueError(f"x has {x.numel()} entries, expected K = {W.K}")
    _room(y, W.M // 2 if fusion.epilogue & Q8_EPI_SWIGLU else W.M, "y")
    if fusion.epilogue & Q8_EPI_RESIDUAL and fusion.residual:
        n = getattr(fusion, "residual_numel", None)
        if n is not None and n < W.M:
            raise ValueError(f"residual has {n} entries, expected {W.M}")
    if fusion.epilogue & Q8_EPI_ARGMAX and fusion.argmax_out:
        n = getattr(fusion, "argmax_numel", None)
        if n is not None and n < 1:
            raise ValueError("argmax_out needs one entry")
    _need(x, torch.float32, "x")
    _need(y, torch.float32, "y")
    wsp, wsb = _ws(workspace,
                   q8_0_workspace_bytes(Q8_OP_GEMV_FUSED, W.M, W.K, fusion.epilogue), x.device)
    _check("q8_0_gemv_fused", lib().q8_0_gemv_fused(ctypes.byref(W.desc), x.data_ptr(),
                                                    y.data_ptr(), W.M, W.K, ctypes.byref(fusion),
                                                    wsp, wsb, _stream(stream)))
    return y


def q8_0_gemv_argmax(W: PackedQ8, x: torch.Tensor, y: torch.Tensor | None = None,
                     argmax_out: torch.Tensor | None = None, workspace=None, stream=None):
    """y[N][M] = x[N][K] @ W^T and argmax_out[n] = lowest index of the largest
    y[n][*], one pick per column; returns (y, argmax_out)."""
    N = _ncols(x, W.K)
    if y is not None:
        _room(y, N * W.M, "y")
    if argmax_out is not None:
        _room(argmax_out, N, "argmax_out")
    _need(x, torch.float32, "x")
    if y is None:
        y = torch.empty((W.M,) if x.dim() == 1 else (N, W.M), dtype=torch.float32,
                        device=x.device)
    if argmax_out is None:
        argmax_out = torch.empty(N, dtype=torch.int32, device=x.device)
    _need(y, torch.float32, "y")
    _need(argmax_out, torch.int32, "argmax_out")
    if argmax_out.numel() < N:
        raise ValueError("argmax_out needs one entry per column")
    wsp, wsb = _ws(workspace, q8_0_workspace_bytes(Q8_OP_GEMV_ARGMAX, W.M, W.K, N), x.device)
    _check("q8_0_gemv_argmax", lib().q8_0_gemv_argmax(ctypes.byref(W.desc), x.data_ptr(),
                                                      y.data_ptr(), W.M, W.K, N,
                                                      argmax_out.data_ptr(), wsp, wsb,
                                                      _stream(stream)))
    return y, argmax_out


def q8_0_quantize_act(x: torch.Tensor, qx: torch.Tensor | None = None,
                      dx: torch.Tensor | None = None, stream=None):
    """Integer-activation variant: x [N][K] fp32 -> (qx int8 [N][K], dx
    binary16 bits as int16 [N][K/32]); see q8_0_quantize_act in q8gemv.h."""
    _need(x, torch.float32, "x")
    x2 = x.reshape(1, -1) if x.dim() == 1 else x
    N, K = x2.shape
    if qx is None:
        qx = torch.empty((N, K), dtype=torch.int8, device=x.device)
    if dx is None:
        dx = torch.empty((N, K // 32), dtype=torch.int16, device=x.device)
    _need(qx, torch.int8, "qx")
    _need(dx, torch.int16, "dx")
    if qx.numel() != N * K or dx.numel() != N * (K // 32):
        raise ValueError("qx / dx sizes do not match x")
    _check("q8_0_quantize_act", lib().q8_0_quantize_act(x2.data_ptr(), K, N, qx.data_ptr(),
                                                        dx.data_ptr(), _stream(stream)))
    return qx, dx


def q8_0_gemv_q8act(W: PackedQ8, qx: torch.Tensor, dx: torch.Tensor,
                    y: torch.Tensor | None = None, workspace=None, stream=None) -> torch.Tensor:
    """y[N][M] from packed weights and integer activations (q8_0_quantize_act)."""
    N = _ncols(qx, W.K, "qx")
    if dx.numel() != N * (W.K // 32):
        raise ValueError(f"dx has {dx.numel()} scales, expected {N * (W.K // 32)}")
    if y is not None:
        _room(y, N * W.M, "y")
    _need(qx, torch.int8, "qx")
    _need(dx, torch.int16, "dx")
    if y is None:
        y = torch.empty((N, W.M), dtype=torch.float32, device=qx.device)
    _need(y, torch.float32, "y")
    wsp, wsb = _ws(workspace, q8_0_workspace_bytes(Q8_OP_GEMV, W.M, W.K, N), qx.device)
    _check("q8_0_gemv_q8act", lib().q8_0_gemv_q8act(ctypes.byref(W.desc), qx.data_ptr(),
                                                    dx.data_ptr(), y.data_ptr(), W.M, W.K, N,
                                                    wsp, wsb, _stream(stream)))
    return y


def q8_0_argmax(v: torch.Tensor, out: torch.Tensor | None = None, workspace=None,
                stream=None) -> torch.Tensor:
    if out is not None:
        _room(out, 1, "out")
    _need(v, torch.float32, "v")
    if out is None:
        out = torch.empty(1, dtype=torch.int32, device=v.device)
    _need(out, torch.int32, "out")
    wsp, wsb = _ws(workspace, q8_0_workspace_bytes(Q8_OP_ARGMAX, v.numel(), 0, 0), v.device)
    _check("q8_0_argmax", lib().q8_0_argmax(v.data_ptr(), v.numel(), out.data_ptr(), wsp, wsb,
                                            _stream(stream)))
    return out


def q8_0_route_topk(logits: torch.Tensor, k: int, expert_ids: torch.Tensor | None = None,
                    slot_weights: torch.Tensor | None = None, stream=None):
    if expert_ids is not None:
        _room(expert_ids, k, "expert_ids")
    if slot_weights is not None:
        _room(slot_weights, k, "slot_weights")
    _need(logits, torch.float32, "logits")
    if expert_ids is None:
        expert_ids = torch.empty(k, dtype=torch.int32, device=logits.device)
    if slot_weights is None:
        slot_weights = torch.empty(k, dtype=torch.float32, device=logits.device)
    _need(expert_ids, torch.int32, "expert_ids")
    _need(slot_weights, torch.float32, "slot_weights")
    _check("q8_0_route_topk", lib().q8_0_route_topk(logits.data_ptr(), logits.numel(), k,
                                                    expert_ids.data_ptr(),
                                                    slot_weights.data_ptr(), _stream(stream)))
    return expert_ids, slot_weights


def q8_0_moe_gemv(W_experts: PackedQ8, expert_ids: torch.Tensor, slot_weights, x: torch.Tensor,
                  y: torch.Tensor, mode: int, shared: PackedQ8 | None = None, shared_gate=None,
                  dev_status: torch.Tensor | None = None, workspace=None,
                  stream=None) -> torch.Tensor:
    """All routed-expert slots (and the shared expert) in one launch; see
    q8_0_moe_gemv in include/q8gemv.h for the modes."""
    S = expert_ids.numel()
    base = mode & ~Q8_MOE_SWIGLU
    half = 2 if mode & Q8_MOE_SWIGLU else 1
    if base == Q8_MOE_SCATTER:
        if x.numel() != W_experts.K or (shared is not None and shared.K != W_experts.K):
            raise ValueError(f"scatter reads one x of K = {W_experts.K} entries "
                             f"(x has {x.numel()})")
        _room(y, S * W_experts.M // half + (shared.M // half if shared is not None else 0), "y")
    else:
        want = S * W_experts.K + (shared.K if shared is not None else 0)
        if x.numel() != want:
            raise ValueError(f"combine reads x of {want} entries (x has {x.numel()})")
        _room(y, W_experts.M, "y")
        if slot_weights is not None:
            _room(slot_weights, S, "slot_weights")
        if shared is not None and shared_gate is not None:
            _room(shared_gate, 1, "shared_gate")
    if dev_status is not None:
        _room(dev_status, 1, "dev_status")
    _need(expert_ids, torch.int32, "expert_ids")
    _need(x, torch.float32, "x")
    _need(y, torch.float32, "y")
    if shared is not None:
        M2, K2 = shared.M, shared.K
    else:
        M2, K2 = 0, 0
    op = Q8_OP_MOE_SCATTER if base == Q8_MOE_SCATTER else Q8_OP_MOE_COMBINE
    wsp, wsb = _ws(workspace, q8_0_workspace_bytes(op, W_experts.M, W_experts.K, S, M2, K2, mode),
                   x.device)
    rc = lib().q8_0_moe_gemv(
        ctypes.byref(W_experts.desc), expert_ids.data_ptr(),
        slot_weights.data_ptr() if slot_weights is not None else None,
        x.data_ptr(), y.data_ptr(), W_experts.M, W_experts.K, S, mode,
        ctypes.byref(shared.desc) if shared is not None else None,
        shared_gate.data_ptr() if shared_gate is not None else None,
        dev_status.data_ptr() if dev_status is not None else None, wsp, wsb, _stream(stream))
    _check("q8_0_moe_gemv", rc)
    return y


def q8_0_moe_route_gemv(W_experts: PackedQ8, logits: torch.Tensor, k: int, x: torch.Tensor,
                        y: torch.Tensor, mode: int = Q8_MOE_SCATTER,
                        shared: PackedQ8 | None = None, expert_ids: torch.Tensor | None = None,
                        slot_weights: torch.Tensor | None = None,
                        dev_status: torch.Tensor | None = None, workspace=None, stream=None):
    """The router and the scatter (gate_up) launch of every slot in one launch;
    see q8_0_moe_route_gemv in include/q8gemv.h.  Returns (y, expert_ids,
    slot_weights), the last two written by the launch for the combine."""
    if mode & ~Q8_MOE_SWIGLU != Q8_MOE_SCATTER:
        raise ValueError("the fused router serves the scatter mode only")
    half = 2 if mode & Q8_MOE_SWIGLU else 1
    if x.numel() != W_experts.K or (shared is not None and shared.K != W_experts.K):
        raise ValueError(f"scatter reads one x of K = {W_experts.K} entries (x has {x.numel()})")
    _room(y, k * W_experts.M // half + (shared.M // half if shared is not None else 0), "y")
    if expert_ids is not None:
        _room(expert_ids, k, "expert_ids")
    if slot_weights is not None:
        _room(slot_weights, k, "slot_weights")
    if dev_status is not None:
        _room(dev_status, 1, "dev_status")
    _need(logits, torch.float32, "logits")
    _need(x, torch.float32, "x")
    _need(y, torch.float32, "y")
    if expert_ids is None:
        expert_ids = torch.empty(k, dtype=torch.int32, device=x.device)
    if slot_weights is None:
        slot_weights = torch.empty(k, dtype=torch.float32, device=x.device)
    _need(expert_ids, torch.int32, "expert_ids")
    _need(slot_weights, torch.float32, "slot_weights")
    M2 = shared.M if shared is not None else 0
    K2 = shared.K if shared is not None else 0
    wsp, wsb = _ws(workspace, q8_0_workspace_bytes(Q8_OP_MOE_SCATTER, W_experts.M, W_experts.K,
                                                   k, M2, K2, mode), x.device)
    rc = lib().q8_0_moe_route_gemv(
        ctypes.byref(W_experts.desc), logits.data_ptr(), logits.numel(), expert_ids.data_ptr(),
        slot_weights.data_ptr(), x.data_ptr(), y.data_ptr(), W_experts.M, W_experts.K, k, mode,
        ctypes.byref(shared.desc) if shared is not None else None,
        dev_status.data_ptr() if dev_status is not None else None, wsp, wsb, _stream(stream))
    _check("q8_0_moe_route_gemv", rc)
    return y, expert_ids, slot_weights


# ---------------------------------------------------------------------------
# Persistent decode chain: one launch per decode step
# ---------------------------------------------------------------------------
class ChainStepError(RuntimeError):
    """A persistent decode step whose outputs are invalid (next_token == -1)."""


class PersistentChain:
    """A whole decode step (n_layers Qwen2-style layers + LM head + argmax) in
    one kernel launch; see q8_0_chain_prepare in include/q8gemv.h.  `layers`
    is a list of dicts of PackedQ8 with keys qkv, wo, gate_up (gate/up pairs
    layout) and down; `lm_head` a PackedQ8 or None."""

    def __init__(self, layers: list, lm_head, hidden: int, n_heads: int, n_kv_heads: int,
                 head_dim: int, intermediate: int, eps: float, stream=None):
        n = len(layers)
        self.layers, self.lm_head = layers, lm_head
        arr = lambda k: (q8_0_weights * max(n, 1))(*[L[k].desc for L in layers])
        self._arrays = {k: arr(k) for k in ("qkv", "wo", "gate_up", "down")}
        self._lm = lm_head.desc if lm_head is not None else None
        self.desc = q8_0_chain_desc(
            n, hidden, n_heads, n_kv_heads, head_dim, intermediate,
            lm_head.M if lm_head is not None else 0, eps,
            self._arrays["qkv"], self._arrays["wo"], self._arrays["gate_up"],
            self._arrays["down"], ctypes.pointer(self._lm) if self._lm is not None else None)
        nbytes = int(lib().q8_0_chain_workspace_bytes(ctypes.byref(self.desc)))
        if nbytes == 0:
            raise Q8Error("q8_0_chain_workspace_bytes", Q8_EINVAL)
        dev = layers[0]["qkv"].qs.device if n else lm_head.qs.device
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.plan = q8_0_chain_plan()
        _check("q8_0_chain_prepare",
               lib().q8_0_chain_prepare(ctypes.byref(self.desc), self.ws.data_ptr(), nbytes,
                                        ctypes.byref(self.plan), _stream(stream)))
        self.hidden, self.vocab = hidden, self.desc.vocab

    def run(self, h_in: torch.Tensor, logits: torch.Tensor | None = None,
            next_token: torch.Tensor | None = None, h_out: torch.Tensor | None = None,
            stream=None, check: bool = False, stamps: torch.Tensor | None = None) -> None:
        """One decode step.  With check=True the call waits for the step and
        raises ChainStepError if it was marked invalid (next_token == -1: a
        wait for another workgroup's data expired).  With stamps (device
        int64 [grid * Q8_CHAIN_STAMP_WORDS]) the step also records its stage
        timestamps (q8_0_chain_run_stamped)."""
        if stamps is not None:
            _need(stamps, torch.int64, "stamps")
            _room(stamps, self.plan.grid * Q8_CHAIN_STAMP_WORDS, "stamps")
        _need(h_in, torch.float32, "h_in")
        if h_in.numel() != self.hidden:
            raise ValueError(f"h_in has {h_in.numel()} entries, expected {self.hidden}")
        if h_out is not None and h_out.numel() != self.hidden:
            raise ValueError(f"h_out has {h_out.numel()} entries, expected {self.hidden}")
        if self.vocab:
            if logits is None or next_token is None:
                raise ValueError("a chain with an LM head needs logits and next_token")
            if logits.numel() < self.vocab or next_token.numel() < 1:
                raise ValueError("logits needs vocab entries and next_token one")
        if check and next_token is None:
            raise ValueError("check=True needs next_token")
        for t, name, dt in ((logits, "logits", torch.float32),
                            (next_token, "next_token", torch.int32),
                            (h_out, "h_out", torch.float32)):
            if t is not None:
                _need(t, dt, name)
        ptr = lambda t: t.data_ptr() if t is not None else None
        if stamps is None:
            _check("q8_0_chain_run",
                   lib().q8_0_chain_run(ctypes.byref(self.plan), self.ws.data_ptr(),
                                        h_in.data_ptr(), ptr(h_out), ptr(logits),
                                        ptr(next_token), _stream(stream)))
        else:
            _check("q8_0_chain_run_stamped",
                   lib().q8_0_chain_run_stamped(ctypes.byref(self.plan), self.ws.data_ptr(),
                                                h_in.data_ptr(), ptr(h_out), ptr(logits),
                                                ptr(next_token), stamps.data_ptr(),
                                                _stream(stream)))
        if check:
            s = stream if stream is not None else torch.cuda.current_stream()
            s.synchronize()
            if int(next_token.cpu()[0]) == -1:
                raise ChainStepError(f"decode step invalid: a wait expired "
                                     f"(status {self.status(stream)})")

    def read(self, layer: int, which: int, stream=None) -> torch.Tensor:
        out = torch.empty(self.plan.len[which], dtype=torch.float32, device=self.ws.device)
        _check("q8_0_chain_read",
               lib().q8_0_chain_read(ctypes.byref(self.plan), self.ws.data_ptr(), layer, which,
                                     out.data_ptr(), _stream(stream)))
        return out

    def status(self, stream=None) -> int:
        out = torch.zeros(1, dtype=torch.int32, device=self.ws.device)
        _check("q8_0_chain_status",
               lib().q8_0_chain_status(self.ws.data_ptr(), out.data_ptr(), _stream(stream)))
        return int(out.cpu()[0])
