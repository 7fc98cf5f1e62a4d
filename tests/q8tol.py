"""Parity tolerance of the Q8_0 GEMV against the fp64 oracle.

Per output: |y_gpu - y_ref| <= 2e-5 * S + 1e-6 with S = sum_k |w_k x_k| (the
oracle's magnitude sum).  An fp32 schedule in which every product passes
through at most D roundings has error <= D * 2^-24 * S (to first order), so
any schedule with D below ~335 passes by construction.  In the GEMV kernels a
product passes through at most 32 (the FMAs of its block) + 1 (the block's
scale) + 64 (the blocks of one unit: the planner gives a unit at most 16 scale
quads) + 8 + 8 + ceil(units / 64) (the fixed three-level fold of a tile's unit
partials) + 2 (segment weight and epilogue) roundings.  Units per tile never
exceed K / 128, so D <= 115 + K / 8192, below 250 for every K the boundary
accepts (K <= 2^20).
"""
import numpy as np

REL = 2e-5
ABS = 1e-6


def bound(S):
    return REL * np.asarray(S, dtype=np.float64) + ABS


def check(y_gpu, y_ref, S, what=""):
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    err = np.abs(y_gpu - y_ref)
    b = bound(S)
    ratio = err / b
    worst = float(ratio.max()) if ratio.size else 0.0
    bad = np.argwhere(~(err <= b))
    assert bad.size == 0, (f"{what}: {bad.shape[0]} outputs out of tolerance; first at "
                           f"{tuple(bad[0])}: gpu={y_gpu[tuple(bad[0])]!r} "
                           f"ref={y_ref[tuple(bad[0])]!r} bound={b[tuple(bad[0])]!r}")
    return worst
