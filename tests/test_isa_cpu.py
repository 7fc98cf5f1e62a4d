"""Checks on the gfx950 assembly of the HIP kernels (CPU only: hipcc
cross-compiles, nothing runs).

* The GEMV's inner loop is inline assembly: v_fmac_f32_dpp with a
  row_newbcast source.  A DPP source VGPR written by a VALU instruction needs
  two wait states before the DPP read, and the compiler does not look inside
  inline assembly for that hazard.  The kernels are written so that DPP
  sources are only produced by memory loads; this test scans the generated
  code to hold them to it (every DPP instruction, compiler-made ones too).
* The integer-activation GEMV chains v_dot4c_i32_i8 in inline assembly; a
  dot result read by another VALU instruction needs three wait states,
  which the compiler does not see through the asm.  The scan holds every
  dot (compiler-made ones too) to that.
* Matrix cores appear in one place only: the GEMV at five or more columns
  runs each block as v_mfma_f32_16x16x32_bf16 products (bf16 parts of the
  activations, exact int8 weights).  No other MFMA instruction may appear in
  gemv.hip, and none at all in the other units (the decode chain, the
  argmax, the repack).
"""
import os
import re
import shutil
import subprocess

import pytest

from block_quantized_gemv_amd import build as B

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not installed")

UNITS = ["gemv.hip", "chain.hip", "select.hip", "repack.hip"]


def device_asm(name: str, tmp_path) -> list[str]:
    out = os.path.join(tmp_path, name + ".s")
    cmd = ["hipcc", f"--offload-arch={B.ARCH}", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I", B.INCLUDE, "-I", B.CSRC, "--cuda-device-only",
           "-S", "-o", out, os.path.join(B.CSRC, name)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as f:
        return f.read().splitlines()


def vregs(op: str) -> set:
    op = op.strip()
    m = re.match(r"v\[(\d+):(\d+)\]$", op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", op)
    return {int(m.group(1))} if m else set()


def instructions(lines):
    """(kind, text) in program order: kind 'L' for a label, 'I' otherwise."""
    out = []
    for raw in lines:
        t = raw.split(";")[0].strip()
        if not t or t.startswith("."):
            continue
        out.append(("L" if t.endswith(":") else "I", t))
    return out


def dpp_hazards(insts):
    """Return (n_dpp, problems): a problem is a VALU write of a DPP source
    register, or a branch target, within the two wait states before the DPP
    instruction (s_nop k counts k + 1)."""
    n, bad = 0, []
    for i, (kind, t) in enumerate(insts):
        if kind != "I" or "_dpp" not in t.split()[0]:
            continue
        n += 1
        src = vregs(t.split(None, 1)[1].split(",")[1])
        ws, j = 0, i - 1
        while j >= 0 and ws < 2:
            kj, tj = insts[j]
            if kj == "L":
                bad.append(f"label before {t}")
                break
            mn = tj.split()[0]
            if mn == "s_nop":
                ws += int(tj.split()[1], 0) + 1
            else:
                if mn.startswith("v_") and len(tj.split()) > 1:
                    if vregs(tj.split(None, 1)[1].split(",")[0]) & src:
                        bad.append(f"{tj} -> {t}")
                ws += 1
            j -= 1
    return n, bad


def dot_result_hazards(insts):
    """Return (n_dot, problems): a problem is a VALU instruction that reads
    the result of a v_dot* within the three wait states after it (another
    dot of the same opcode accumulating into that register excepted), or a
    label inside that window."""
    n, bad = 0, []
    for i, (kind, t) in enumerate(insts):
        if kind != "I" or not t.split()[0].startswith("v_dot"):
            continue
        n += 1
        op = t.split()[0]
        dst = vregs(t.split(None, 1)[1].split(",")[0])
        ws, j = 0, i + 1
        while j < len(insts) and ws < 3:
            kj, tj = insts[j]
            if kj == "L":
                bad.append(f"label after {t}")
                break
            mn = tj.split()[0]
            if mn == "s_nop":
                ws += int(tj.split()[1], 0) + 1
            else:
                if mn.startswith("v_") and len(tj.split()) > 1:
                    ops = tj.split(None, 1)[1].split(",")
                    same_acc = mn == op and vregs(ops[0]) == dst
                    reads = set().union(*(vregs(o.split()[0]) for o in ops[1:] if o.strip()))
                    if not same_acc and (reads & dst or (mn.endswith("c") or "fmac" in mn)
                                         and vregs(ops[0]) & dst):
                        bad.append(f"{t} -> {tj}")
                ws += 1
            j += 1
    return n, bad


def test_dot_scanner_finds_planted_hazards():
    """A conversion reading a dot result one instruction later is flagged;
    after s_nop 2, or as the next dot's accumulator, it is not."""
    dot = "v_dot4c_i32_i8_dpp v15, v66, v5 row_newbcast:15 row_mask:0xf bank_mask:0xf"
    bad_code = [dot, "v_mul_f32_e32 v5, v10, v20", "v_cvt_f32_i32_e32 v4, v15"]
    ok_code = [dot, "s_nop 2", "v_cvt_f32_i32_e32 v4, v15"]
    chain = [dot, "v_dot4c_i32_i8_dpp v15, v66, v6 row_newbcast:14 row_mask:0xf bank_mask:0xf",
             "s_nop 2", "v_cvt_f32_i32_e32 v4, v15"]
    acc_code = [dot, "v_fmac_f32_e32 v15, v1, v2"]
    assert len(dot_result_hazards(instructions(bad_code))[1]) == 1
    assert dot_result_hazards(instructions(ok_code))[1] == []
    assert dot_result_hazards(instructions(chain))[1] == []
    assert len(dot_result_hazards(instructions(acc_code))[1]) == 1


def test_hazard_scanner_finds_planted_hazards():
    """The scanner itself: a VALU write of the DPP source right before the
    read is flagged, one covered by s_nop 1 is not."""
    bad_code = ["v_mov_b32_e32 v4, v9", "v_fmac_f32_dpp v12, v4, v11 row_newbcast:0"]
    ok_code = ["v_mov_b32_e32 v4, v9", "s_nop 1", "v_fmac_f32_dpp v12, v4, v11 row_newbcast:0"]
    far_code = ["v_mov_b32_e32 v4, v9", "v_add_f32_e32 v1, v2, v3", "v_add_f32_e32 v1, v2, v3",
                "v_fmac_f32_dpp v12, v4, v11 row_newbcast:0"]
    range_code = ["v_mov_b32_e32 v[4:5], v[8:9]", "v_fmac_f32_dpp v12, v5, v11 row_newbcast:0"]
    assert len(dpp_hazards(instructions(bad_code))[1]) == 1
    assert dpp_hazards(instructions(ok_code))[1] == []
    assert dpp_hazards(instructions(far_code))[1] == []
    assert len(dpp_hazards(instructions(range_code))[1]) == 1


@pytest.mark.parametrize("unit", UNITS)
def test_kernel_assembly(unit, tmp_path):
    lines = device_asm(unit, str(tmp_path))
    insts = instructions(lines)
    n, bad = dpp_hazards(insts)
    assert bad == [], f"{unit}: {len(bad)} DPP source hazards, first: {bad[:3]}"
    if unit == "gemv.hip":
        assert n > 0, "the GEMV inner loop should use DPP row-broadcast FMAs"
    nd, badd = dot_result_hazards(insts)
    assert badd == [], f"{unit}: {len(badd)} dot result hazards, first: {badd[:3]}"
    if unit == "gemv.hip":
        assert nd > 0, "the integer-activation GEMV should use v_dot4c"
    mfma = [t.split()[0] for k, t in insts if k == "I" and t.split()[0].startswith("v_mfma")]
    if unit == "gemv.hip":
        assert mfma, "the GEMV at N >= 5 should use matrix-core products"
        assert set(mfma) == {"v_mfma_f32_16x16x32_bf16"}, sorted(set(mfma))
    else:
        assert mfma == [], f"{unit}: matrix-core instructions found: {mfma[:3]}"
