"""Mutation check of the oracle pins (CPU only).

Each mutant is a copy of the oracle source with one plausible mistake planted
(a dropped term, a wrong sign, index or byte order, a wrong tie rule, a
missing renormalisation ...).  The copy is compiled to a temporary library and
the pin checks are re-run against it in a subprocess; at least one pin must
fail for every mutant.  The real oracle source is never modified.
"""
import concurrent.futures as cf
import json
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "q8_oracle.c")

MUTANTS = {
    "f16_exponent_bias": ("e - 25)", "e - 24)"),
    "f16_subnormal_flush": ("ldexp((double)m, -24)", "0.0 * m"),
    "f16_implicit_bit": ("ldexp((double)(1024 + m)", "ldexp((double)(1023 + m)"),
    "f16_sign_dropped": ("return s ? -v : v;", "return v;"),
    "f16_byte_order": ("blk[0] | (blk[1] << 8)", "blk[1] | (blk[0] << 8)"),
    "scale_wrong_block": ("(r * nb + k / QK)", "(r * nb + (k / QK + 1) % nb)"),
    "quant_offset": ("blk[2 + k % QK]", "blk[1 + k % QK]"),
    "quant_unsigned": ("oracle_f16_to_f64(dbits) * (double)q;", "oracle_f16_to_f64(dbits) * (double)(uint8_t)q;"),
    "last_block_dropped": ("for (int64_t k = 0; k < j->K; ++k) {",
                           "for (int64_t k = 0; k < j->K - QK; ++k) {"),
    "magnitude_signed": ("mag += fabs(p);", "mag += p;"),
    "x_wrong_column": ("* xn[k];", "* j->x[k];"),
    "argmax_last_tie": ("if (v[i] > v[best]) best = i;\n  return best;\n}\n\nint64_t oracle_argmax_f64",
                        "if (v[i] >= v[best]) best = i;\n  return best;\n}\n\nint64_t oracle_argmax_f64"),
    "router_tie_high": ("logits[e] > logits[best]", "logits[e] >= logits[best]"),
    "router_not_renormalised": ("w[s] = exp((double)logits[ids[s]] - lmax) / den;",
                                "w[s] = exp((double)logits[ids[s]] - lmax) / (den + 1.0);"),
    "silu_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "rmsnorm_no_mean": ("sqrt(ss / (double)n + eps)", "sqrt(ss + eps)"),
    "gqa_interleaved": ("v[(int64_t)(h / group) * head_dim + j]",
                        "v[(int64_t)(h % n_kv_heads) * head_dim + j]"),
    "moe_slot_weight": ("y[r] += w[s] * t[r];", "y[r] += w[0] * t[r];"),
    "moe_gate_up_swapped": ("oracle_swiglu(gu, gu + I, I, hr + s * I);",
                            "oracle_swiglu(gu + I, gu, I, hr + s * I);"),
    "moe_gamma_dropped": ("y[r] += gamma * t[r];", "y[r] += t[r];"),
    "layer_residual_dropped": ("for (int64_t i = 0; i < hidden; ++i) h[i] += t[i];\n  oracle_rmsnorm",
                               "for (int64_t i = 0; i < hidden; ++i) h[i] = t[i];\n  oracle_rmsnorm"),
    "layer_v_offset": ("qkv + qdim + kvdim,", "qkv + qdim,"),
    "act_divisor_128": ("const float d = amax / 127.0f;", "const float d = amax / 128.0f;"),
    "act_round_floor": ("q = nearbyintf(xb[j] / d);", "q = floorf(xb[j] / d);"),
    "act_amax_signed": ("const float a = fabsf(xb[j]);", "const float a = xb[j];"),
    "act_f16_truncated": ("double frac = nearbyint((2.0 * m - 1.0) * 1024.0);",
                          "double frac = floor((2.0 * m - 1.0) * 1024.0);"),
    "act_dot_column0": ("(int64_t)qx[n * K + b * QK + j];", "(int64_t)qx[b * QK + j];"),
    "act_weight_unsigned": ("(int64_t)(int8_t)blk[2 + j] *", "(int64_t)blk[2 + j] *"),
    "q4k_scale_min_swapped": ("*sj = sc[j] & 63;\n    *mj = sc[j + 4] & 63;",
                              "*sj = sc[j + 4] & 63;\n    *mj = sc[j] & 63;"),
    "q4k_high_bits_wrong_byte": ("16 * (sc[j - 4] >> 6);", "16 * (sc[j] >> 6);"),
    "q4k_high_bits_unshifted": ("+ 16 * (sc[j] >> 6);", "+ (sc[j] >> 6);"),
    "q4k_nibble_swapped": ("(byte & 15) : (byte >> 4);", "(byte >> 4) : (byte & 15);"),
    "q4k_group_stride": ("b[16 + 32 * (kk / 64) + kk % 32]", "b[16 + 32 * (kk / 64) + kk % 16]"),
    "q4k_min_sign": ("- dmin * (double)mj;", "+ dmin * (double)mj;"),
    "q4k_d_dmin_swapped": ("(uint16_t)(b[0] | (b[1] << 8)));\n  *dmin",
                           "(uint16_t)(b[2] | (b[3] << 8)));\n  *dmin"),
    "q5k_fifth_bit_index": ("const int fifth = (b[16 + kk % 32] >> j) & 1;",
                            "const int fifth = (b[16 + kk % 32] >> (j / 2)) & 1;"),
    "q5k_fifth_weight": ("(double)(low + 16 * fifth)", "(double)(low + 32 * fifth)"),
    "q5k_qs_offset": ("byte5 = b[48 + 32 * (kk / 64) + kk % 32]", "byte5 = b[16 + 32 * (kk / 64) + kk % 32]"),
    "q5k_nibble_swapped": ("(byte5 & 15) : (byte5 >> 4);", "(byte5 >> 4) : (byte5 & 15);"),
    "q5k_min_sign": ("- dmin * (double)m5;", "+ dmin * (double)m5;"),
    "q5k_wrong_subblock": ("const int j = kk / 32; /* sub-block */",
                           "const int j = kk / 64; /* sub-block */"),
    "q5k_qh_byte": ("(b[16 + kk % 32] >> j)", "(b[16 + kk % 16] >> j)"),
    "q6k_nibble_swapped": ("const int low = (a < 2) ? (lb & 15) : (lb >> 4);",
                           "const int low = (a < 2) ? (lb >> 4) : (lb & 15);"),
    "q6k_high_shift": (">> (2 * a)) & 3;", ">> a) & 3;"),
    "q6k_offset_dropped": ("const int q = low + 16 * high - 32;", "const int q = low + 16 * high;"),
    "q6k_high_weight": ("const int q = low + 16 * high - 32;", "const int q = low + 4 * high - 32;"),
    "q6k_scale_group_32": ("b[192 + kk / 16]", "b[192 + kk / 32]"),
    "q6k_scale_unsigned": ("const int sc = (int8_t)b[192 + kk / 16];",
                           "const int sc = (uint8_t)b[192 + kk / 16];"),
    "q6k_ql_half_dropped": ("b[64 * h + 32 * (a % 2) + l]", "b[64 * h + l]"),
    "q6k_d_offset": ("(uint16_t)(b[208] | (b[209] << 8))", "(uint16_t)(b[207] | (b[208] << 8))"),
    "q4k_wrong_subblock": ("const int kk = (int)(k % QKK), j = kk / 32;",
                           "const int kk = (int)(k % QKK), j = (kk / 32) ^ 1;"),
}

RUNNER = r"""
import json, sys, traceback
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle_pins as P
failed = []
for c in P.ALL_CHECKS:
    try:
        c()
    except Exception as e:
        failed.append(c.__name__)
print(json.dumps(failed))
"""


def _run_mutant(name, tmp):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/found"
    path = os.path.join(tmp, f"{name}.c")
    lib = os.path.join(tmp, f"lib_{name}.so")
    open(path, "w").write(src.replace(old, new))
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", lib, path, "-lm",
                    "-lpthread"], check=True, capture_output=True)
    env = dict(os.environ, Q8_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    code = RUNNER.format(root=ROOT, tests=os.path.join(ROOT, "tests"))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=600)
    if r.returncode != 0:  # a crash also counts as caught, but report it
        return name, ["<crashed>"]
    return name, json.loads(r.stdout.strip().splitlines()[-1])


def test_every_mutant_is_caught():
    with tempfile.TemporaryDirectory() as tmp:
        with cf.ThreadPoolExecutor(max_workers=4) as ex:
            results = dict(ex.map(lambda n: _run_mutant(n, tmp), MUTANTS))
    missed = [n for n, f in results.items() if not f]
    assert not missed, f"mutants not caught by any pin: {missed}"
