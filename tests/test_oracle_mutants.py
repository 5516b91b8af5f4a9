"""The oracle's pins catch planted mistakes.

Each case below plants one plausible mistake (a swapped nibble, a wrong
index, a dropped sign, a wrong rounding rule, a wrong offset or divisor) in a
copy of the oracle's C source, builds that copy into a temporary library,
and runs the pin tests (tests/test_oracle_pins.py) against it in a child
process. Every mutant must make a pin fail, and the unmodified source, built
the same way, must pass. The cases cover each format's layout reading
(Q8_0, Q4_K, Q4_0, Q5_0, Q6_K and the Q8K activation blocks), the
quantizers' rules, the f16 conversion, and both products.

CPU only: gcc and the pin suite, nothing on the GPU.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

import pytest

from oracle import build as oracle_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (what the mistake is, exact text in the oracle's source, the mistaken text)
MUTANTS = [
    ("Q4_K: 6-bit scale high bits from the wrong byte",
     "*sc = (s[j + 4] & 0x0f) | ((s[j - 4] >> 6) << 4);",
     "*sc = (s[j + 4] & 0x0f) | ((s[j] >> 6) << 4);"),
    ("Q4_K: low and high nibble swapped",
     "return l < 32 ? (byte & 0x0f) : (byte >> 4);",
     "return l < 32 ? (byte >> 4) : (byte & 0x0f);"),
    ("quantizers: ties to even everywhere",
     "return even ? (int)rintf(t) : (int)roundf(t);",
     "return (int)rintf(t);"),
    ("Q4_K mode (b): sign of the mins term",
     "acc += dx * (d * (double)s[i * 10 + 8] - dmin * (double)s[i * 10 + 9]);",
     "acc += dx * (d * (double)s[i * 10 + 8] + dmin * (double)s[i * 10 + 9]);"),
    ("Q8K quantizer: the last of equal magnitudes sets the scale",
     "j < QK_K; ++j) {\n                float a = fabsf(v[j]);\n                if (a > amax)",
     "j < QK_K; ++j) {\n                float a = fabsf(v[j]);\n                if (a >= amax)"),
    ("signed maximum (Q4_0, Q5_0, Q6_K): the last of equal magnitudes wins",
     "j < n; ++j) {\n        float a = fabsf(v[j]);\n        if (a > amax)",
     "j < n; ++j) {\n        float a = fabsf(v[j]);\n        if (a >= amax)"),
    ("Q8K: group sums read from the wrong slot",
     "int16_t b1 = (int16_t)rd16(xb + 260 + 2 * (2 * j + 1));",
     "int16_t b1 = (int16_t)rd16(xb + 260 + 2 * (2 * j));"),
    ("Q8_0: scale divides by 128",
     "float d = amax / 127.0f;",
     "float d = amax / 128.0f;"),
    ("f16 conversion: ties rounded up",
     "if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1u;",
     "if (rem >= 0x1000u) h += 1u;"),
    ("mode (a): weight row read backwards",
     "double p = (double)x[m * K + k] * wr[k];",
     "double p = (double)x[m * K + k] * wr[K - 1 - k];"),
    ("Q6_K: low bits without the 32-byte step of odd groups",
     "*lo_byte = 64 * half + 32 * (g & 1) + l;",
     "*lo_byte = 64 * half + l;"),
    ("Q6_K: high bits from the neighbouring byte",
     "*hi_byte = 128 + 32 * half + l;",
     "*hi_byte = 128 + 32 * half + (l ^ 1);"),
    ("Q6_K: bit pairs in reverse order",
     "*pair = g;",
     "*pair = 3 - g;"),
    ("Q6_K: nibble chosen by the wrong bit of the group",
     "*nib = g >> 1;",
     "*nib = g & 1;"),
    ("Q6_K: one scale per 32 values",
     "out[b * QK_K + e] = d * (double)(int8_t)blk[192 + e / 16]",
     "out[b * QK_K + e] = d * (double)(int8_t)blk[192 + e / 32]"),
    ("Q5_0: fifth bits in reverse order",
     "return lo | (int)(((qh >> j) & 1u) << 4);",
     "return lo | (int)(((qh >> (31 - j)) & 1u) << 4);"),
    ("Q4_0 / Q5_0: low and high nibble swapped",
     "return j < 16 ? (blk[2 + j] & 15) : (blk[2 + j - 16] >> 4);",
     "return j < 16 ? (blk[2 + j] >> 4) : (blk[2 + j - 16] & 15);"),
    ("Q4_0 / Q5_0 quantizer: truncation without the half",
     "t = t + (off + 0.5f);",
     "t = t + off;"),
    ("Q4_0 / Q5_0 quantizer: sign of the scale",
     "float d = mx / -off;",
     "float d = mx / off;"),
    ("Q6_K mode (b): offset 31",
     "for (int l = 0; l < 16; ++l) s += (int64_t)(q6k_value(wb, 16 * j + l) - 32) * q8[16 * j + l];",
     "for (int l = 0; l < 16; ++l) s += (int64_t)(q6k_value(wb, 16 * j + l) - 31) * q8[16 * j + l];"),
    ("Q6_K mode (b): scales read unsigned",
     "sumi += (int64_t)(int8_t)wb[192 + j] * s;",
     "sumi += (int64_t)wb[192 + j] * s;"),
    ("Q5_0 paired with Q8K activations",
     "return (wfmt == ORC_Q8_0 || wfmt == ORC_Q4_0 || wfmt == ORC_Q5_0) ? ORC_Q8_0 : ORC_Q8_K;",
     "return (wfmt == ORC_Q8_0 || wfmt == ORC_Q4_0) ? ORC_Q8_0 : ORC_Q8_K;"),
    ("Q6_K mode (b): last scaled sum taken for the total",
     "acc += dx * d * (double)s[i * 17 + 16];",
     "acc += dx * d * (double)s[i * 17 + 15];"),
    ("Q6_K quantizer: scale divides by 127",
     "float d = smax / -128.0f;",
     "float d = smax / -127.0f;"),
    ("Q4_0 / Q5_0 quantizer: overflow sent to zero",
     "if (q > qmax) q = qmax;",
     "if (q > qmax) q = 0;"),
]


def _source() -> str:
    with open(oracle_build.SRC) as f:
        return f.read()


def _run_pins(src_text: str, tag: str, tmp: str) -> tuple[int, str]:
    """Build `src_text` as an oracle library and run the pins against it."""
    src = os.path.join(tmp, f"oracle_{tag}.c")
    lib = os.path.join(tmp, f"liboracle_{tag}.so")
    with open(src, "w") as f:
        f.write(src_text)
    oracle_build.build(src=src, out=lib)
    env = dict(os.environ, QMM_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run(
        [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"),
         "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr).strip().splitlines()
    return r.returncode, tail[-1] if tail else ""


def test_every_mutant_applies_once():
    src = _source()
    for what, old, new in MUTANTS:
        assert src.count(old) == 1, f"{what}: text not found exactly once"
        assert old != new


def test_pins_catch_planted_mistakes(tmp_path):
    src = _source()
    rc, tail = _run_pins(src, "unmodified", str(tmp_path))
    assert rc == 0, f"the unmodified oracle fails its pins when built apart: {tail}"

    def one(i):
        what, old, new = MUTANTS[i]
        return what, _run_pins(src.replace(old, new), f"m{i}", str(tmp_path))

    missed, broken = [], []
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        for what, (rc, tail) in ex.map(one, range(len(MUTANTS))):
            if rc == 0:
                missed.append(what)
            elif not (rc == 1 or rc < 0):  # 1: a pin failed; < 0: the mutant crashed
                broken.append(f"{what}: pytest exit {rc}: {tail}")
    assert not broken, "mutant runs did not complete: " + "; ".join(broken)
    assert not missed, "pins passed with a planted mistake: " + "; ".join(missed)
