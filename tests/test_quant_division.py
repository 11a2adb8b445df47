"""The pack kernel's per-element division identity, checked exhaustively on
the CPU.

Codes are rint(fl32(x / s)) (SpectrumKV Algorithm 1 "transfer", symmetric
absmax quantization computed from the stored fp16 scale).  The kernel
replaces the division by a reciprocal and one fused correction step
(q0 = x r, e = fma(-q0, s, x), q1 = fma(e, r, q0) with r = fl32(1 / s)); the
codes are bit-exact only if q1 equals the correctly rounded quotient for
every pair the quantizer can meet.  The row's scale needs two more
divisions, done the same way: fl32(a / qmax) by a multiply and one fused
correction, and fl32(1 / s) by one Newton step from the hardware
reciprocal, which lies within one ulp of 1 / s; both are checked for every
fp16 input (and every start within one ulp).  tests/native/quant_div_check.c checks
that over every positive fp16 scale and every fp16 x with |x / s| <= 300,
both signs (1.47e9 pairs, about a second on 8 cores), with the IEEE binary32
arithmetic of the C compiler (no contraction, no fast math) and the C
library's correctly rounded fmaf."""

import os
import shutil
import subprocess

import pytest

SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "quant_div_check.c")
PAIRS = 1469703037      # 734,851,519 non-negative x plus as many negative, over 31,743 scales


def _build(tmp_path, *defines):
    gcc = shutil.which("gcc") or shutil.which("cc")
    if gcc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path / "quant_div_check")
    base = [gcc, "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", *defines, SRC,
            "-o", exe, "-lm"]
    r = subprocess.run(base[:1] + ["-fopenmp"] + base[1:], capture_output=True, text=True)
    if r.returncode != 0:                       # no OpenMP: the same check, one thread
        r = subprocess.run(base, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


SCALE_CHECKS = 158717   # 2 x 31,744 values of a, plus 3 x 31,743 reciprocal starts


def _run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    fields = dict(kv.split("=") for kv in r.stdout.strip().splitlines()[-1].split())
    return r.returncode, {k: int(v) for k, v in fields.items()}, r.stdout


def test_reciprocal_correction_equals_division_on_every_pair(tmp_path):
    rc, f, out = _run(_build(tmp_path))
    assert f["pairs"] == PAIRS and f["scale_checks"] == SCALE_CHECKS, out
    assert rc == 0 and f["mismatches"] == 0 and f["scale_mismatches"] == 0, out


def test_checker_fails_without_the_correction_step(tmp_path):
    rc, f, out = _run(_build(tmp_path, "-DDROP_CORRECTION"))
    assert f["pairs"] == PAIRS and f["scale_checks"] == SCALE_CHECKS
    assert rc == 1 and f["mismatches"] > 0 and f["scale_mismatches"] > 0, out
