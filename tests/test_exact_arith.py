"""The page writers' quantizer replaces two IEEE float32 divisions by shorter sequences
(a multiply by the rounded reciprocal of 2^b - 1 with one FMA correction, and the hardware
reciprocal of an fp16 scale with one Newton step).  Both are claimed to return the correctly
rounded result for every input they receive; this runs the check of that claim on the host:
every float32 dividend below 2^-87 and whole binades above it (where the sequence scales
exactly with the dividend's power of two), and every positive finite fp16 scale with any
seed within 2 ulp."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(__file__)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_division_and_reciprocal_sequences_are_correctly_rounded(tmp_path):
    exe = str(tmp_path / "exact_arith_check")
    src = os.path.join(HERE, "exact_arith_check.c")
    flags = ["-O2", "-ffp-contract=off", "-fopenmp"]
    r = subprocess.run(["gcc", *flags, "-mfma", "-o", exe, src, "-lm"], capture_output=True,
                       text=True)
    if r.returncode != 0:      # no FMA instructions to target: libm's fmaf, slower but exact
        r = subprocess.run(["gcc", *flags, "-o", exe, src, "-lm"], capture_output=True,
                           text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout
    assert out.stdout.count(": 0 mismatches") == 4, out.stdout
