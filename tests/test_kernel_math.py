"""Exhaustive CPU proof of the arithmetic shortcuts the gfx950 kernels take:
division by the grid's largest code via one FMA correction, the binary16
reciprocal via one Newton step from any estimate within 2 ulp, and
round-to-nearest-even via the 1.5 * 2^23 magic number after clamping.
(The kernels themselves are checked against the oracle on the GPU.)"""
import os
import subprocess
import tempfile

SRC = os.path.join(os.path.dirname(__file__), "kernel_math_check.c")


def test_kernel_arithmetic_identities():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "kmc")
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                               "-o", exe, SRC, "-lm"])
        r = subprocess.run([exe], capture_output=True, text=True, timeout=900)
    print(r.stdout)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), r.stdout
