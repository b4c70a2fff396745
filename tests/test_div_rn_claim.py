"""The dynamic-quantization kernels replace a division per value by one
reciprocal per group and Markstein's FMA correction (P. Markstein, IBM J.
Res. Dev. 34(1), 1990).  This test compiles a C restatement of that scheme
and checks, on a sample of group maxima and every 16-bit input within them,
that it reproduces the correctly rounded binary32 quotient the oracle
computes (the GPU parity tests compare the kernels' codes with the oracle's
bit for bit)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("fp16", [0, 1])
def test_fma_corrected_quotient_is_correctly_rounded(tmp_path, fp16):
    exe = tmp_path / "div_rn_check"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", os.path.join(HERE, "c", "div_rn_check.c"),
                    "-o", str(exe), "-lm"], check=True)
    out = subprocess.run([str(exe), "61", str(fp16)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    checked = int(out.stdout.split()[1])
    assert checked > 10_000_000 and out.stdout.split()[3] == "0"
