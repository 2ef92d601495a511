"""Host-side pin of an arithmetic shortcut in the int8 quantiser (no GPU).

The quantise kernel forms the per-row scale max|x| / 127 without a division:
one product with the rounded reciprocal of 127 and one fused correction step.
It is only valid if that equals the IEEE quotient for every input the kernel
can see, so a small C program compares the two over the fp32 bit patterns
(a strided sample here; stride 1 in KDA_DIV127_STRIDE=1 runs all 2^31 - 2^23
non-negative finite values, which has been done with zero mismatches).  The
kernel's element codes use a reciprocal only where the result provably
matches, and fall back to the division elsewhere; that part is exercised
bit for bit against the oracle by the GPU test at rounding ties."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_division_free_scale_matches_ieee(tmp_path):
    exe = tmp_path / "div127_check"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", str(exe), os.path.join(HERE, "div127_check.c"),
                    "-lm"], check=True)
    stride = os.environ.get("KDA_DIV127_STRIDE", "257")
    r = subprocess.run([str(exe), stride], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout
    assert " 0 mismatches" in r.stdout, r.stdout
