"""Exhaustive host checks of two pieces of the write kernel's arithmetic,
compiled with gcc (hardware fma) and run on the CPU: the value-code rule
(vquot_row / quant_v) and the scale division by 448 (div448).  They check
the device's algorithms, not the oracle; the GPU tests check the device's
results against the oracle."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "host")


def run_c(name, timeout):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, name)
        subprocess.run([gcc, "-O2", "-mfma", "-o", exe, os.path.join(HERE, name + ".c"), "-lm"], check=True)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=timeout)
    return r


def test_value_code_rule_is_exact_rne():
    r = run_c("vquant_exhaustive", 120)
    assert r.returncode == 0, r.stdout
    assert "mismatches r=RN 0 r-1ulp 0 r+1ulp 0" in r.stdout, r.stdout


def test_div448_equals_the_division():
    r = run_c("div448_exhaustive", 300)
    assert r.returncode == 0, r.stdout
    assert " 0 of " in r.stdout, r.stdout
