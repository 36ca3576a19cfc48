"""The table-driven fp64 exp of the bulk FFN quantizer (SwiGLU's e^-g; common.hpp) against the
host library's exp on the CPU: within 3 ulps over the normal range (2 measured; the parity
tests accept an fp32 difference of h only within 16 fp64 ulps of a tie), and the same zeros,
infinities and NaN at the ends of the range.  Built with hipcc for the host."""

import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_exp_tab_against_host_library(tmp_path):
    exe = str(tmp_path / "exp_tab_check")
    src = os.path.join(HERE, "host", "exp_tab_check.hip")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-ffp-contract=off",
                    src, "-o", exe], check=True, capture_output=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    vals = dict(line.split(" ", 1) for line in out.strip().splitlines() if " " in line)
    assert int(vals["kind_mismatches"]) == 0, out
    assert float(vals["max_ulps"].split()[0]) <= 3.0, out
