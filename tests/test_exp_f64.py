"""Accuracy of the fp64 exponential the sampling kernels use for masses
(csrc/exp_f64.h, Tang's table-driven method), built for the host from the
same header: at most 1.5 units in the last place against extended-precision
expl over 3.2 million arguments (the derived bound: half an ulp from the
2^(j/32) table, half from the final fma, the polynomial's remainder below
4e-18), and the special values; the variant for arguments <= 0 equals it
bit for bit there and reaches 0 by itself below -746. The masses' parity tolerance (a relative
1e-9 between the two sides' cumulative shares) rests on this."""
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent


def test_exp_table_is_within_its_error_bound(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    exe = tmp_path / "exp_check"
    subprocess.run([gxx, "-O2", "-std=c++17", "-ffp-contract=off", "-I", str(ROOT / "paged_kv_cache_17_amd" / "csrc"),
                    str(ROOT / "tests" / "native" / "exp_check.cpp"), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    fig = dict(line.split(" ", 1) for line in out.strip().splitlines())
    assert int(fig["checked"]) > 3_000_000
    assert float(fig["max_ulp"]) <= 1.5, out
    assert fig["special"] == "1", out
    assert fig["nonpos_mismatch"] == "0", out
