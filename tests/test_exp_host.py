"""The selector's fp64 exponential (csrc/rtp_exp.h), compiled for the host
with g++ and checked against the C library's long-double expl: the table
2^(j/256) correctly rounded, and the function within 1.5 ulp of the exact
value for normal results (subnormal results within 1.5 subnormal ulps)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_long_context_indexer_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "native", "exp_check.cpp")


def test_exp_tang_against_expl(tmp_path):
    exe = str(tmp_path / "exp_check")
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-I", CSRC, SRC,
                           "-o", exe, "-lm"])
    out = subprocess.check_output([exe], text=True)
    vals = dict(line.split() for line in out.strip().splitlines())
    assert float(vals["table_max_ulp"]) <= 0.5
    assert float(vals["normal_max_ulp"]) <= 1.5, out
    assert float(vals["subnormal_max_ulp"]) <= 1.5, out
    assert vals["specials_ok"] == "1"
