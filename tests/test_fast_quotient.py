"""The reciprocal quotient of the bf16 quantisation kernels is exact.

The kernels replace the IEEE division x / s of the per-token quantisation
("Qwen3.6-27B-Quark-W8A8-INT8" model card, Quantization Scheme; codes
round to nearest) by a reciprocal and one fused correction step.  bf16 inputs
make the domain finite, so the claim that the rounded code never changes is
checked for every (x, row maximum) pair, in C with IEEE fp32 and fmaf.  The
kernels read the code off fl(q + 1.5 * 2^23) with no clamp (the quotient stays
within +-127.5 here); that is checked against the clamped rint for x and -x.
"""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_reciprocal_quotient_matches_ieee_division_on_all_bf16(tmp_path):
    exe = str(tmp_path / "fast_quotient_check")
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-o", exe,
                           os.path.join(HERE, "fast_quotient_check.c"), "-lm"])
    out = subprocess.check_output([exe], timeout=600).decode().split()
    pairs, bad, bad_product, bad_code = (int(v) for v in out)
    assert pairs > 500_000_000
    assert bad == 0
    assert bad_code == 0
    # the check is sharp enough to see the error of the bare product
    assert bad_product > 0
