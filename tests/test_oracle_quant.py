"""Pins for the oracle's per-row int8 quantisation (O1 / O2).

What pins it (none of these re-types the oracle's formula):
  - hand-derived worked cases (tests/golden/quant_worked.txt);
  - brute force: every code is the integer in [-127, 127] nearest to x/scale,
    ties to even, found by enumerating all 255 candidates;
  - invariants: |x - q*s| <= s/2 (plus rounding of x/s), the amax element maps
    to +-127, quant(2^j x) = (q, 2^j s) exactly, quant(-x) = (-q, s), a
    permutation of the row permutes the codes.
Source: "Qwen3.6-27B-Quark-W8A8-INT8" model card, Quantization Scheme table
(per-token / per-channel symmetric INT8); "Qwen3.6-35B-A3B IQ8R - radiance
container", Trunk row (codes -127..127, round to nearest).
"""
import os

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quant_worked.txt")


def _golden_cases():
    cases = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        xs, s, qs = (part.split() for part in line.split("|"))
        cases.append((np.array([float(v) for v in xs], np.float32), float(s[0]),
                      np.array([int(v) for v in qs], np.int8)))
    return cases


@pytest.mark.parametrize("case", range(len(_golden_cases())))
def test_worked_cases_fp32_and_bf16(orc, case):
    x, s_exp, q_exp = _golden_cases()[case]
    for arr in (x[None, :], synth.to_bf16_bits(x[None, :])):
        q, s = orc.quant_rows(arr)
        assert s[0] == np.float32(s_exp)
        np.testing.assert_array_equal(q[0], q_exp)


def _brute_codes(x, s):
    """Nearest integer code in [-127,127] to x/s by enumeration, ties to even."""
    cand = np.arange(-127, 128, dtype=np.float64)
    out = np.empty(x.shape, np.int8)
    for i, xv in enumerate(x):
        t = float(np.float32(xv) / np.float32(s))  # the fp32 quotient
        d = np.abs(cand - t)
        best = np.flatnonzero(d == d.min())
        if best.size > 1:  # a tie: the even candidate
            best = best[(cand[best] % 2) == 0]
        out[i] = int(cand[best[0]])
    return out


def test_brute_force_small_rows(orc):
    r = np.random.default_rng(7)
    for trial in range(40):
        K = int(r.integers(1, 40))
        x = (r.standard_normal(K) * r.choice([0.01, 1.0, 30.0])).astype(np.float32)
        if trial % 5 == 0:  # plant exact half-integers relative to the scale
            x[0] = 127.0
            x[1:] = (r.integers(-254, 255, K - 1) / 2.0).astype(np.float32)
        q, s = orc.quant_rows(x[None, :])
        np.testing.assert_array_equal(q[0], _brute_codes(x, s[0]))


def test_zero_rows(orc):
    x = np.zeros((3, 64), np.float32)
    x[1, 5] = 1.0
    q, s = orc.quant_rows(x)
    assert s[0] == 0 and s[2] == 0 and not q[0].any() and not q[2].any()
    assert q[1, 5] == 127


def test_invariants_random(orc):
    cfg = synth.small_linear()
    xb = synth.activations(cfg["xkey"], 64, 512, 4, 20.0)
    x = orc.bf16_to_f32(xb)
    q, s = orc.quant_rows(xb)
    # reconstruction error bound: half a step plus the rounding of x/s
    err = np.abs(x - q.astype(np.float32) * s[:, None])
    assert np.all(err <= s[:, None] * (0.5 + 2e-6) + np.abs(x) * 2.0 ** -22)
    # the amax element of each row maps to +-127
    idx = np.argmax(np.abs(x), axis=1)
    np.testing.assert_array_equal(np.abs(q[np.arange(64), idx]), 127)
    # codes never reach -128
    assert q.min() >= -127
    # scale equivariance by powers of two (exact)
    for j in (-3, 1, 5):
        q2, s2 = orc.quant_rows(x * np.float32(2.0 ** j))
        np.testing.assert_array_equal(q2, q)
        np.testing.assert_array_equal(s2, s * np.float32(2.0 ** j))
    # odd symmetry
    q3, s3 = orc.quant_rows(-x)
    np.testing.assert_array_equal(q3, -q)
    np.testing.assert_array_equal(s3, s)
    # permutation of a row permutes its codes
    perm = np.random.default_rng(3).permutation(512)
    q4, s4 = orc.quant_rows(np.ascontiguousarray(x[:, perm]))
    np.testing.assert_array_equal(q4, q[:, perm])
    np.testing.assert_array_equal(s4, s)


def test_bf16_path_equals_fp32_path(orc):
    xb = synth.activations((9, 9), 8, 1000, 10, 10.0)
    qa, sa = orc.quant_rows(xb)
    qb, sb = orc.quant_rows(orc.bf16_to_f32(xb))
    np.testing.assert_array_equal(qa, qb)
    np.testing.assert_array_equal(sa, sb)


def test_scale_is_amax_over_127(orc):
    # the scale times 127 gives back amax to within one fp32 rounding
    for amax in (127.0, 254.0, 63.5, 31.75, 3.0, 1e-3):
        x = np.array([[amax, -amax / 4]], np.float32)
        _, s = orc.quant_rows(x)
        assert abs(float(s[0]) * 127.0 - amax) <= amax * 2.0 ** -23
