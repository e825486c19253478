"""Pin of the oracle's rotated weight preparation (two-level u8 / bf16 scale)
against hand-worked cases, and proof that the cases tell it apart from the
plausible misreadings.

Source: "Qwen3.6-35B-A3B IQ8R - radiance container", Trunk row (int8 codes
-127..127, a u8 scale per row and 256 of K under a bf16 scale per row, each
128 of K rotated by the unnormalised Hadamard, round to nearest) and the
recipe under "How this file was made" (group=256 scale=u8 scale2=bf16
block2=1x* transform=fwht128 clamp=sym).  The recipe names the pieces but not
the arithmetic; tests/golden/g256_prep_worked.txt works the reading out by
hand on rows whose rotated values are known in closed form.

The second test plants each misreading in a copy of the oracle's C source
(CPU only), rebuilds it, and checks that the worked cases reject it.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "g256_prep_worked.txt")
U = 2.0 ** -10
K = 512


def _load_cases():
    rows, s2, su8, codes = [], [], [], []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        ent, s2t, sut, cdt = [p.strip() for p in line.split("|")]
        w = np.zeros(K, np.float32)
        if ent != "-":
            for e in ent.split():
                k, v = e.split(":")
                w[int(k)] = np.float32(float(v) * U)
        rows.append(w)
        s2.append(float(s2t) * U)
        su8.append([int(v) for v in sut.split()])
        codes.append([tuple(int(c) for c in p.split(",")) for p in cdt.split()])
    return np.stack(rows), np.array(s2), np.array(su8, np.uint8), codes


def _expected_codes(codes):
    q = np.zeros((len(codes), K), np.int8)
    for r, blocks in enumerate(codes):
        for b, (ev, od) in enumerate(blocks):
            q[r, b * 128:(b + 1) * 128:2] = ev
            q[r, b * 128 + 1:(b + 1) * 128:2] = od
    return q


def _matches(prep, W, s2, su8, q):
    qw, su, s2b = prep(W)
    return (np.array_equal(oracle.bf16_to_f32(s2b).astype(np.float64), s2)
            and np.array_equal(su, su8) and np.array_equal(qw, q))


def test_worked_cases_reproduced():
    W, s2, su8, codes = _load_cases()
    q = _expected_codes(codes)
    qw, su, s2b = oracle.weight_prep_g256(W)
    np.testing.assert_array_equal(oracle.bf16_to_f32(s2b).astype(np.float64), s2)
    np.testing.assert_array_equal(su, su8)
    np.testing.assert_array_equal(qw, q)


# misreadings of the recipe, each as (the oracle's text, the planted text)
MUTANTS = {
    "row scale over 256": ("smax / 255.0f", "smax / 256.0f"),
    "u8 scale floored": ("nearbyintf(sg[g] / s2f)", "floorf(sg[g] / s2f)"),
    "u8 scale rounded up": ("nearbyintf(sg[g] / s2f)", "ceilf(sg[g] / s2f)"),
    "u8 scale may be 0": ("if (r < 1.0f) r = 1.0f;", ""),
    "codes round half away": ("nearbyintf(row[k] / eff)", "roundf(row[k] / eff)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_worked_cases_reject_misreadings(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    assert src.count(old) == 1, f"mutation site not unique: {old!r}"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", *oracle.CFLAGS, "-o", str(so), str(path), "-lm"])
    lib = ctypes.CDLL(str(so))

    def prep(W):
        W = np.ascontiguousarray(W, np.float32)
        N = W.shape[0]
        qw = np.empty((N, K), np.int8)
        su = np.empty((N, K // 256), np.uint8)
        s2 = np.empty((N,), np.uint16)
        lib.orc_weight_prep_g256(ctypes.c_void_p(W.ctypes.data), ctypes.c_int64(N),
                                 ctypes.c_int64(K), ctypes.c_void_p(qw.ctypes.data),
                                 ctypes.c_void_p(su.ctypes.data), ctypes.c_void_p(s2.ctypes.data))
        return qw, su, s2

    W, s2, su8, codes = _load_cases()
    q = _expected_codes(codes)
    assert _matches(oracle.weight_prep_g256, W, s2, su8, q)
    assert not _matches(prep, W, s2, su8, q), f"the worked cases accept the mutant: {name}"
