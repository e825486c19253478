"""Pins for the oracle's fwht128 (O11), rotated weight prep (O12) and g256 GEMM (O13).

What pins it:
  - closed forms: the transform of e_i is column i of the Sylvester Hadamard
    matrix (scipy.linalg.hadamard(128)); H H = 128 I, so applying it twice
    gives 128 x exactly on small integers; Parseval; <Hx, Hw> = 128 <x, w>;
  - an independent recursive formulation (H_2n = [[H_n, H_n], [H_n, -H_n]]) in
    numpy float32, which performs the same additions in the same order and so
    must agree bit for bit (this pins the stage order h = 1, 2, ..., 64);
  - weight prep invariants: u8 scales in [1, 255], reconstruction within half
    a step, the row scale is a bf16 value;
  - g256 GEMM: int64 group sums from numpy matmuls; the end-to-end result
    approximates the float64 product x @ W^T (pins the 2^-7 and the scales).
Source: "Qwen3.6-35B-A3B IQ8R - radiance container", Trunk and Activations
rows (codes -127..127, u8 scale per row and 256 of K under a bf16 row scale,
each 128 of K rotated by the unnormalised Hadamard) and the recipe under "How
this file was made" (group=256 scale=u8 scale2=bf16 block2=1x* transform=fwht128
clamp=sym).
"""
import numpy as np
import scipy.linalg

import synth

H128 = scipy.linalg.hadamard(128).astype(np.int64)


def test_basis_vectors_give_hadamard_columns(orc):
    eye = np.eye(128, dtype=np.float32)
    out = orc.fwht128_rows(eye)  # row i = transform of e_i
    np.testing.assert_array_equal(out.astype(np.int64), H128.T)


def test_twice_is_128x_and_integer_exact(orc):
    r = np.random.default_rng(21)
    x = r.integers(-50, 51, size=(4, 256)).astype(np.float32)
    y = orc.fwht128_rows(x)
    for b in range(2):
        np.testing.assert_array_equal(
            y[:, b * 128:(b + 1) * 128].astype(np.int64),
            x[:, b * 128:(b + 1) * 128].astype(np.int64) @ H128.T)
    np.testing.assert_array_equal(orc.fwht128_rows(y), x * 128)
    # Parseval, exact for integers
    np.testing.assert_array_equal((y.astype(np.int64) ** 2).sum(1),
                                  128 * (x.astype(np.int64) ** 2).sum(1))


def _fwht_recursive(v):
    n = v.shape[-1]
    if n == 1:
        return v
    a = _fwht_recursive(v[..., : n // 2])
    b = _fwht_recursive(v[..., n // 2:])
    return np.concatenate([a + b, a - b], axis=-1)


def test_bit_exact_against_recursive_form(orc):
    xb = synth.activations((5, 99), 16, 2048, 20, 10.0, heavy_tail=True)
    x = orc.bf16_to_f32(xb)
    y = orc.fwht128_rows(x)
    ref = np.concatenate([_fwht_recursive(x[:, b:b + 128]) for b in range(0, 2048, 128)], 1)
    assert ref.dtype == np.float32
    np.testing.assert_array_equal(y, ref)
    # and close to the float64 matrix product
    m = np.concatenate([x[:, b:b + 128].astype(np.float64) @ H128.T for b in range(0, 2048, 128)],
                       1)
    np.testing.assert_allclose(y, m, rtol=0, atol=np.abs(x).max() * 128 * 2 ** -20)


def test_fwht_quant_is_transform_then_row_quant(orc):
    xb = synth.activations((5, 98), 8, 2048, 20, 10.0, heavy_tail=True)
    q, s = orc.fwht128_quant(xb)
    q2, s2 = orc.quant_rows(orc.fwht128_rows(orc.bf16_to_f32(xb)))
    np.testing.assert_array_equal(q, q2)
    np.testing.assert_array_equal(s, s2)


def test_weight_prep_invariants(orc):
    W = synth.weights((5, 97), 64, 2048)
    qw, su8, s2 = orc.weight_prep_g256(W)
    s2f = orc.bf16_to_f32(s2)
    assert su8.min() >= 1 and su8.max() <= 255
    assert (su8 == 255).any(axis=1).mean() > 0.5
    eff = s2f[:, None] * su8.astype(np.float32)  # [N, 8]
    wr = orc.fwht128_rows(W)
    effk = np.repeat(eff, 256, axis=1)
    err = np.abs(wr - qw.astype(np.float32) * effk)
    clamped = np.abs(qw) == 127
    assert np.all(err[~clamped] <= effk[~clamped] * (0.5 + 1e-5))
    # the group maximum is represented with at most one extra step of error
    gmax = np.abs(wr).reshape(64, 8, 256).max(2)
    assert np.all(np.abs(gmax - 127 * eff) <= eff * 1.6)
    # zero rows and zero groups
    Wz = W[:2].copy()
    Wz[0] = 0
    Wz[1, :256] = 0
    qz, suz, s2z = orc.weight_prep_g256(Wz)
    assert s2z[0] == 0 and not suz[0].any() and not qz[0].any()
    assert suz[1, 0] == 0 and not qz[1, :256].any() and suz[1, 1:].min() >= 1


def test_g256_group_sums_and_scaling(orc):
    r = np.random.default_rng(22)
    M, N, K = 5, 12, 1024
    qa = r.integers(-127, 128, size=(M, K)).astype(np.int8)
    qw = r.integers(-127, 128, size=(N, K)).astype(np.int8)
    su8 = r.integers(1, 256, size=(N, K // 256)).astype(np.uint8)
    s2 = synth.to_bf16_bits(r.random(N).astype(np.float32) * 1e-3)
    sa = r.random(M).astype(np.float32) * 0.1
    y, ts = orc.gemm_g256(qa, sa, qw, su8, s2, return_tsum=True)
    ref_ts = np.zeros((M, N), np.int64)
    for g in range(K // 256):
        accg = qa[:, g * 256:(g + 1) * 256].astype(np.int64) @ \
            qw[:, g * 256:(g + 1) * 256].astype(np.int64).T
        ref_ts += accg * su8[:, g].astype(np.int64)[None, :]
    np.testing.assert_array_equal(ts, ref_ts)
    val = ref_ts * sa[:, None].astype(np.float64) * orc.bf16_to_f32(s2)[None, :] / 128.0
    np.testing.assert_allclose(orc.bf16_to_f32(y), val, rtol=2 ** -8, atol=0)
    yp, tp = orc.gemm_g256_points(qa, sa, qw, su8, s2, [0, 4, 2], [11, 0, 5])
    np.testing.assert_array_equal(yp, y[[0, 4, 2], [11, 0, 5]])


def test_rotated_inner_product_identity(orc):
    # <Hx, Hw> = 128 <x, w> exactly for integer vectors
    r = np.random.default_rng(23)
    x = r.integers(-8, 9, size=(3, 256)).astype(np.float32)
    w = r.integers(-8, 9, size=(4, 256)).astype(np.float32)
    hx = orc.fwht128_rows(x).astype(np.int64)
    hw = orc.fwht128_rows(w).astype(np.int64)
    np.testing.assert_array_equal(hx @ hw.T, 128 * (x.astype(np.int64) @ w.astype(np.int64).T))


def test_end_to_end_approximates_float_product(orc):
    xb = synth.activations((5, 96), 16, 2048, 20, 10.0, heavy_tail=True)
    W = synth.weights((5, 95), 256, 2048)
    qw, su8, s2 = orc.weight_prep_g256(W)
    qa, sa = orc.fwht128_quant(xb)
    y = orc.bf16_to_f32(orc.gemm_g256(qa, sa, qw, su8, s2)).astype(np.float64)
    ref = orc.bf16_to_f32(xb).astype(np.float64) @ W.astype(np.float64).T
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert rel < 0.03
    # the rotation helps on heavy-tailed outliers: compare with plain per-token W8A8
    qw1, sw1 = orc.quant_rows(W)
    y1 = orc.bf16_to_f32(orc.linear_w8a8(xb, qw1, sw1)).astype(np.float64)
    rel1 = np.linalg.norm(y1 - ref) / np.linalg.norm(ref)
    assert rel < rel1
