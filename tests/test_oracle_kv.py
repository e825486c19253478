"""Pins for the oracle's int8 KV-cache quantisation with an f16 scale per token
and head (O15) and its fp32 -> f16 rounding.

What pins it:
  - the f16 rounding against numpy's IEEE float16 conversion: every f16
    value and the midpoints around it (ties to even), subnormals, the
    overflow threshold, random values over the whole range;
  - hand-worked rows (scale exactly 1; a scale that rounds in f16 and moves a
    code across a half-integer; a zero row; a scale below the smallest f16
    subnormal);
  - a composition from numpy pieces (float32 maximum and division, float16
    conversion, rint) that must agree bit for bit;
  - the cache-slot mapping: tokens land in the rows named by the slots,
    negative slots skip, and the reconstruction code * s is within s/2.
Source: "Qwen3.6-35B-A3B IQ8R - radiance container", Serve: kv-cache-dtype i8
stores the attention cache as int8 with an f16 scale per token and head.
"""
import numpy as np

import synth


def _f16_bits(v):
    with np.errstate(over="ignore"):
        return np.asarray(v, np.float32).astype(np.float16).view(np.uint16)


def test_f16_rounding_against_numpy(orc):
    every = np.arange(0, 0x7c00, dtype=np.uint16).view(np.float16).astype(np.float32)
    nxt = np.arange(1, 0x7c01, dtype=np.uint16).view(np.float16).astype(np.float32)
    nxt[-1] = 65536.0
    mids = ((every.astype(np.float64) + nxt.astype(np.float64)) / 2).astype(np.float32)
    r = np.random.default_rng(3)
    rnd = (r.standard_normal(200000) * np.exp(r.uniform(-30, 12, 200000))).astype(np.float32)
    edge = np.array([65504.0, 65519.0, 65520.0, 70000.0, 2.0 ** -14, 2.0 ** -24, 2.0 ** -25,
                     2.0 ** -26, 3 * 2.0 ** -26, 0.0], np.float32)
    for vals in (every, mids, np.nextafter(mids, np.float32(np.inf)),
                 np.nextafter(mids, np.float32(0)), rnd, edge):
        for v in (vals, -vals):
            np.testing.assert_array_equal(orc.f32_to_f16(v), _f16_bits(v))


def _row(vals, D=16):
    row = np.zeros(D, np.float32)
    row[:len(vals)] = vals
    return synth.to_bf16_bits(row)


def test_worked_rows(orc):
    # scale exactly 1: codes are the values rounded half to even
    x = np.stack([_row([127, 2.5, -2.5, 3.5, 0.5, -126.5])])[:, None, :]
    q, s = orc.kv_quant_i8(x)
    assert s[0, 0] == 0x3c00
    np.testing.assert_array_equal(q[0, 0, :6], [127, 2, -2, 4, 0, -126])
    # amax = 1.015625: amax/127 = 0.0079970 rounds to the f16 value
    # 1048/1024 * 2^-7 = 0.00799560546875 (bits: exponent -7 -> 8, fraction 24).
    # Against it 0.33984375 -> 42.504 -> 43 and 0.8515625 -> 106.504 -> 107;
    # against the unrounded fp32 scale they would be 42.496 -> 42 and
    # 106.485 -> 106.  0.25 -> 31.27 -> 31.
    x = np.stack([_row([1.015625, 0.33984375, -0.8515625, 0.25])])[:, None, :]
    q, s = orc.kv_quant_i8(x)
    assert s[0, 0] == (8 << 10) | 24
    np.testing.assert_array_equal(q[0, 0, :4], [127, 43, -107, 31])
    # zero row, and a row whose scale is below half the smallest f16 subnormal
    x = np.stack([_row([0.0]), _row([1e-9, -5e-10])])[:, None, :]
    q, s = orc.kv_quant_i8(x)
    assert not s.any() and not q.any()


def test_composition_from_numpy(orc):
    T, Hk, D = 37, 4, 256
    xb = synth.activations((99, 1), T, Hk * D, 40, 10.0).reshape(T, Hk, D)
    xb[3, 2] = 0
    q, s = orc.kv_quant_i8(xb)
    x = orc.bf16_to_f32(xb)
    amax = np.abs(x).max(axis=2)
    s16 = (amax / np.float32(127.0)).astype(np.float16)
    np.testing.assert_array_equal(s, s16.view(np.uint16))
    sf = s16.astype(np.float32)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        ref = np.clip(np.rint(x / sf), -127, 127)
    ref = np.where(sf == 0, 0, ref).astype(np.int8)
    np.testing.assert_array_equal(q, ref)
    # the cache holds code * s within half a step of every value
    err = np.abs(x - q.astype(np.float32) * sf)
    assert np.all(err <= sf * 0.5 * (1 + 2 ** -10))


def test_slot_mapping(orc):
    T, Hk, D = 9, 2, 64
    xb = synth.activations((99, 2), T, Hk * D, 4, 10.0).reshape(T, Hk, D)
    q0, s0 = orc.kv_quant_i8(xb)
    slots = np.array([12, 3, -1, 7, 0, 15, -1, 1, 8], np.int32)
    q, s = orc.kv_quant_i8(xb, slots, rows=16)
    for t, row in enumerate(slots):
        if row >= 0:
            np.testing.assert_array_equal(q[row], q0[t])
            np.testing.assert_array_equal(s[row], s0[t])
    untouched = sorted(set(range(16)) - set(int(v) for v in slots if v >= 0))
    assert not q[untouched].any() and not s[untouched].any()
