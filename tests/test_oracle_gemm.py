"""Pins for the oracle's int8 GEMM and fp32 epilogue (O3).

What pins it:
  - library: numpy int64 matmul and CPU torch._int_mm give the same int32 sums;
  - brute force: a Python triple loop on tiny shapes;
  - a hand-worked example with exact scales;
  - the bf16 rounding of the epilogue against torch's fp32 -> bf16 conversion;
  - invariants: permuting K on both operands, y(2^j x) = 2^j y(x) bit-exactly,
    y(-x) = -y(x); all-(+-127) codes at the largest K (no int32 overflow);
  - an informational sanity check against a float64 product of the
    dequantised operands.
Source: "[gfx1151] Online INT8 W8A8 for Qwen3.6 27B / 35B-A3B on RDNA3.5, with
working MTP" (ATOM pull request), Changes (per-token int8 activations, int8
weights with per-channel fp32 scales, bf16 out).
"""
import numpy as np
import torch

import synth


def _rand_i8(r, shape):
    return r.integers(-127, 128, size=shape, dtype=np.int64).astype(np.int8)


def test_acc_matches_int64_matmul_and_int_mm(orc):
    r = np.random.default_rng(1)
    for (M, N, K) in [(1, 1, 64), (16, 256, 512), (33, 17, 200), (8, 40, 5120)]:
        qa, qw = _rand_i8(r, (M, K)), _rand_i8(r, (N, K))
        acc = orc.gemm_i32(qa, qw)
        ref = qa.astype(np.int64) @ qw.astype(np.int64).T
        np.testing.assert_array_equal(acc, ref)
        if M >= 17 and K % 8 == 0 and N % 8 == 0:
            tm = torch._int_mm(torch.from_numpy(qa), torch.from_numpy(qw).t().contiguous())
            np.testing.assert_array_equal(acc, tm.numpy())


def test_acc_brute_force_tiny(orc):
    r = np.random.default_rng(2)
    M, N, K = 3, 5, 17
    qa, qw = _rand_i8(r, (M, K)), _rand_i8(r, (N, K))
    acc = orc.gemm_i32(qa, qw)
    for m in range(M):
        for n in range(N):
            s = 0
            for k in range(K):
                s += int(qa[m, k]) * int(qw[n, k])
            assert acc[m, n] == s


def test_worked_example(orc):
    # acc = [[1*3 + 2*4, 1*(-1) + 2*0], [-5*3 + 6*4, -5*(-1) + 6*0]] = [[11, -1], [9, 5]]
    qa = np.array([[1, 2], [-5, 6]], np.int8)
    qw = np.array([[3, 4], [-1, 0]], np.int8)
    sa = np.array([0.5, 2.0], np.float32)
    sw = np.array([0.25, 4.0], np.float32)
    y = orc.bf16_to_f32(orc.gemm_w8a8(qa, sa, qw, sw))
    np.testing.assert_array_equal(y, np.array([[11 * 0.125, -1 * 2.0], [9 * 0.5, 5 * 8.0]],
                                              np.float32))


def test_epilogue_rounding_against_torch_bf16(orc):
    r = np.random.default_rng(3)
    M, N = 32, 64
    acc = r.integers(-2 ** 27, 2 ** 27, size=(M, N)).astype(np.int32)
    sa = (r.random(M) * 0.1).astype(np.float32)
    sw = (r.random(N) * 0.01).astype(np.float32)
    y = orc.epilogue(acc, sa, sw)
    t = (torch.from_numpy(acc).to(torch.float32) * torch.from_numpy(sa)[:, None]) \
        * torch.from_numpy(sw)[None, :]
    ref = t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(y, ref)


def test_invariants(orc):
    cfg = synth.small_linear()
    xb = synth.activations(cfg["xkey"], cfg["M"], cfg["K"], 4, 20.0)
    W = synth.weights(cfg["wkey"], cfg["N"], cfg["K"])
    qw, sw = orc.quant_rows(W)
    x = orc.bf16_to_f32(xb)
    y = orc.linear_w8a8(xb, qw, sw)
    # permuting K identically on activations and weights changes nothing
    perm = np.random.default_rng(4).permutation(cfg["K"])
    y_p = orc.linear_w8a8(np.ascontiguousarray(xb[:, perm]), np.ascontiguousarray(qw[:, perm]),
                          sw)
    np.testing.assert_array_equal(y_p, y)
    # power-of-two scaling of x scales y exactly; negation negates y
    yf = orc.bf16_to_f32(y)
    for j in (-2, 3):
        y2 = orc.bf16_to_f32(orc.linear_w8a8(synth.to_bf16_bits(x * np.float32(2.0 ** j)),
                                             qw, sw))
        np.testing.assert_array_equal(y2, yf * np.float32(2.0 ** j))
    y3 = orc.bf16_to_f32(orc.linear_w8a8(synth.to_bf16_bits(-x), qw, sw))
    np.testing.assert_array_equal(y3, -yf)


def test_no_overflow_at_largest_k(orc):
    K = 8704
    qa = np.full((2, K), 127, np.int8)
    qa[1] = -127
    qw = np.full((3, K), 127, np.int8)
    qw[2, ::2] = -127
    acc = orc.gemm_i32(qa, qw)
    big = 127 * 127 * K
    np.testing.assert_array_equal(acc, np.array([[big, big, 0], [-big, -big, 0]]))


def test_points_match_full(orc):
    r = np.random.default_rng(5)
    qa, qw = _rand_i8(r, (9, 300)), _rand_i8(r, (70, 300))
    sa = r.random(9).astype(np.float32)
    sw = r.random(70).astype(np.float32)
    y = orc.gemm_w8a8(qa, sa, qw, sw)
    ms = r.integers(0, 9, 50)
    ns = r.integers(0, 70, 50)
    acc_p, y_p = orc.gemm_w8a8_points(qa, sa, qw, sw, ms, ns)
    np.testing.assert_array_equal(y_p, y[ms, ns])
    np.testing.assert_array_equal(acc_p, orc.gemm_i32(qa, qw)[ms, ns])


def test_sanity_against_dequantised_fp64(orc):
    # informational bound: W8A8 output vs float64 x @ W^T on the small workload
    cfg = synth.small_linear()
    xb = synth.activations(cfg["xkey"], cfg["M"], cfg["K"], 4, 20.0)
    W = synth.weights(cfg["wkey"], cfg["N"], cfg["K"])
    qw, sw = orc.quant_rows(W)
    y = orc.bf16_to_f32(orc.linear_w8a8(xb, qw, sw)).astype(np.float64)
    ref = orc.bf16_to_f32(xb).astype(np.float64) @ W.astype(np.float64).T
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert rel < 0.05
