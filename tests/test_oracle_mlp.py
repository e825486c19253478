"""Pins for the oracle's dense W8A8 MLP block (O14).

What pins it:
  - an independent chain from library pieces: numpy int64 matmuls for both
    contractions, float32 scaling in the epilogue's order, torch's float64
    SiLU, and the separately pinned row quantiser;
  - the routed layer with one expert, top-1 and weight 1 is the same block:
    every intermediate and the output agree bit for bit (out = bf16(1 * y2));
  - a hand-built example whose gate and up differ, so swapping them or the
    sign inside the SiLU changes the result;
  - invariants: permuting the intermediate channels (gate/up row pairs with
    the matching down-weight columns) leaves the output bit-identical; a zero
    gate or a zero up gives a zero output; rows are independent.
Source: "[gfx1151] Online INT8 W8A8 for Qwen3.6 27B / 35B-A3B on RDNA3.5, with
working MTP" (ATOM pull request): A8W8 for all dense GEMMs (intro), and the
order quant -> gemm1 with gated SiLU -> per-token requant -> gemm2 of its
Changes, fused_moe_triton.py bullet.
"""
import math

import numpy as np
import torch

import synth


def _inputs(orc, M, K, I, N, seed):
    key = (91, seed)
    x = synth.activations(key, M, K, max(1, K // 100), 10.0)
    qgu, sgu = orc.quant_rows(synth.weights(key, 2 * I, K))
    qd, sd = orc.quant_rows(synth.weights(key, N, I, tensor_id=synth.T_W2))
    return x, qgu, sgu, qd, sd


def test_chain_from_library_pieces(orc):
    M, K, I, N = 6, 512, 192, 128
    x, qgu, sgu, qd, sd = _inputs(orc, M, K, I, N, 1)
    y, d = orc.mlp_forward(x, qgu, sgu, qd, sd, debug=True)
    qx, sx = orc.quant_rows(x)
    np.testing.assert_array_equal(d["qx"], qx)
    np.testing.assert_array_equal(d["sx"], sx)
    acc1 = qx.astype(np.int64) @ qgu.astype(np.int64).T
    np.testing.assert_array_equal(d["acc1"], acc1)
    h = (acc1.astype(np.float32) * sx[:, None]) * sgu[None, :]
    g, u = h[:, 0::2], h[:, 1::2]
    silu = torch.nn.functional.silu(torch.from_numpy(g.astype(np.float64))).numpy()
    act = silu.astype(np.float32) * u
    # SiLU from torch in float64 vs the oracle's: at most one fp32 ulp apart
    np.testing.assert_allclose(d["act"], act, rtol=2 ** -22, atol=1e-30)
    qa, sa = orc.quant_rows(d["act"])
    np.testing.assert_array_equal(d["qa"], qa)
    np.testing.assert_array_equal(d["sa"], sa)
    acc2 = qa.astype(np.int64) @ qd.astype(np.int64).T
    np.testing.assert_array_equal(d["acc2"], acc2)
    y2 = (acc2.astype(np.float32) * sa[:, None]) * sd[None, :]
    ref = torch.from_numpy(y2).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(y, ref)


def test_equals_single_expert_routed_layer(orc):
    M, K, I, N = 5, 256, 128, 256
    x, qgu, sgu, qd, sd = _inputs(orc, M, K, I, N, 2)
    y, d = orc.mlp_forward(x, qgu, sgu, qd, sd, debug=True)
    ids = np.zeros((M, 1), np.int32)
    w = np.ones((M, 1), np.float32)
    out, dm = orc.moe_forward(x, ids, w, qgu[None], sgu[None], qd[None], sd[None], debug=True)
    np.testing.assert_array_equal(y, out)
    for a, b in (("acc1", "acc1"), ("act", "act"), ("qa", "qa"), ("sa", "sa2"),
                 ("acc2", "acc2"), ("qx", "qx"), ("sx", "sx")):
        np.testing.assert_array_equal(d[a], dm[b])


def test_gate_up_order_and_silu_sign(orc):
    # x = [127, 0, ...]: scale exactly 1, codes [127, 0, ...].  Gate row code 1
    # with scale 2^-6 -> gate = 127 * 2^-6; up row code 1 with scale 2^-5 ->
    # up = 127 * 2^-5.  Swapping gate and up, or the sign inside the sigmoid,
    # gives a different activation.
    K = 64
    xf = np.zeros((1, K), np.float32)
    xf[0, 0] = 127.0
    x = synth.to_bf16_bits(xf)
    qgu = np.zeros((2, K), np.int8)
    qgu[:, 0] = 1
    sgu = np.array([2.0 ** -6, 2.0 ** -5], np.float32)
    qd = np.array([[1], [-2]], np.int8)
    sd = np.array([0.5, 0.25], np.float32)
    y, d = orc.mlp_forward(x, qgu, sgu, qd, sd, debug=True)
    gate, up = 127 * 2.0 ** -6, 127 * 2.0 ** -5
    act = np.float32(np.float32(gate / (1.0 + math.exp(-gate))) * np.float32(up))
    assert d["act"][0, 0] == act
    swapped = np.float32(np.float32(up / (1.0 + math.exp(-up))) * np.float32(gate))
    flipped = np.float32(np.float32(gate / (1.0 + math.exp(gate))) * np.float32(up))
    assert act != swapped and act != flipped
    # one activation: code 127, scale act/127; outputs act/2 and -act/2 (bf16)
    sa = np.float32(act / np.float32(127.0))
    assert d["sa"][0] == sa and d["qa"][0, 0] == 127
    want = [np.float32(np.float32(np.float32(127 * c) * sa) * s) for c, s in ((1, 0.5), (-2, 0.25))]
    np.testing.assert_array_equal(orc.bf16_to_f32(y[0]), orc.bf16_to_f32(orc.bf16_round(
        np.array(want, np.float32))))


def test_channel_permutation_and_zero_invariants(orc):
    M, K, I, N = 4, 256, 96, 64
    x, qgu, sgu, qd, sd = _inputs(orc, M, K, I, N, 3)
    x[2] = 0
    y = orc.mlp_forward(x, qgu, sgu, qd, sd)
    assert not y[2].any()
    perm = np.random.default_rng(5).permutation(I)
    rows = np.stack([2 * perm, 2 * perm + 1], 1).ravel()
    yp = orc.mlp_forward(x, np.ascontiguousarray(qgu[rows]), np.ascontiguousarray(sgu[rows]),
                         np.ascontiguousarray(qd[:, perm]), sd)
    np.testing.assert_array_equal(yp, y)
    for zero_rows in (slice(0, None, 2), slice(1, None, 2)):  # all gates / all ups zero
        qz = qgu.copy()
        qz[zero_rows] = 0
        assert not orc.mlp_forward(x, qz, sgu, qd, sd).any()
    for m in (0, 3):
        np.testing.assert_array_equal(orc.mlp_forward(x[m:m + 1], qgu, sgu, qd, sd)[0], y[m])
