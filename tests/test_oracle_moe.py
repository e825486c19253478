"""Pins for the oracle's router (O4), expert counts (O5) and MoE forward (O6-O10).

What pins it:
  - router: brute force over all k-subsets (the kept set maximises the summed
    logit), numpy's stable argsort for the slot order, scipy's float64 softmax
    for the weights, the top-k sum check, ties to the lower expert index;
  - MoE: an independent chain built from numpy int64 matmuls, float32 scaling
    and torch's float64 SiLU for one expert / one slot; a hand-built example
    that separates gate from up and the sign inside the SiLU; token
    permutation equivariance and batch invariance; T=1 as the weighted sum of
    eight single-expert chains.
Source: "[gfx1151] Online INT8 W8A8 for Qwen3.6 27B / 35B-A3B on RDNA3.5, with
working MTP" (ATOM pull request), Changes: routing -> per-token int8 quant ->
gemm1 with gated SiLU over interleaved w13 -> per-token int8 quant -> gemm2
with scatter/combine; int8 w13/w2 with per-channel fp32 scales.
"""
import itertools

import numpy as np
import scipy.special
import torch

import synth


def test_router_brute_force_subsets(orc):
    r = np.random.default_rng(11)
    for _ in range(30):
        E = int(r.integers(2, 10))
        k = int(r.integers(1, min(E, 4) + 1))
        logits = r.standard_normal((1, E)).astype(np.float32)
        ids, w = orc.route_topk(logits, k)
        best = max(itertools.combinations(range(E), k),
                   key=lambda c: sum(float(logits[0, e]) for e in c))
        assert set(ids[0].tolist()) == set(best)


def test_router_against_argsort_and_softmax(orc):
    cfg = synth.moe(64)
    logits = synth.router_logits(cfg["xkey"], 64, 256)
    ids, w = orc.route_topk(logits, 8)
    np.testing.assert_array_equal(ids, np.argsort(-logits, axis=1, kind="stable")[:, :8])
    p = scipy.special.softmax(logits.astype(np.float64), axis=1)
    pk = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    ref = pk / pk.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(w, ref, rtol=2 ** -23, atol=0)
    np.testing.assert_allclose(w.astype(np.float64).sum(axis=1), 1.0, atol=1e-6)
    for t in range(64):
        assert len(set(ids[t].tolist())) == 8
    counts = orc.expert_counts(ids, 256)
    assert counts.sum() == 64 * 8
    np.testing.assert_array_equal(counts, np.bincount(ids.ravel(), minlength=256))


def test_router_ties_go_to_lower_index(orc):
    logits = np.array([[0.5, 2.0, 1.0, 2.0, 1.0, -3.0]], np.float32)
    ids, w = orc.route_topk(logits, 4)
    np.testing.assert_array_equal(ids[0], [1, 3, 2, 4])
    np.testing.assert_allclose(w[0, 0], w[0, 1])


def _moe_inputs(orc, T, E, H, I, k, seed):
    key = (90, seed)
    x = synth.activations(key, T, H, 0, 1.0)
    w13f = np.stack([synth.expert_weights(key, e, 2 * I, H, synth.T_W) for e in range(E)])
    w2f = np.stack([synth.expert_weights(key, e, H, I, synth.T_W2) for e in range(E)])
    q13, s13 = orc.quant_rows(w13f.reshape(E * 2 * I, H))
    q2, s2 = orc.quant_rows(w2f.reshape(E * H, I))
    logits = synth.router_logits(key, T, E)
    ids, w = orc.route_topk(logits, k)
    return (x, ids, w, q13.reshape(E, 2 * I, H), s13.reshape(E, 2 * I),
            q2.reshape(E, H, I), s2.reshape(E, H))


def _chain_reference(orc, x, e, wt, q13, s13, q2, s2):
    """One token through one expert, from library pieces: numpy int64 matmuls,
    float32 scaling, torch float64 SiLU, the (separately pinned) row quant."""
    qx, sx = orc.quant_rows(x[None, :])
    acc1 = qx.astype(np.int64) @ q13[e].astype(np.int64).T
    h = (acc1.astype(np.float32) * sx[:, None]) * s13[e][None, :]
    g, u = h[:, 0::2], h[:, 1::2]
    silu = torch.nn.functional.silu(torch.from_numpy(g.astype(np.float64))).numpy()
    act = silu.astype(np.float32) * u
    qa, sa2 = orc.quant_rows(act)
    acc2 = qa.astype(np.int64) @ q2[e].astype(np.int64).T
    y2 = (acc2.astype(np.float32) * sa2[:, None]) * s2[e][None, :]
    return act[0], y2[0] * np.float32(wt)


def test_single_expert_chain(orc):
    T, E, H, I, k = 5, 3, 256, 64, 1
    x, ids, w, q13, s13, q2, s2 = _moe_inputs(orc, T, E, H, I, k, 1)
    out, dbg = orc.moe_forward(x, ids, w, q13, s13, q2, s2, debug=True)
    for t in range(T):
        act_ref, y_ref = _chain_reference(orc, x[t], ids[t, 0], w[t, 0], q13, s13, q2, s2)
        # SiLU from torch in float64 vs the oracle's: at most one fp32 ulp apart
        np.testing.assert_allclose(dbg["act"][t], act_ref, rtol=2 ** -22, atol=1e-30)
        ref_bf16 = torch.from_numpy(y_ref).to(torch.bfloat16).to(torch.float32).numpy()
        got = orc.bf16_to_f32(out[t])
        np.testing.assert_allclose(got, ref_bf16, rtol=2 ** -7, atol=1e-6)


def test_t1_is_weighted_sum_of_eight_chains(orc):
    T, E, H, I, k = 1, 16, 256, 64, 8
    x, ids, w, q13, s13, q2, s2 = _moe_inputs(orc, T, E, H, I, k, 2)
    out = orc.bf16_to_f32(orc.moe_forward(x, ids, w, q13, s13, q2, s2)[0])
    ref = np.zeros(H, np.float64)
    for j in range(k):
        _, yj = _chain_reference(orc, x[0], ids[0, j], w[0, j], q13, s13, q2, s2)
        ref += yj.astype(np.float64)
    np.testing.assert_allclose(out, ref, rtol=1e-2, atol=1e-3)
    assert np.abs(out - ref).max() <= np.abs(ref).max() * 2 ** -7


def test_gate_up_order_and_silu_sign(orc):
    # One expert, H = 2, I = 1.  x = [127, 127] -> sx = 1, qx = [127, 127].
    # w13 row 0 (gate) = [1, 0] -> gate h0 = 127*127*(1/127) ~= 127
    # w13 row 1 (up)   = [1, 1] -> scale 1/127, codes [127, 127] -> h1 ~= 254
    # silu(127) * 254 ~= 127*254; with gate/up swapped it would be silu(254)*127,
    # with the sign inside the sigmoid flipped it would be ~0.
    x = synth.to_bf16_bits(np.array([[127.0, 127.0]], np.float32))
    w13f = np.array([[1.0, 0.0], [1.0, 1.0]], np.float32)
    q13, s13 = orc.quant_rows(w13f)
    w2f = np.array([[1.0], [0.5]], np.float32)
    q2, s2 = orc.quant_rows(w2f)
    ids = np.zeros((1, 1), np.int32)
    w = np.ones((1, 1), np.float32)
    out, dbg = orc.moe_forward(x, ids, w, q13[None], s13[None], q2[None], s2[None], debug=True)
    h0 = (np.float32(127 * 127) * np.float32(1.0)) * s13[0]
    h1 = (np.float32(127 * 127 * 2) * np.float32(1.0)) * s13[1]
    silu_ref = float(h0) / (1.0 + np.exp(-float(h0)))
    np.testing.assert_allclose(dbg["act"][0, 0], silu_ref * float(h1), rtol=1e-6)
    assert abs(float(dbg["act"][0, 0]) - 127.0 * 254.0) < 127.0 * 254.0 * 1e-4
    # act quantises to code 127 with scale act/127; gemm2 rows [1] and [0.5]
    y = orc.bf16_to_f32(out[0])
    np.testing.assert_allclose(y, [dbg["act"][0, 0], dbg["act"][0, 0] * 0.5], rtol=2 ** -7)


def test_token_permutation_and_batch_invariance(orc):
    T, E, H, I, k = 12, 8, 128, 64, 4
    x, ids, w, q13, s13, q2, s2 = _moe_inputs(orc, T, E, H, I, k, 3)
    out = orc.moe_forward(x, ids, w, q13, s13, q2, s2)
    perm = np.random.default_rng(0).permutation(T)
    out_p = orc.moe_forward(np.ascontiguousarray(x[perm]), np.ascontiguousarray(ids[perm]),
                            np.ascontiguousarray(w[perm]), q13, s13, q2, s2)
    np.testing.assert_array_equal(out_p, out[perm])
    for t in (0, 7):
        o1 = orc.moe_forward(x[t:t + 1], ids[t:t + 1], w[t:t + 1], q13, s13, q2, s2)
        np.testing.assert_array_equal(o1[0], out[t])


def test_debug_intermediates_consistent(orc):
    T, E, H, I, k = 4, 4, 128, 32, 2
    x, ids, w, q13, s13, q2, s2 = _moe_inputs(orc, T, E, H, I, k, 4)
    out, d = orc.moe_forward(x, ids, w, q13, s13, q2, s2, debug=True)
    qx, sx = orc.quant_rows(x)
    np.testing.assert_array_equal(d["qx"], qx)
    np.testing.assert_array_equal(d["sx"], sx)
    for r in range(T * k):
        t, e = r // k, ids.ravel()[r]
        np.testing.assert_array_equal(
            d["acc1"][r], qx[t].astype(np.int64) @ q13[e].astype(np.int64).T)
        qa, sa = orc.quant_rows(d["act"][r:r + 1])
        np.testing.assert_array_equal(d["qa"][r], qa[0])
        assert d["sa2"][r] == sa[0]
        np.testing.assert_array_equal(
            d["acc2"][r], d["qa"][r].astype(np.int64) @ q2[e].astype(np.int64).T)
