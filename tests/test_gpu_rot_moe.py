"""GPU parity of the Hadamard-domain MoE pieces through the C ABI: the g128
weight preparation, the bf16 router gate, the routed experts on the rotated
grid (g128 bf16 scales) and the shared expert, against the CPU oracle.

Bar:
  - weight preparation: codes and bf16 scales bit-exact;
  - router gate: fp32 logits within the fp32 summation bound H 2^-24 sum|x w|
    of the exact sum (the oracle's fp64 sum rounded once), and bit-exact on
    small-integer operands where every partial sum is exact; repeated calls
    bit-identical;
  - routed experts: routing ids exact, weights within 1 fp32 ulp, rotated
    codes and scales of x bit-exact, the SiLU activation within 1 fp32 ulp
    (the fp64 fold of the group sums is the oracle's operation sequence; the
    device exp may differ from the host's by an ulp), the rotated requant
    codes and scales bit-exact on every pair row whose activation agrees,
    elsewhere within one code step (rare); the bf16 output within 1e-3 abs +
    1e-2 rel and bit-exact for every token whose pairs' codes all agree;
  - shared expert: the same bar on its activation and codes; fp32 y within
    1e-3 abs + 1e-2 rel and bit-exact on rows whose codes agree.
"""
import numpy as np
import pytest
import torch

import moe_quant_token_amd as mq
import synth
from tests._util import (tie_logits, assert_bf16_close, bf16_dev, bf16_host, dev, host, say,
                         ulp_diff_f32)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mq.lib()


# ---------------------------------------------------------------- weights --

def _rot_weights(orc, wkey, E, H, I):
    q13 = np.empty((E, 2 * I, H), np.int8)
    s13 = np.empty((E, 2 * I, H // 128), np.uint16)
    q2 = np.empty((E, H, I), np.int8)
    s2 = np.empty((E, H, I // 128), np.uint16)
    for e in range(E):
        q13[e], s13[e] = orc.weight_prep_g128(synth.expert_weights(wkey, e, 2 * I, H, synth.T_W))
        q2[e], s2[e] = orc.weight_prep_g128(synth.expert_weights(wkey, e, H, I, synth.T_W2))
    return q13, s13, q2, s2


def _dev_rot_weights(W):
    q13, s13, q2, s2 = W
    p13, p2 = mq.pack_moe_weights(dev(q13), dev(q2))
    return p13, bf16_dev(s13), p2, bf16_dev(s2)


def _shared_weights(orc, wkey, H, Is):
    wgu, su8, s2 = orc.weight_prep_g256(synth.weights(wkey, 2 * Is, H, tensor_id=synth.T_W))
    wd, sd = orc.weight_prep_g128(synth.weights(wkey, H, Is, tensor_id=synth.T_W2))
    return wgu, su8, s2, wd, sd


def _dev_shared_weights(S):
    wgu, su8, s2, wd, sd = S
    return (mq.pack_weights(dev(wgu)), dev(su8), bf16_dev(s2), mq.pack_weights(dev(wd)),
            bf16_dev(sd))


@pytest.mark.parametrize("N,K", [(48, 384), (33, 128), (16, 2048), (7, 4096)])
def test_weight_prep_g128(orc, N, K):
    W = synth.weights((90, N), N, K)
    W[3, 128:256] = 0  # an all-zero group
    if N > 5:
        W[5] = 0  # an all-zero row
    W[0, 7] = 3.0  # a group dominated by one large value
    q_ref, s_ref = orc.weight_prep_g128(W)
    q, s = mq.fwht128_weight_prep_g128(dev(W))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(q), q_ref)
    np.testing.assert_array_equal(bf16_host(s), s_ref)


# ----------------------------------------------------------- router gate --

# one wave per expert (up to 16 tokens), 16 x 16 tiles over 8 slices of H (up
# to 256), 16 x 64 tiles over 4 slices beyond (ragged last token block); the
# 16 x 16 tiles over 2 slices where E is not a multiple of 64
@pytest.mark.parametrize("T,E", [(1, 256), (3, 256), (16, 256), (17, 256), (100, 256),
                                 (300, 256), (1000, 256), (2048, 256), (300, 48)])
def test_router_gate(orc, T, E):
    H = 2048
    x = synth.activations((91, T), T, H, 20, 10.0)
    wg = synth.to_bf16_bits(synth.weights((91, E), E, H))
    ref = orc.router_gate_bf16(x, wg)
    lg = mq.router_gate_bf16(bf16_dev(x), bf16_dev(wg))
    lg2 = mq.router_gate_bf16(bf16_dev(x), bf16_dev(wg))
    torch.cuda.synchronize()
    got = host(lg)
    np.testing.assert_array_equal(got, host(lg2))
    xf = orc.bf16_to_f32(x).astype(np.float64)
    wf = orc.bf16_to_f32(wg).astype(np.float64)
    bound = H * 2.0 ** -24 * (np.abs(xf) @ np.abs(wf).T) + 1e-30
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    assert (err <= bound).all(), f"router T={T} E={E}: max err / bound {(err / bound).max():.3f}"
    say(f"router T={T} E={E}: max err / bound {(err / bound).max():.4f}")


def test_router_gate_wide_forms_agree():
    # beyond 256 tokens the expert block per workgroup follows the batch size
    # (64, 32 or 16 experts); a token's logits are the same sums either way
    H, E = 2048, 256
    x = synth.activations((92, 2048), 2048, H, 20, 10.0)
    wg = bf16_dev(synth.to_bf16_bits(synth.weights((92, E), E, H)))
    xd = bf16_dev(x)
    full = host(mq.router_gate_bf16(xd, wg))
    for T in (1000, 300):
        part = host(mq.router_gate_bf16(xd[:T].contiguous(), wg))
        np.testing.assert_array_equal(part, full[:T])


@pytest.mark.parametrize("T", [5, 40])
def test_router_gate_integer_exact(orc, T):
    # small integers: every product and partial sum is exact in fp32
    H, E = 512, 32
    r = np.random.default_rng(92 + T)
    x = r.integers(-8, 9, (T, H)).astype(np.float32)
    wg = r.integers(-8, 9, (E, H)).astype(np.float32)
    ref = orc.router_gate_bf16(synth.to_bf16_bits(x), synth.to_bf16_bits(wg))
    np.testing.assert_array_equal(ref, x @ wg.T)
    got = host(mq.router_gate_bf16(bf16_dev(synth.to_bf16_bits(x)),
                                   bf16_dev(synth.to_bf16_bits(wg))))
    np.testing.assert_array_equal(got, ref)


def test_router_gate_strided(orc):
    T, H, E = 20, 256, 48
    x = synth.activations((93, 0), T, H + 64, 2, 10.0)
    wg = synth.to_bf16_bits(synth.weights((93, 1), E, H))
    ref = orc.router_gate_bf16(np.ascontiguousarray(x[:, :H]), wg)
    lgbig = torch.full((T, E + 16), -7.0, dtype=torch.float32, device="cuda:0")
    mq.router_gate_bf16(bf16_dev(x)[:, :H], bf16_dev(wg), logits=lgbig[:, :E])
    got = host(lgbig)
    assert (got[:, E:] == -7.0).all()
    xf = orc.bf16_to_f32(np.ascontiguousarray(x[:, :H])).astype(np.float64)
    bound = H * 2.0 ** -24 * (np.abs(xf) @ np.abs(orc.bf16_to_f32(wg).astype(np.float64)).T)
    assert (np.abs(got[:, :E] - ref) <= bound + 1e-30).all()


# --------------------------------------------------------- routed experts --

def _check_rot(orc, x, logits, k, W, Wd, label, shared=None, tokens=None):
    """Run the GPU layer on all of x; compare with the oracle on ``tokens``
    (all by default: a token's output depends only on its own row and ids)."""
    q13, s13, q2, s2 = W
    T = x.shape[0]
    ids_ref, w_ref = orc.route_topk(logits, k)
    out, ids, w, dbg = mq.moe_w8a8_rot_forward(
        bf16_dev(x), dev(logits), *Wd, topk=k,
        shared=None if shared is None else dev(shared), debug=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(ids), ids_ref)
    assert ulp_diff_f32(host(w), w_ref).max() <= 1
    sel = np.arange(T) if tokens is None else np.asarray(tokens)
    pairs = (sel[:, None] * k + np.arange(k)[None, :]).reshape(-1)
    out_ref, dref = orc.moe_rot_forward(
        np.ascontiguousarray(x[sel]), ids_ref[sel], w_ref[sel], q13, s13, q2, s2,
        shared=None if shared is None else np.ascontiguousarray(shared[sel]), debug=True)
    np.testing.assert_array_equal(host(dbg["qx"])[sel], dref["qx"])
    np.testing.assert_array_equal(host(dbg["sx"])[sel], dref["sx"])
    act = host(dbg["act"])[pairs]
    assert ulp_diff_f32(act, dref["act"]).max() <= 1, f"{label}: activation"
    same = (act == dref["act"]).all(axis=1)
    assert same.mean() > 0.99
    qa, sa2 = host(dbg["qa"])[pairs], host(dbg["sa2"])[pairs]
    np.testing.assert_array_equal(qa[same], dref["qa"][same])
    np.testing.assert_array_equal(sa2[same], dref["sa2"][same])
    assert np.abs(qa.astype(np.int32) - dref["qa"]).max() <= 1
    flips = int((qa != dref["qa"]).sum())
    assert flips <= max(2, qa.size // 1000), f"{label}: {flips} requant flips"
    got = bf16_host(out)[sel]
    mism = assert_bf16_close(got, out_ref, label)
    pair_ok = ((qa == dref["qa"]).all(axis=1) & (sa2 == dref["sa2"])).reshape(-1, k)
    tok_ok = pair_ok.all(axis=1)
    np.testing.assert_array_equal(got[tok_ok], out_ref[tok_ok])
    say(f"{label}: pairs with equal act {same.mean():.4f}, requant flips {flips}, "
        f"bf16 mismatches {mism} of {out_ref.size}")
    return out


# small shapes: the single-token path, the split-K GEMMs (with the requant in
# gemm2's prologue up to 256 pairs, around the requant kernel beyond); ragged
# expert segments, a zero token
@pytest.mark.parametrize("T,k", [(1, 2), (5, 2), (32, 8), (33, 8), (300, 2), (600, 8)])
def test_rot_moe_small(orc, T, k):
    E, H, I = 8, 256, 128
    W = _rot_weights(orc, (94, 0), E, H, I)
    Wd = _dev_rot_weights(W)
    x = synth.activations((94, T), T, H, 3, 10.0)
    if T > 3:
        x[2] = 0
    logits = synth.router_logits((94, T), T, E)
    _check_rot(orc, x, logits, k, W, Wd, f"rot moe small T={T} k={k}")


@pytest.mark.parametrize("pattern", ["top3", "all", "boundary", "pairs"])
def test_rot_moe_single_token_tied_logits(orc, pattern):
    # one token: each gemm1 workgroup finds its own slot's expert; tied logits
    # must give every slot the expert of the full lower-index selection
    E, H, I, k = 256, 256, 128, 8
    W = _rot_weights(orc, (93, 1), E, H, I)
    Wd = _dev_rot_weights(W)
    x = synth.activations((93, 1), 1, H, 0, 1.0)
    _check_rot(orc, x, tie_logits(pattern, E), k, W, Wd, f"rot moe T=1 ties {pattern}")


def test_rot_moe_wave_per_tile_shapes(orc):
    # 640 pairs take the one-wave-per-tile grouped GEMMs: gemm1 with K = 1024
    # (16 k steps a wave), gemm2 with K = 1536 (24 of 32 k steps, 12 groups),
    # ragged 16-pair blocks in every expert
    E, H, I, k, T = 16, 1024, 1536, 4, 160
    W = _rot_weights(orc, (99, 0), E, H, I)
    Wd = _dev_rot_weights(W)
    x = synth.activations((99, T), T, H, 5, 10.0)
    x[7] = 0
    logits = synth.router_logits((99, T), T, E)
    _check_rot(orc, x, logits, k, W, Wd, "rot moe wave-per-tile shapes")


@pytest.mark.parametrize("T", [3, 100])
def test_rot_moe_with_shared_term(orc, T):
    E, H, I, k = 16, 512, 256, 4
    W = _rot_weights(orc, (95, 0), E, H, I)
    Wd = _dev_rot_weights(W)
    x = synth.activations((95, T), T, H, 5, 10.0)
    logits = synth.router_logits((95, T), T, E)
    shared = (np.random.default_rng(95 + T).standard_normal((T, H)) * 0.05).astype(np.float32)
    _check_rot(orc, x, logits, k, W, Wd, f"rot moe + shared T={T}", shared=shared)


@pytest.mark.parametrize("T", [1, 90, 200])
def test_rot_moe_given_ids_and_skew(orc, T):
    # every token picks expert 0 first: one long segment, the rest short
    E, H, I, k = 8, 256, 256, 3
    W = _rot_weights(orc, (96, 0), E, H, I)
    Wd = _dev_rot_weights(W)
    x = synth.activations((96, T), T, H, 3, 10.0)
    r = np.random.default_rng(96)
    ids = np.stack([np.zeros(T, np.int64)] +
                   [r.integers(1, E, T) for _ in range(k - 1)], axis=1).astype(np.int32)
    for t in range(T):  # distinct ids per token
        while len(set(ids[t])) < k:
            ids[t, 1:] = r.integers(1, E, k - 1)
    w = r.uniform(0.1, 1.0, (T, k)).astype(np.float32)
    out, _, _, dbg = mq.moe_w8a8_rot_forward(bf16_dev(x), None, *Wd, topk=k,
                                             topk_ids=dev(ids), topk_w=dev(w), debug=True)
    torch.cuda.synchronize()
    out_ref, dref = orc.moe_rot_forward(x, ids, w, *W, debug=True)
    assert ulp_diff_f32(host(dbg["act"]), dref["act"]).max() <= 1
    assert_bf16_close(bf16_host(out), out_ref, "rot moe given ids")


@pytest.mark.parametrize("T,I", [(1100, 256), (40, 256), (600, 768)])
def test_rot_moe_wide_scale_range(orc, T, I):
    # some weight rows have one 128-group scaled down by 2^-28: the fold still
    # matches the fp64 in-order sum of the definition (workgroups holding such
    # a column fold in fp64, the others with integers); 40 tokens take the
    # small-batch gemm2 that rotates the activations itself, 600 tokens with
    # I = 768 the gemm2 of eight 128-groups
    E, H, k = 4, 256, 4
    key = (97, 0)
    q13 = np.empty((E, 2 * I, H), np.int8)
    s13 = np.empty((E, 2 * I, H // 128), np.uint16)
    q2 = np.empty((E, H, I), np.int8)
    s2 = np.empty((E, H, I // 128), np.uint16)
    for e in range(E):
        a = synth.expert_weights(key, e, 2 * I, H, synth.T_W)
        b = synth.expert_weights(key, e, H, I, synth.T_W2)
        a[:32, :128] *= np.float32(2.0 ** -28)
        a[200:203, 128:] *= np.float32(2.0 ** -26)
        b[64:96, 128:256] *= np.float32(2.0 ** -30)
        q13[e], s13[e] = orc.weight_prep_g128(a)
        q2[e], s2[e] = orc.weight_prep_g128(b)
    W = (q13, s13, q2, s2)
    x = synth.activations((97, T), T, H, 3, 10.0)
    logits = synth.router_logits((97, T), T, E)
    _check_rot(orc, x, logits, k, W, _dev_rot_weights(W), "rot moe wide scale range")


@pytest.fixture(scope="module")
def full_rot_weights(orc):
    cfg = synth.moe(1)
    E, H, I = cfg["E"], cfg["H"], cfg["I"]
    say(f"preparing rotated expert weights E={E} H={H} I={I}")
    W = _rot_weights(orc, (98, 0), E, H, I)
    return W, _dev_rot_weights(W)


@pytest.mark.parametrize("T", [1, 8, 64, 2048])
def test_rot_moe_full_size(orc, full_rot_weights, T):
    W, Wd = full_rot_weights
    cfg = synth.moe(T)
    E, H, k = cfg["E"], cfg["H"], cfg["k"]
    x = synth.activations((98, T), T, H, 0, 1.0)
    logits = synth.router_logits((98, T), T, E)
    # every token of the batch against the oracle (intermediates included)
    out = _check_rot(orc, x, logits, k, W, Wd, f"rot moe full T={T}")
    out2, _, _ = mq.moe_w8a8_rot_forward(bf16_dev(x), dev(logits), *Wd, topk=k)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bf16_host(out2), bf16_host(out))


# ------------------------------------------------------------ shared expert --

def _check_shared(orc, x, S, Sd, label):
    y_ref, act_ref = orc.shared_expert(x, *S, debug=True)
    y, dbg = mq.shared_expert_w8a8_rot(bf16_dev(x), *Sd, debug=True)
    torch.cuda.synchronize()
    act = host(dbg["act"])
    assert ulp_diff_f32(act, act_ref).max() <= 1, f"{label}: activation"
    same = (act == act_ref).all(axis=1)
    qa_ref, sa_ref = orc.rot_quant_rows(act_ref)
    qa, sa = host(dbg["qa"]), host(dbg["sa"])
    np.testing.assert_array_equal(qa[same], qa_ref[same])
    np.testing.assert_array_equal(sa[same], sa_ref[same])
    assert np.abs(qa.astype(np.int32) - qa_ref).max() <= 1
    yh = host(y)
    err = np.abs(yh.astype(np.float64) - y_ref)
    assert (err <= 1e-3 + 1e-2 * np.abs(y_ref)).all(), f"{label}: max err {err.max():.3e}"
    rows = (qa == qa_ref).all(axis=1) & (sa == sa_ref)
    np.testing.assert_array_equal(yh[rows], y_ref[rows])
    say(f"{label}: rows with equal act {same.mean():.4f}, rows bit-exact {rows.mean():.4f}")
    return y, y_ref


@pytest.mark.parametrize("H", [512, 4096])
def test_shared_expert_wide_scale_range(orc, H):
    # more than 64 rows (H = 512: the one-wave-per-tile GEMMs, which fold in
    # fp64 in group order; H = 4096: the tiled GEMMs, where down-weight rows
    # with one 128-group scaled down by 2^-30 span more than the integer fold
    # allows, so those waves fold in fp64 group by group while the others take
    # the integer fold)
    Is, T = 256, 200
    wgu, su8, s2 = orc.weight_prep_g256(synth.weights((98, 5), 2 * Is, H, tensor_id=synth.T_W))
    Wd = synth.weights((98, 5), H, Is, tensor_id=synth.T_W2)
    Wd[:32, :128] *= np.float32(2.0 ** -30)
    Wd[H // 2:H // 2 + 1, 128:] *= np.float32(2.0 ** -25)
    wd, sd = orc.weight_prep_g128(Wd)
    S = (wgu, su8, s2, wd, sd)
    x = synth.activations((98, 6), T, H, 4, 10.0)
    _check_shared(orc, x, S, _dev_shared_weights(S), f"shared wide scale range H={H}")


@pytest.mark.parametrize("T", [1, 7, 64, 65, 300])
def test_shared_expert_small(orc, T):
    H, Is = 512, 256
    S = _shared_weights(orc, (99, 0), H, Is)
    x = synth.activations((99, T), T, H, 4, 10.0)
    if T > 2:
        x[1] = 0
    _check_shared(orc, x, S, _dev_shared_weights(S), f"shared small T={T}")


@pytest.mark.parametrize("T", [1, 64, 2048])
def test_shared_then_routed_full_size(orc, full_rot_weights, T):
    """The layer as the container runs it: shared expert + routed experts."""
    W, Wd = full_rot_weights
    cfg = synth.moe(T)
    E, H, I, k = cfg["E"], cfg["H"], cfg["I"], cfg["k"]
    S = _shared_weights(orc, (100, 0), H, I)
    x = synth.activations((100, T), T, H, 0, 1.0)
    logits = synth.router_logits((100, T), T, E)
    sel = np.arange(T)
    y, _ = _check_shared(orc, np.ascontiguousarray(x[sel]), S, _dev_shared_weights(S),
                         f"shared full T={len(sel)}")
    y_ref = orc.shared_expert(np.ascontiguousarray(x[sel]), *S)
    Sd = _dev_shared_weights(S)
    y_all = mq.shared_expert_w8a8_rot(bf16_dev(x), *Sd)
    out, _, _ = mq.moe_w8a8_rot_forward(bf16_dev(x), dev(logits), *Wd, topk=k, shared=y_all)
    torch.cuda.synchronize()
    # the shared expert in its own call agrees with the one checked above
    np.testing.assert_array_equal(host(y_all)[sel], host(y))
    ids_ref, w_ref = orc.route_topk(logits[sel], k)
    out_ref = orc.moe_rot_forward(np.ascontiguousarray(x[sel]), ids_ref, w_ref, *W,
                                  shared=y_ref)
    mism = assert_bf16_close(bf16_host(out)[sel], out_ref, f"shared + routed T={T}")
    say(f"shared + routed T={T}: bf16 mismatches {mism} of {out_ref.size}")


# ------------------------------------------------ the layer with its shared --

def _check_layer(orc, x, logits, k, W, Wd, S, Sd, label):
    """The one-call layer: bit for bit the two-call composition on the GPU
    (shared expert, then the routed layer with its output as the shared
    term), and against the oracle's routed layer with the oracle's shared
    expert as its shared term."""
    out, ids, wt = mq.moe_w8a8_rot_shared_forward(bf16_dev(x), dev(logits), *Wd, topk=k,
                                                  shared_w=Sd)
    y = mq.shared_expert_w8a8_rot(bf16_dev(x), *Sd)
    out2, ids2, wt2 = mq.moe_w8a8_rot_forward(bf16_dev(x), dev(logits), *Wd, topk=k, shared=y)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(ids), host(ids2))
    np.testing.assert_array_equal(host(wt), host(wt2))
    np.testing.assert_array_equal(bf16_host(out), bf16_host(out2))
    ids_ref, w_ref = orc.route_topk(logits, k)
    np.testing.assert_array_equal(host(ids), ids_ref)
    assert ulp_diff_f32(host(wt), w_ref).max() <= 1
    y_ref = orc.shared_expert(x, *S)
    out_ref = orc.moe_rot_forward(x, ids_ref, w_ref, *W, shared=y_ref)
    mism = assert_bf16_close(bf16_host(out), out_ref, label)
    say(f"{label}: bf16 mismatches {mism} of {out_ref.size}")


# one token runs the shared expert inside the two routed launches (gate/up
# tiles beside gemm1's, the down projection as one more pair of gemm2) when
# k <= 15, I <= 1024, Is <= 1024 and k I/128 + Is/128 <= 64; else, and for
# more tokens, the shared expert and the routed layer run one after the other
@pytest.mark.parametrize("T,E,H,I,Is,k", [
    (1, 8, 256, 128, 128, 2),
    (1, 16, 512, 256, 384, 4),    # more shared gate/up tiles than routed ones
    (1, 16, 512, 384, 128, 4),    # fewer
    (1, 32, 256, 128, 128, 15),   # the most pairs the single-token form takes
    (1, 32, 256, 128, 128, 16),   # one more: composed
    (1, 8, 256, 128, 1152, 2),    # a shared row longer than 1024: composed
    (3, 8, 256, 128, 128, 2),
    (40, 16, 512, 256, 256, 4),
])
def test_rot_layer_with_shared(orc, T, E, H, I, Is, k):
    W = _rot_weights(orc, (101, E, I), E, H, I)
    S = _shared_weights(orc, (101, Is), H, Is)
    x = synth.activations((101, T), T, H, 3, 10.0)
    logits = synth.router_logits((101, T, E), T, E)
    _check_layer(orc, x, logits, k, W, _dev_rot_weights(W), S, _dev_shared_weights(S),
                 f"rot layer + shared T={T} E={E} I={I} Is={Is} k={k}")


@pytest.mark.parametrize("T", [1, 64, 2048])
def test_rot_layer_with_shared_full_size(orc, full_rot_weights, T):
    W, Wd = full_rot_weights
    cfg = synth.moe(T)
    E, H, I, k = cfg["E"], cfg["H"], cfg["I"], cfg["k"]
    S = _shared_weights(orc, (102, 0), H, I)
    x = synth.activations((102, T), T, H, 0, 1.0)
    logits = synth.router_logits((102, T), T, E)
    _check_layer(orc, x, logits, k, W, Wd, S, _dev_shared_weights(S),
                 f"rot layer + shared full T={T}")

