"""GPU parity of the routed int8 MoE layer through the C ABI.

Routing ids are compared exactly (inputs are tie-free at the top-k boundary,
checked), routing weights to within 1 fp32 ulp, the debug int32 sums of both
grouped GEMMs bit-exactly (gemm2 wherever the requantised codes agree), the
SiLU activation to within 1 fp32 ulp, and the bf16 output within
1e-3 abs + 1e-2 rel.  Requantised codes may differ by one only where the
oracle's act/scale lies next to a rounding boundary.
"""
import numpy as np
import pytest
import torch

import moe_quant_token_amd as mq
import synth
from tests._util import (DEV, assert_bf16_close, bf16_dev, bf16_host, dev, host, say,
                         tie_logits, ulp_diff_f32)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mq.lib()


def _weights(orc, wkey, E, H, I):
    q13 = np.empty((E, 2 * I, H), np.int8)
    s13 = np.empty((E, 2 * I), np.float32)
    q2 = np.empty((E, H, I), np.int8)
    s2 = np.empty((E, H), np.float32)
    for e in range(E):
        q13[e], s13[e] = orc.quant_rows(synth.expert_weights(wkey, e, 2 * I, H, synth.T_W))
        q2[e], s2[e] = orc.quant_rows(synth.expert_weights(wkey, e, H, I, synth.T_W2))
    return q13, s13, q2, s2


def _tie_free(logits, k):
    srt = -np.sort(-logits, axis=1)
    return bool((srt[:, k - 1] != srt[:, k]).all()) if logits.shape[1] > k else True


def _dev_weights(W, packed):
    q13, s13, q2, s2 = [dev(a) for a in W]
    if packed:
        q13, q2 = mq.pack_moe_weights(q13, q2)
    return q13, s13, q2, s2


def _check_full(orc, x, logits, k, W, T, label, packed=False, Wd=None):
    q13, s13, q2, s2 = W
    E = q13.shape[0]
    ids_ref, w_ref = orc.route_topk(logits, k)
    out_ref, dref = orc.moe_forward(x, ids_ref, w_ref, q13, s13, q2, s2, debug=True)
    Wd = _dev_weights(W, packed) if Wd is None else Wd
    out, ids, w, dbg = mq.moe_w8a8_forward(bf16_dev(x), dev(logits), *Wd, topk=k, debug=True,
                                           packed=packed)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(ids), ids_ref)
    assert ulp_diff_f32(host(w), w_ref).max() <= 1
    np.testing.assert_array_equal(host(dbg["qx"]), dref["qx"])
    np.testing.assert_array_equal(host(dbg["sx"]), dref["sx"])
    np.testing.assert_array_equal(host(dbg["acc1"]), dref["acc1"])
    act = host(dbg["act"])
    assert ulp_diff_f32(act, dref["act"]).max() <= 1, "SiLU activation"
    qa = host(dbg["qa"])
    same_row = (act == dref["act"]).all(axis=1)
    assert same_row.mean() > 0.99
    np.testing.assert_array_equal(qa[same_row], dref["qa"][same_row])
    np.testing.assert_array_equal(host(dbg["sa2"])[same_row], dref["sa2"][same_row])
    flips = int((qa != dref["qa"]).sum())
    assert np.abs(qa.astype(np.int32) - dref["qa"]).max() <= 1
    assert flips <= max(2, qa.size // 1000)
    qa_same = (qa == dref["qa"]).all(axis=1)
    np.testing.assert_array_equal(host(dbg["acc2"])[qa_same], dref["acc2"][qa_same])
    mism = assert_bf16_close(bf16_host(out), out_ref, label)
    say(f"{label}: requant flips {flips}, bf16 mismatches {mism} of {out_ref.size}")
    return out


@pytest.mark.parametrize("packed", [False, True])
def test_small_full_pipeline(orc, packed):
    T, E, H, I, k = 37, 16, 256, 128, 4
    key = (40, 1)
    W = _weights(orc, key, E, H, I)
    x = synth.activations(key, T, H, 0, 1.0)
    logits = synth.router_logits(key, T, E)
    assert _tie_free(logits, k)
    Wd = _dev_weights(W, packed)
    out = _check_full(orc, x, logits, k, W, T, "moe small", packed=packed, Wd=Wd)
    # determinism: a second run is bit-identical
    out2 = mq.moe_w8a8_forward(bf16_dev(x), dev(logits), *Wd, topk=k, packed=packed)[0]
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("H,k,zero", [(256, 8, False), (2112, 1, False), (2112, 16, False),
                                      (256, 8, True)])
def test_single_token_fused_path(orc, H, k, zero, packed):
    # T=1 with router logits: routing and quant run inside gemm1 (every
    # workgroup routes the token itself).  H=256 leaves waves without a k
    # chunk; H=2112 takes a second, partial round of weight loads; an
    # all-zero token has scale 0 and zero activations.
    T, E, I = 1, 32, 128
    key = (48, H * 100 + k)
    W = _weights(orc, key, E, H, I)
    x = synth.activations(key, T, H, 0, 1.0)
    if zero:
        x[:] = 0
    logits = synth.router_logits(key, T, E)
    assert _tie_free(logits, k)
    out = _check_full(orc, x, logits, k, W, T, f"moe T=1 H={H} k={k}", packed=packed)
    if zero:
        assert not bf16_host(out).any()


@pytest.mark.parametrize("packed", [False, True])
def test_large_batch_path(orc, packed):
    # more than 2048 routed pairs: the routing/sort/quant kernels, the
    # 128-pair m-block grouped GEMMs (several blocks per expert here) and the
    # separate requant kernel
    T, E, H, I, k = 700, 8, 128, 64, 4
    key = (43, 1)
    W = _weights(orc, key, E, H, I)
    x = synth.activations(key, T, H, 0, 1.0)
    logits = synth.router_logits(key, T, E)
    logits[:, 2] += 1.5  # a hot expert: most tokens route to expert 2
    assert _tie_free(logits, k)
    _check_full(orc, x, logits, k, W, T, "moe large-batch path", packed=packed)


@pytest.mark.parametrize("packed", [False, True])
def test_large_batch_narrow_hidden(orc, packed):
    # large path with H % 128 != 0: gemm2 uses 64-row weight blocks
    T, E, H, I, k = 600, 4, 192, 128, 4
    key = (44, 1)
    W = _weights(orc, key, E, H, I)
    x = synth.activations(key, T, H, 0, 1.0)
    logits = synth.router_logits(key, T, E)
    assert _tie_free(logits, k)
    _check_full(orc, x, logits, k, W, T, "moe large-batch H=192", packed=packed)


@pytest.mark.parametrize("packed", [False, True])
def test_large_batch_wide_hidden(orc, packed):
    # large path with H = 1024: each gemm2 workgroup walks 8 weight blocks
    T, E, H, I, k = 520, 4, 1024, 64, 4
    key = (46, 1)
    W = _weights(orc, key, E, H, I)
    x = synth.activations(key, T, H, 0, 1.0)
    logits = synth.router_logits(key, T, E)
    assert _tie_free(logits, k)
    _check_full(orc, x, logits, k, W, T, "moe large-batch H=1024", packed=packed)


def test_large_batch_wide_intermediate(orc):
    # large path with I > 1024 (the requant keeps 64 values per lane)
    T, E, H, I, k = 520, 4, 64, 1088, 4
    key = (45, 1)
    W = _weights(orc, key, E, H, I)
    x = synth.activations(key, T, H, 0, 1.0)
    logits = synth.router_logits(key, T, E)
    assert _tie_free(logits, k)
    _check_full(orc, x, logits, k, W, T, "moe large-batch I=1088", packed=True)


def test_large_batch_more_pairs_than_one_sort_batch(orc):
    # 16800 routed pairs: more than the 16 x 1024 the sort keeps in registers,
    # so it takes the path that stores each pair's rank and reads it back
    T, E, H, I, k = 2100, 16, 64, 64, 8
    key = (47, 1)
    W = _weights(orc, key, E, H, I)
    x = synth.activations(key, T, H, 0, 1.0)
    logits = synth.router_logits(key, T, E)
    assert T * k > 16 * 1024 and _tie_free(logits, k)
    _check_full(orc, x, logits, k, W, T, "moe 16800 pairs", packed=True)


@pytest.mark.parametrize("T", [1, 5, 40])
def test_routing_more_than_256_experts(orc, T):
    # E > 256: each routing lane holds 16 logits instead of 4; T=1 takes the
    # fused single-token path, T=5 the one-workgroup prep, T=40 routing +
    # quant one wave per token
    E, H, I, k = 320, 128, 64, 8
    key = (49, T)
    W = _weights(orc, key, E, H, I)
    x = synth.activations(key, T, H, 0, 1.0)
    logits = synth.router_logits(key, T, E)
    logits[:, 300:] += 0.5  # favour experts past 256 so some are selected
    assert _tie_free(logits, k)
    _check_full(orc, x, logits, k, W, T, f"moe E=320 T={T}", packed=True)


def test_given_routing_hot_expert_and_edges(orc):
    # logits=None: the caller supplies ids/weights.  Most tokens go to expert 3
    # (a segment far longer than one 64-pair pass); expert 0 gets none.
    T, E, H, I, k = 150, 8, 128, 64, 2
    key = (41, 1)
    W = _weights(orc, key, E, H, I)
    x = synth.activations(key, T, H, 0, 1.0)
    x[5] = 0  # an all-zero token
    r = np.random.default_rng(5)
    ids = np.stack([np.full(T, 3), r.integers(1, E, T)], 1).astype(np.int32)
    ids[ids[:, 1] == 3, 1] = 4
    w = r.random((T, k)).astype(np.float32)
    w /= w.sum(1, keepdims=True)
    out_ref = orc.moe_forward(x, ids, w, *W)
    for packed in (False, True):
        out, ids_o, w_o = mq.moe_w8a8_forward(bf16_dev(x), None, *_dev_weights(W, packed), topk=k,
                                              topk_ids=dev(ids), topk_w=dev(w), packed=packed)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(ids_o), ids)
        got = bf16_host(out)
        assert_bf16_close(got, out_ref, "moe given routing")
        assert not got[5].any()


def test_single_expert_top1(orc):
    T, E, H, I, k = 9, 1, 192, 64, 1
    key = (42, 1)
    W = _weights(orc, key, E, H, I)
    x = synth.activations(key, T, H, 0, 1.0)
    logits = synth.router_logits(key, T, E)
    _check_full(orc, x, logits, k, W, T, "moe E=1 k=1")


def test_routing_ties_lower_index():
    T, E, k = 4, 32, 8
    logits = np.zeros((T, E), np.float32)
    logits[0, [5, 9, 2]] = 1.0          # three-way tie at the top
    logits[1, :] = 0.5                  # all equal: ids 0..7
    logits[2, ::-1] = np.arange(E, dtype=np.float32)
    logits[3, [31, 30]] = 2.0
    H, I = 64, 64
    x = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    w13 = torch.zeros((E, 2 * I, H), dtype=torch.int8, device=DEV)
    s13 = torch.zeros((E, 2 * I), dtype=torch.float32, device=DEV)
    w2 = torch.zeros((E, H, I), dtype=torch.int8, device=DEV)
    s2 = torch.zeros((E, H), dtype=torch.float32, device=DEV)
    out, ids, w = mq.moe_w8a8_forward(x, dev(logits), w13, s13, w2, s2, topk=k)
    ids = host(ids)
    np.testing.assert_array_equal(ids[0, :3], [2, 5, 9])
    np.testing.assert_array_equal(ids[0, 3:], [0, 1, 3, 4, 6])
    np.testing.assert_array_equal(ids[1], np.arange(8))
    np.testing.assert_array_equal(ids[2], np.arange(8))
    np.testing.assert_array_equal(ids[3, :2], [30, 31])
    np.testing.assert_allclose(host(w).sum(1), 1.0, atol=1e-6)
    assert not bf16_host(out).any()


@pytest.mark.parametrize("E", [32, 256])
@pytest.mark.parametrize("pattern", ["top3", "all", "boundary", "pairs"])
def test_single_token_tied_logits(orc, E, pattern):
    # T=1: each gemm1 workgroup finds its own slot's expert; with tied logits
    # every slot must still follow the lower-index rule of the full selection
    # (checked through each slot's int32 sums against the oracle)
    T, H, I, k = 1, 256, 128, 8
    key = (49, E)
    W = _weights(orc, key, E, H, I)
    x = synth.activations(key, T, H, 0, 1.0)
    _check_full(orc, x, tie_logits(pattern, E), k, W, T, f"moe T=1 ties {pattern} E={E}",
                packed=True)


@pytest.fixture(scope="module")
def full_moe(orc):
    cfg = synth.moe(1)
    E, H, I = cfg["E"], cfg["H"], cfg["I"]
    say("generating full-size MoE weights (256 experts)")
    W = _weights(orc, cfg["wkey"], E, H, I)
    return W, _dev_weights(W, True)


@pytest.mark.parametrize("T", [1, 64])
def test_full_size_all_tokens(orc, full_moe, T):
    cfg = synth.moe(T)
    say(f"moe full size T={T}")
    W, Wd = full_moe
    x = synth.activations(cfg["xkey"], T, cfg["H"], 0, 1.0)
    logits = synth.router_logits(cfg["xkey"], T, cfg["E"])
    assert _tie_free(logits, cfg["k"])
    _check_full(orc, x, logits, cfg["k"], W, T, f"moe T={T}", packed=True, Wd=Wd)


def test_full_size_t2048_all_tokens(orc, full_moe):
    # every token and every intermediate of the large-batch path at full size
    cfg = synth.moe(2048)
    T, k = 2048, cfg["k"]
    say("moe full size T=2048 (all tokens, all intermediates)")
    W, Wd = full_moe
    x = synth.activations(cfg["xkey"], T, cfg["H"], 0, 1.0)
    logits = synth.router_logits(cfg["xkey"], T, cfg["E"])
    assert _tie_free(logits, k)
    _check_full(orc, x, logits, k, W, T, "moe T=2048", packed=True, Wd=Wd)


@pytest.mark.parametrize("T", [1, 5, 40, 600])
def test_hidden_above_4096(orc, T):
    # H > 4096: the token rows no longer fit the registers the routing/quant
    # waves hold them in and are read a second time (single token, one-
    # workgroup prep, wave-per-token routing + quant, large path)
    E, H, I, k = 16, 4160, 64, 4
    key = (56, T)
    W = _weights(orc, key, E, H, I)
    x = synth.activations(key, T, H, 0, 1.0)
    logits = synth.router_logits(key, T, E)
    assert _tie_free(logits, k)
    _check_full(orc, x, logits, k, W, T, f"moe H=4160 T={T}", packed=True)


@pytest.mark.parametrize("packed", [False, True])
def test_few_pairs_wide_intermediate(orc, packed):
    # few routed pairs but I > 2048: too wide for the small-batch gemm2's LDS
    # rows, so the large-batch kernels run on a handful of pairs
    T, E, H, I, k = 3, 4, 128, 2112, 2
    key = (57, 1)
    W = _weights(orc, key, E, H, I)
    x = synth.activations(key, T, H, 0, 1.0)
    logits = synth.router_logits(key, T, E)
    assert _tie_free(logits, k)
    _check_full(orc, x, logits, k, W, T, "moe I=2112 T=3", packed=packed)
