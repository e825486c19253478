"""Run-to-run determinism and batch invariance of the GPU path, through the C ABI.

Determinism: 100 back-to-back runs of the same call on the same inputs give
bit-identical outputs (decode linear, tiled prefill linear, Hadamard linear,
MoE at 1, 64 and 2048 tokens).  Nothing in the kernels depends on timing:
integer sums are exact and every floating-point reduction has a fixed order.

Batch invariance: a token's output does not depend on the batch it arrives
in, although each batch size takes other kernels (one-launch decode linear,
decode GEMM, the tiles of the prefill plan; single-token, small-batch and
large-batch MoE paths).  Every path performs the same exact integer sums and
the same fp32 operations per output, so the rows must agree bit for bit; the
first rows are also checked against the oracle.
"""
import numpy as np
import pytest
import torch

import moe_quant_token_amd as mq
import synth
from tests._util import bf16_dev, bf16_host, dev, say

pytestmark = pytest.mark.gpu

REPEATS = 100


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mq.lib()


def _same(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def _repeat(fn, what):
    ref = fn().clone()
    for i in range(REPEATS - 1):
        out = fn()
        assert _same(out, ref), f"{what}: run {i + 1} differs from run 0"
    torch.cuda.synchronize()
    return ref


@pytest.fixture(scope="module")
def dense_weights(orc):
    out = {}
    for si, (K, N, name) in enumerate(synth.DECODE_SHAPES):
        W = synth.weights(synth.decode_linear(1, si)["wkey"], N, K)
        qw, sw = orc.quant_rows(W)
        out[name] = (qw, sw, mq.pack_weights(dev(qw)), dev(sw))
    return out


@pytest.mark.parametrize("name", ["gate_up", "down"])
def test_dense_linear_repeat_and_batch_invariance(orc, dense_weights, name):
    qw, sw, qp, sw_d = dense_weights[name]
    N, K = qw.shape
    x = synth.activations((60, K), 4096, K, int(round(0.01 * K)), 10.0)
    x_d = bf16_dev(x)
    ys = {}
    for M in (1, 2, 8, 16, 17, 64, 300, 4096):
        xm = x_d[:M]
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x_d.device)
        ws = torch.empty(max(1, mq.linear_w8a8_workspace_bytes(M, N, K)), dtype=torch.uint8,
                         device=x_d.device)
        say(f"{name} M={M}: {REPEATS} repeats")
        ys[M] = _repeat(lambda: mq.linear_w8a8_packed(xm, qp, sw_d, N, y=y, ws=ws),
                        f"{name} M={M}")
    for M, y in ys.items():
        assert _same(y, ys[4096][:M]), f"{name}: rows of the M={M} batch differ from M=4096"
    np.testing.assert_array_equal(bf16_host(ys[8]), orc.linear_w8a8(x[:8], qw, sw))


@pytest.fixture(scope="module")
def moe_layer(orc):
    cfg = synth.moe(1)
    E, H, I = cfg["E"], cfg["H"], cfg["I"]
    q13 = np.empty((E, 2 * I, H), np.int8)
    s13 = np.empty((E, 2 * I), np.float32)
    q2 = np.empty((E, H, I), np.int8)
    s2 = np.empty((E, H), np.float32)
    for e in range(E):
        q13[e], s13[e] = orc.quant_rows(synth.expert_weights(cfg["wkey"], e, 2 * I, H, synth.T_W))
        q2[e], s2[e] = orc.quant_rows(synth.expert_weights(cfg["wkey"], e, H, I, synth.T_W2))
    w13, w2 = mq.pack_moe_weights(dev(q13), dev(q2))
    return (q13, s13, q2, s2), (w13, dev(s13), w2, dev(s2))


def test_moe_repeat_and_batch_invariance(orc, moe_layer):
    W, Wd = moe_layer
    cfg = synth.moe(2048)
    T, H, E, k = 2048, cfg["H"], cfg["E"], cfg["k"]
    x = synth.activations(cfg["xkey"], T, H, 0, 1.0)
    logits = synth.router_logits(cfg["xkey"], T, E)
    x_d, l_d = bf16_dev(x), dev(logits)
    outs = {}
    for t in (1, 64, 2048):
        xs, ls = x_d[:t], l_d[:t]
        out = torch.empty((t, H), dtype=torch.bfloat16, device=x_d.device)
        ids = torch.empty((t, k), dtype=torch.int32, device=x_d.device)
        wt = torch.empty((t, k), dtype=torch.float32, device=x_d.device)
        ws = torch.empty(mq.moe_w8a8_workspace_bytes(t, H, E, cfg["I"], k), dtype=torch.uint8,
                         device=x_d.device)
        say(f"moe T={t}: {REPEATS} repeats")
        outs[t] = _repeat(lambda: mq.moe_w8a8_forward(xs, ls, *Wd, topk=k, topk_ids=ids,
                                                      topk_w=wt, out=out, ws=ws,
                                                      packed=True)[0], f"moe T={t}")
    assert _same(outs[64], outs[2048][:64]), "MoE: the 64-token batch differs from T=2048"
    # single tokens at several places of the batch (the single-token path)
    for t in (0, 5, 63, 1000, 2047):
        one = mq.moe_w8a8_forward(x_d[t:t + 1], l_d[t:t + 1], *Wd, topk=k, packed=True)[0]
        assert _same(one, outs[2048][t:t + 1]), f"MoE: token {t} alone differs from the batch"
    ids_ref, w_ref = orc.route_topk(logits[:1], k)
    np.testing.assert_array_equal(bf16_host(outs[1]), orc.moe_forward(x[:1], ids_ref, w_ref, *W))


def test_hadamard_linear_repeat_and_batch_invariance(orc):
    cfg = synth.hadamard_linear(256)
    K, N = cfg["K"], cfg["N"]
    qw, su8, s2 = orc.weight_prep_g256(synth.weights(cfg["wkey"], N, K))
    qp, su_d, s2_d = mq.pack_weights(dev(qw)), dev(su8), dev(s2)
    x = synth.activations(cfg["xkey"], 256, K, cfg["n_outliers"], cfg["outlier_scale"],
                          heavy_tail=True)
    x_d = bf16_dev(x)
    ys = {}
    for M in (1, 4, 16, 17, 32, 100, 256):
        xm = x_d[:M]
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x_d.device)
        ws = torch.empty(max(256, mq.linear_w8a8_g256_workspace_bytes(M, N, K)),
                         dtype=torch.uint8, device=x_d.device)
        say(f"g256 linear M={M}: {REPEATS} repeats")
        ys[M] = _repeat(lambda: mq.linear_w8a8_g256_packed(xm, qp, su_d, s2_d, y=y, ws=ws),
                        f"g256 M={M}")
    for M, y in ys.items():
        assert _same(y, ys[256][:M]), f"g256: rows of the M={M} batch differ from M=256"
    qa, sa = orc.fwht128_quant(x[:4])
    np.testing.assert_array_equal(bf16_host(ys[4]), orc.gemm_g256(qa, sa, qw, su8, s2))
