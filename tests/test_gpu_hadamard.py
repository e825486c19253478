"""GPU parity of the Hadamard-domain (fwht128, g256) path through the C ABI.

fwht128_quant codes/scales, the rotated weight preparation (codes, u8 group
scales, bf16 row scales) and the g256 GEMM are compared bit-exactly with the
oracle: the transform performs the same fp32 additions in the same stage
order, and the g256 epilogue is an exact int64 sum followed by the same fp64
products.  bf16 outputs are also checked against the 1e-3 abs + 1e-2 rel bar.
"""
import numpy as np
import pytest
import torch

import moe_quant_token_amd as mq
import synth
from tests._util import assert_bf16_close, bf16_dev, bf16_host, dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mq.lib()


@pytest.mark.parametrize("M,K", [(1, 2048), (256, 2048), (7, 128), (3, 16384), (33, 640),
                                 (40, 4096), (17, 4224), (21, 384)])
def test_fwht128_quant_bit_exact(orc, M, K):
    say(f"fwht128_quant M={M} K={K}")
    x = synth.activations((50, M, K), M, K, max(1, K // 100), 10.0, heavy_tail=True)
    if M > 2:
        x[2] = 0
    q_ref, s_ref = orc.fwht128_quant(x)
    q, s = mq.fwht128_quant(bf16_dev(x))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(s), s_ref)
    np.testing.assert_array_equal(host(q), q_ref)


@pytest.mark.parametrize("N,K", [(64, 512), (8192, 2048), (16, 16384)])
def test_weight_prep_bit_exact(orc, N, K):
    say(f"weight prep N={N} K={K}")
    W = synth.weights((51, N), N, K)
    W[3 % N] = 0
    W[min(5, N - 1), :256] = 0
    qw_ref, su_ref, s2_ref = orc.weight_prep_g256(W)
    qw, su8, s2 = mq.fwht128_weight_prep_g256(dev(W))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bf16_host(s2), s2_ref)
    np.testing.assert_array_equal(host(su8), su_ref)
    np.testing.assert_array_equal(host(qw), qw_ref)


@pytest.fixture(scope="module")
def rotated_weights(orc):
    cfg = synth.hadamard_linear(1)
    W = synth.weights(cfg["wkey"], cfg["N"], cfg["K"])
    return orc.weight_prep_g256(W)


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("M", [1, 4, 16, 17, 256])
def test_g256_full_size(orc, rotated_weights, M, packed):
    cfg = synth.hadamard_linear(M)
    K, N = cfg["K"], cfg["N"]
    say(f"g256 M={M} K={K} N={N} packed={packed}")
    qw, su8, s2 = rotated_weights
    x = synth.activations(cfg["xkey"], M, K, cfg["n_outliers"], cfg["outlier_scale"],
                          heavy_tail=True)
    qa, sa = orc.fwht128_quant(x)
    qa_d, sa_d = mq.fwht128_quant(bf16_dev(x))
    qw_d = mq.pack_weights(dev(qw)) if packed else dev(qw)
    y = mq.gemm_w8a8_g256(qa_d, sa_d, qw_d, dev(su8), dev(s2), packed=packed)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(qa_d), qa)
    yh = bf16_host(y)
    y_ref = orc.gemm_g256(qa, sa, qw, su8, s2)
    np.testing.assert_array_equal(yh, y_ref)
    assert_bf16_close(yh, y_ref, "g256")


@pytest.mark.parametrize("M", [1, 16, 17, 256])
def test_linear_g256_full_size(orc, rotated_weights, M):
    # the fused entry: fwht128 + quant (tile-layout codes when M > 16) + g256
    cfg = synth.hadamard_linear(M)
    K, N = cfg["K"], cfg["N"]
    say(f"linear g256 M={M}")
    qw, su8, s2 = rotated_weights
    x = synth.activations(cfg["xkey"], M, K, cfg["n_outliers"], cfg["outlier_scale"],
                          heavy_tail=True)
    if M > 2:
        x[1] = 0
    qa, sa = orc.fwht128_quant(x)
    y = bf16_host(mq.linear_w8a8_g256_packed(bf16_dev(x), mq.pack_weights(dev(qw)), dev(su8),
                                             dev(s2)))
    np.testing.assert_array_equal(y, orc.gemm_g256(qa, sa, qw, su8, s2))
    if M > 2:
        assert not y[1].any()


@pytest.mark.parametrize("K,N,zero", [(256, 16, False), (768, 48, False), (4096, 64, False),
                                       (4096, 32, True), (4352, 32, False)])
def test_linear_g256_single_token(orc, K, N, zero):
    # one token: rotation, quant and GEMM in one launch up to K=4096, the
    # two-launch path beyond; bit-exact either way, an all-zero row included
    say(f"linear g256 single token K={K} N={N} zero={zero}")
    W = synth.weights((54, K), N, K)
    qw, su8, s2 = orc.weight_prep_g256(W)
    x = synth.activations((55, K), 1, K, 4, 10.0, heavy_tail=True)
    if zero:
        x[:] = 0
    qa, sa = orc.fwht128_quant(x)
    y = mq.linear_w8a8_g256_packed(bf16_dev(x), mq.pack_weights(dev(qw)), dev(su8),
                                   dev(s2.view(np.int16)).view(torch.bfloat16))
    np.testing.assert_array_equal(bf16_host(y), orc.gemm_g256(qa, sa, qw, su8, s2))
    if zero:
        assert not bf16_host(y).any()


@pytest.mark.parametrize("M,K,N", [(33, 1024, 128), (64, 2048, 256), (100, 2048, 1152),
                                   (200, 1024, 384), (256, 2048, 8192), (129, 4096, 80),
                                   (257, 2048, 96), (128, 2048, 1040), (320, 1024, 2048)])
def test_linear_g256_mid_batches(orc, M, K, N):
    # 33 to 320 rows through the fused entry (tile-layout codes, the g256 tile
    # kernel), ragged last row tile, K = 4096, a half-filled last 32-column
    # block, a last 64-column tile with one 16-column tile, an all-zero row
    say(f"linear g256 mid batches M={M} K={K} N={N}")
    W = synth.weights((58, K, N), N, K)
    qw, su8, s2 = orc.weight_prep_g256(W)
    x = synth.activations((59, M, K), M, K, max(1, K // 100), 10.0, heavy_tail=True)
    x[M // 2] = 0
    qa, sa = orc.fwht128_quant(x)
    y = mq.linear_w8a8_g256_packed(bf16_dev(x), mq.pack_weights(dev(qw)), dev(su8),
                                   dev(s2.view(np.int16)).view(torch.bfloat16))
    got = bf16_host(y)
    np.testing.assert_array_equal(got, orc.gemm_g256(qa, sa, qw, su8, s2))
    assert not got[M // 2].any()


def test_linear_g256_ragged_stride(orc):
    r = np.random.default_rng(9)
    M, K, N = 37, 768, 80
    W = synth.weights((52, N), N, K)
    qw, su8, s2 = orc.weight_prep_g256(W)
    x = synth.activations((53, M), M, K, 8, 10.0, heavy_tail=True)
    big = np.zeros((M, K + 128), np.uint16)
    big[:, :K] = x
    qa, sa = orc.fwht128_quant(x)
    y = mq.linear_w8a8_g256_packed(bf16_dev(big)[:, :K], mq.pack_weights(dev(qw)), dev(su8),
                                   dev(s2.view(np.int16)).view(torch.bfloat16))
    np.testing.assert_array_equal(bf16_host(y), orc.gemm_g256(qa, sa, qw, su8, s2))


@pytest.mark.parametrize("packed", [False, True])
def test_g256_small_all_edges(orc, packed):
    r = np.random.default_rng(3)
    for (M, K, N) in [(1, 256, 16), (5, 512, 48), (40, 768, 80), (16, 16384, 32),
                      (70, 2304, 144), (17, 1280, 48), (32, 2048, 112)]:
        qa = r.integers(-127, 128, (M, K)).astype(np.int8)
        qw = r.integers(-127, 128, (N, K)).astype(np.int8)
        qa[0] = 127
        qw[0] = 127  # large sums: 255 * 127^2 * K exceeds int32
        su8 = r.integers(1, 256, (N, K // 256)).astype(np.uint8)
        su8[0] = 255
        s2 = synth.to_bf16_bits(r.random(N).astype(np.float32) * 1e-4)
        sa = (r.random(M) * 0.1).astype(np.float32)
        y_ref = orc.gemm_g256(qa, sa, qw, su8, s2)
        qw_d = mq.pack_weights(dev(qw)) if packed else dev(qw)
        y = mq.gemm_w8a8_g256(dev(qa), dev(sa), qw_d, dev(su8),
                              dev(s2.view(np.int16)).view(torch.bfloat16), packed=packed)
        np.testing.assert_array_equal(bf16_host(y), y_ref)
