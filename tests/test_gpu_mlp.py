"""GPU parity of the dense W8A8 MLP block (gate_up -> SiLU(gate)*up -> per-token
requant -> down) through the C ABI, against the CPU oracle.

Bar: the fp32 activation within 1 fp32 ulp (the GPU's fp64 exp is not the
host's libm exp); the requantised codes and scales bit-exact on every row
whose activation agrees bit for bit, elsewhere codes within one step where
the quotient sits next to a rounding boundary (counted, rare); the bf16
output within 1e-3 abs + 1e-2 rel, and bit-exact on rows whose codes agree.
"""
import numpy as np
import pytest
import torch

import moe_quant_token_amd as mq
import synth
from tests._util import assert_bf16_close, bf16_dev, bf16_host, dev, host, say, ulp_diff_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mq.lib()


def _weights(orc, key, K, I, N):
    qgu, sgu = orc.quant_rows(synth.weights(key, 2 * I, K))
    qd, sd = orc.quant_rows(synth.weights(key, N, I, tensor_id=synth.T_W2))
    return qgu, sgu, qd, sd


def _dev_weights(W):
    qgu, sgu, qd, sd = W
    return mq.pack_weights(dev(qgu)), dev(sgu), mq.pack_weights(dev(qd)), dev(sd)


def _check(orc, x, W, Wd, label, x_d=None):
    qgu, sgu, qd, sd = W
    I, N = qgu.shape[0] // 2, qd.shape[0]
    y_ref, d = orc.mlp_forward(x, qgu, sgu, qd, sd, debug=True)
    y, g = mq.mlp_w8a8_packed(bf16_dev(x) if x_d is None else x_d, Wd[0], Wd[1], Wd[2], Wd[3],
                              I, N, debug=True)
    torch.cuda.synchronize()
    act = host(g["act"])
    assert ulp_diff_f32(act, d["act"]).max() <= 1, f"{label}: activation"
    same = (act == d["act"]).all(axis=1)
    qa, sa = host(g["qa"]), host(g["sa"])
    np.testing.assert_array_equal(qa[same], d["qa"][same])
    np.testing.assert_array_equal(sa[same], d["sa"][same])
    assert np.abs(qa.astype(np.int32) - d["qa"]).max() <= 1
    flips = int((qa != d["qa"]).sum())
    assert flips <= max(2, qa.size // 1000), f"{label}: {flips} requant flips"
    yh = bf16_host(y)
    mism = assert_bf16_close(yh, y_ref, label)
    rows = (qa == d["qa"]).all(axis=1) & (sa == d["sa"])
    np.testing.assert_array_equal(yh[rows], y_ref[rows])
    say(f"{label}: rows with equal act {same.mean():.4f}, requant flips {flips}, "
        f"bf16 mismatches {mism} of {y_ref.size}")
    return y


@pytest.mark.parametrize("M", [1, 2, 3, 16, 17, 100, 300])
def test_mlp_small(orc, M):
    K, I, N = 512, 192, 128
    key = (95, M)
    W = _weights(orc, key, K, I, N)
    x = synth.activations(key, M, K, 4, 20.0)
    if M >= 2:
        x[M - 1] = 0  # an all-zero token
    y = _check(orc, x, W, _dev_weights(W), f"mlp small M={M}")
    if M >= 2:
        assert not bf16_host(y)[M - 1].any()


def test_mlp_single_zero_token(orc):
    # one token: the requant runs inside the down GEMM's launch; an all-zero
    # token has a zero activation row (scale 0, codes 0) and a zero output
    K, I, N = 512, 192, 128
    W = _weights(orc, (95, 99), K, I, N)
    x = np.zeros((1, K), np.uint16)
    y = _check(orc, x, W, _dev_weights(W), "mlp zero token M=1")
    assert not bf16_host(y).any()


def test_mlp_strided_and_ragged(orc):
    M, K, I, N = 37, 640, 320, 96
    key = (96, 1)
    W = _weights(orc, key, K, I, N)
    x = synth.activations(key, M, K, 4, 20.0)
    big = np.zeros((M, K + 64), np.uint16)
    big[:, :K] = x
    _check(orc, x, W, _dev_weights(W), "mlp strided", x_d=bf16_dev(big)[:, :K])


@pytest.fixture(scope="module")
def full_weights(orc):
    K, N = synth.DECODE_SHAPES[0][0], synth.DECODE_SHAPES[1][1]
    I = synth.DECODE_SHAPES[1][0]
    say(f"generating MLP weights K={K} I={I} N={N}")
    W = _weights(orc, (97, 0), K, I, N)
    return W, _dev_weights(W)


@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_mlp_decode_full_size(orc, full_weights, M):
    W, Wd = full_weights
    K = W[0].shape[1]
    x = synth.activations((97, M), M, K, int(round(0.01 * K)), 10.0)
    _check(orc, x, W, Wd, f"mlp decode M={M}")


def test_mlp_prefill_full_size(orc, full_weights):
    W, Wd = full_weights
    M, K = 4096, W[0].shape[1]
    say("mlp prefill M=4096 (oracle takes a while)")
    x = synth.activations((97, M), M, K, 4, 20.0)
    _check(orc, x, W, Wd, "mlp prefill M=4096")
