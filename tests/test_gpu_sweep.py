"""GPU parity over seeded random shapes, through the C ABI.

Every entry point picks its kernels from the shape (decode or tiled GEMM, the
one-launch decode linear for one or two tokens on few tiles a CU, the
one-launch Hadamard linear for one token, the four MoE batch paths), so a
sweep of odd sizes reaches the dispatch edges the fixed-size tests do not.
Dense and Hadamard outputs are compared bit-exactly with the oracle; the MoE
layer as in test_gpu_moe (ids exact, int32 sums exact, bf16 output within
1e-3 abs + 1e-2 rel).
"""
import numpy as np
import pytest
import torch

import moe_quant_token_amd as mq
import synth
from tests._util import bf16_dev, bf16_host, dev, say
from tests.test_gpu_moe import _check_full, _tie_free, _weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mq.lib()


def test_sweep_dense_linear(orc):
    r = np.random.default_rng(71)
    for i in range(36):
        M = int(r.choice([1, 1, 2, 2, 3, 5, 8, 13, 16, 17, 24, 32, 33, 70, 100, 130, 200]))
        K = 64 * int(r.integers(1, 41))
        N = 16 * int(r.integers(1, 49))
        packed = bool(r.integers(0, 2))
        say(f"sweep linear {i}: M={M} K={K} N={N} packed={packed}")
        x = synth.activations((60, i), M, K, 2, 20.0)
        if M > 1 and r.integers(0, 3) == 0:
            x[int(r.integers(0, M))] = 0
        qw, sw = orc.quant_rows(synth.weights((61, i), N, K))
        y_ref = orc.linear_w8a8(x, qw, sw)
        if packed:
            qp = mq.pack_weights(dev(qw))
            y = mq.linear_w8a8_packed(bf16_dev(x), qp, dev(sw), N)
            # the GEMM alone on codes with a row stride past K
            qa, sa = orc.quant_rows(x)
            wide = torch.zeros((M, K + 48), dtype=torch.int8, device="cuda")
            wide[:, :K] = dev(qa)
            y_g = mq.gemm_w8a8_packed(wide[:, :K], dev(sa), qp, dev(sw), N)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(bf16_host(y_g), y_ref, err_msg=f"case {i} gemm")
        else:
            y = mq.linear_w8a8(bf16_dev(x), dev(qw), dev(sw))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bf16_host(y), y_ref, err_msg=f"case {i}")


def test_sweep_hadamard_linear(orc):
    r = np.random.default_rng(72)
    for i in range(16):
        M = int(r.choice([1, 1, 1, 2, 5, 16, 17, 40]))
        K = 256 * int(r.integers(1, 9))
        N = 16 * int(r.integers(1, 21))
        say(f"sweep g256 linear {i}: M={M} K={K} N={N}")
        qw, su8, s2 = orc.weight_prep_g256(synth.weights((62, i), N, K))
        x = synth.activations((63, i), M, K, max(1, K // 100), 10.0, heavy_tail=True)
        qa, sa = orc.fwht128_quant(x)
        y = mq.linear_w8a8_g256_packed(bf16_dev(x), mq.pack_weights(dev(qw)), dev(su8),
                                       dev(s2.view(np.int16)).view(torch.bfloat16))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bf16_host(y), orc.gemm_g256(qa, sa, qw, su8, s2),
                                      err_msg=f"case {i}")


# (T, E, k, H, I): one token, the one-workgroup prep (<= 16 tokens), the
# route/sort/skinny path (<= 2048 pairs) and the large-batch path beyond
_MOE_CASES = [(1, 8, 2, 128, 64), (1, 64, 8, 320, 192), (3, 16, 4, 192, 128),
              (16, 64, 8, 128, 64), (17, 8, 1, 256, 128), (40, 16, 2, 64, 320),
              (300, 16, 8, 128, 128), (520, 64, 4, 192, 64)]


@pytest.mark.parametrize("case", range(len(_MOE_CASES)))
def test_sweep_moe(orc, case):
    T, E, k, H, I = _MOE_CASES[case]
    packed = case % 2 == 1
    say(f"sweep moe {case}: T={T} E={E} k={k} H={H} I={I} packed={packed}")
    W = _weights(orc, (64, case), E, H, I)
    x = synth.activations((65, case), T, H, 0, 1.0)
    logits = synth.router_logits((66, case), T, E)
    assert _tie_free(logits, k)
    _check_full(orc, x, logits, k, W, T, f"sweep moe {case}", packed=packed)
