"""linear_w8a8_packed_noalloc (the library's static scratch instead of a
caller workspace) against linear_w8a8_packed, through the C ABI.

Two calls in a row, the second with a smaller input, so the second runs on
scratch that still holds the first call's codes; both must equal the
workspace entry point bit for bit (and, at the small sizes, the oracle).
Covers the paths that use the scratch (tile-layout codes for M > 16, row-major
codes for 3..16 tokens) and the one-launch path for one or two tokens.
"""
import numpy as np
import pytest
import torch

import moe_quant_token_amd as mq
import synth
from tests._util import bf16_dev, bf16_host, dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mq.lib()


def _weights(orc, K, N, seed):
    qw, sw = orc.quant_rows(synth.weights((80, seed), N, K))
    return qw, sw, mq.pack_weights(dev(qw)), dev(sw)


@pytest.mark.parametrize("K,N,Ms", [(5120, 5120, (4096, 300)), (8704, 5120, (64, 8)),
                                    (5120, 17408, (8, 2)), (1024, 1280, (17, 1))])
def test_noalloc_matches_workspace_call(orc, K, N, Ms):
    qw, sw, qp, sw_d = _weights(orc, K, N, K + N)
    for i, M in enumerate(Ms):
        say(f"noalloc K={K} N={N} call {i} M={M}")
        x = synth.activations((81, K, M), M, K, max(1, K // 100), 10.0)
        x_d = bf16_dev(x)
        y_ws = mq.linear_w8a8_packed(x_d, qp, sw_d, N)
        y_na = mq.linear_w8a8_packed_noalloc(x_d, qp, sw_d, N)
        torch.cuda.synchronize()
        assert torch.equal(y_ws.view(torch.int16), y_na.view(torch.int16)), \
            f"M={M}: the scratch call differs from the workspace call"
        if M <= 300:
            np.testing.assert_array_equal(bf16_host(y_na), orc.linear_w8a8(x, qw, sw))


def test_noalloc_rejects_beyond_scratch():
    # 4096 tokens at K = 8704 need 35.7 MB of codes: more than the scratch
    M, K, N = 4096, 8704, 64
    need = mq.linear_w8a8_workspace_bytes(M, N, K)
    assert need > mq.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    qp = torch.zeros((N * K,), dtype=torch.int8, device="cuda")
    sw = torch.ones((N,), dtype=torch.float32, device="cuda")
    y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mq.W8A8Error) as ei:
        mq.linear_w8a8_packed_noalloc(x, qp, sw, N, y=y)
    assert ei.value.status == -2
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()), "a rejected call wrote its output"
