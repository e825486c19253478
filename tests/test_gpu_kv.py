"""GPU parity of the int8 KV-cache quantisation (f16 scale per token and head)
through the C ABI: codes and f16 scale bits bit-exact against the oracle,
including rows whose scale is an f16 subnormal, rounds to zero or sits next to
the f16 overflow, the cache-slot mapping (skipped and out-of-range slots leave
the cache untouched) and strided token rows.
"""
import numpy as np
import pytest
import torch

import moe_quant_token_amd as mq
import synth
from tests._util import DEV, bf16_dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mq.lib()


def _x(T, Hk, D, seed):
    x = synth.activations((100, seed), T, Hk * D, max(1, Hk * D // 100), 10.0).reshape(T, Hk, D)
    return np.ascontiguousarray(x)


# D in {64, 128, 256} with at least 256 rows takes several rows a wave (ragged
# last wave), everything else one row a wave
@pytest.mark.parametrize("T,Hk,D", [(1, 4, 256), (8, 4, 256), (4096, 4, 256), (37, 8, 128),
                                    (9, 5, 64), (61, 5, 64), (5, 2, 4096), (3, 1, 8),
                                    (70, 3, 520)])
def test_kv_quant_bit_exact(orc, T, Hk, D):
    say(f"kv quant T={T} Hk={Hk} D={D}")
    x = _x(T, Hk, D, T * 1000 + D)
    if T > 2:
        x[1, 0] = 0
        r = np.random.default_rng(T)
        f = r.standard_normal((3, D)).astype(np.float32)
        x[2, 0] = synth.to_bf16_bits(f[0] * np.float32(1e-6))   # subnormal f16 scale
        x[0, Hk - 1] = synth.to_bf16_bits(f[1] * np.float32(1e-10))  # scale rounds to 0
        x[T - 1, 0] = synth.to_bf16_bits(f[2] / np.abs(f[2]).max() * np.float32(8.0e6))
    q_ref, s_ref = orc.kv_quant_i8(x)
    q, s = mq.kv_quant_i8(bf16_dev(x.reshape(T, Hk * D)).reshape(T, Hk, D))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(s).view(np.uint16), s_ref)
    np.testing.assert_array_equal(host(q), q_ref)


@pytest.mark.parametrize("T", [11, 100])
def test_kv_quant_slots_and_stride(orc, T):
    Hk, D, rows = 4, 256, T + 9
    x = _x(T, Hk, D, 7)
    r = np.random.default_rng(T)
    slots = r.permutation(rows + 6)[:T].astype(np.int32) - 3  # some negative, some past the end
    ok = (slots >= 0) & (slots < rows)
    q_ref, s_ref = orc.kv_quant_i8(x[ok], slots[ok], rows=rows)
    big = np.zeros((T, Hk * D + 64), np.uint16)
    big[:, :Hk * D] = x.reshape(T, Hk * D)
    xd = bf16_dev(big)[:, :Hk * D].unflatten(1, (Hk, D))
    q = torch.full((rows, Hk, D), 55, dtype=torch.int8, device=DEV)
    s = torch.full((rows, Hk), 3.0, dtype=torch.float16, device=DEV)
    mq.kv_quant_i8(xd, q, s, slots=torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    qh, sh = host(q), host(s).view(np.uint16)
    written = sorted(int(v) for v in slots[ok])
    np.testing.assert_array_equal(qh[written], q_ref[written])
    np.testing.assert_array_equal(sh[written], s_ref[written])
    rest = sorted(set(range(rows)) - set(written))
    assert (qh[rest] == 55).all() and (sh[rest] == np.float16(3.0).view(np.uint16)).all()
