"""Host-side checks of the C ABI (no GPU needed).

The library loads, exports every function include/w8a8.h declares, and
rejects bad arguments with the documented status before touching the device.
Every call below fails validation (or is a zero-size no-op), so no kernel is
launched and the fake pointers are never dereferenced.
"""
import ctypes

import pytest

import moe_quant_token_amd as mq

OK, INVALID, SHAPE, MISALIGNED, WS_SMALL = 0, -1, -2, -3, -4
A = 1 << 20  # a fake 16-byte aligned "device pointer" (never dereferenced)


@pytest.fixture(scope="module")
def L():
    return mq.lib()


def test_exports_every_declared_function(L):
    names = mq.header_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(mq._SIGS), "binding signatures out of sync with the header"


def test_status_strings(L):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert L.w8a8_status_string(code)
    assert L.w8a8_status_string(-99) == b"unknown status"
    assert L.w8a8_version() >= 100


def test_quant_validation(L):
    f = L.quant_per_token_i8
    assert f(None, 0, 4, 64, 64, None, 64, None, None) == INVALID
    assert f(A, 2, 4, 64, 64, A, 64, A, None) == INVALID          # bad dtype
    assert f(A, 0, 4, 64, 32, A, 64, A, None) == INVALID          # ldx < K
    assert f(A, 0, 4, 50, 64, A, 64, A, None) == SHAPE            # K % 16
    assert f(A + 2, 0, 4, 64, 64, A, 64, A, None) == MISALIGNED
    assert f(A, 0, 4, 64, 72, A, 64, A, None) == MISALIGNED       # ldx % 16
    assert f(None, 0, 0, 64, 64, None, 64, None, None) == OK      # M == 0


def test_gemm_validation(L):
    f = L.gemm_w8a8
    assert f(A, A, 4, 100, 128, A, A, 64, 128, A, 64, None, 0, None) == SHAPE   # K % 64
    assert f(A, A, 4, 128, 128, A, A, 40, 128, A, 40, None, 0, None) == SHAPE   # N % 16
    assert f(A, A, 4, 128, 64, A, A, 64, 128, A, 64, None, 0, None) == INVALID  # lda < K
    assert f(A, A, 4, 128, 128, A, A, 64, 128, A, 32, None, 0, None) == INVALID  # ldy < N
    assert f(None, A, 4, 128, 128, A, A, 64, 128, A, 64, None, 0, None) == INVALID
    assert f(A + 4, A, 4, 128, 128, A, A, 64, 128, A, 64, None, 0, None) == MISALIGNED
    assert f(None, None, 0, 128, 128, None, None, 64, 128, None, 64, None, 0, None) == OK
    g = L.gemm_w8a8_i32acc
    assert g(A, 4, 96, 96, A, 64, 96, A, 64, None, 0, None) == SHAPE
    assert g(A, 4, 128, 128, None, 64, 128, A, 64, None, 0, None) == INVALID
    # packed weights, more than 16 rows: the activation codes are repacked
    # into a caller workspace of ceil(M/16)*16*K bytes
    assert L.gemm_w8a8_workspace_bytes(16, 64, 128) == 0
    need = L.gemm_w8a8_workspace_bytes(20, 64, 128)
    assert need >= 32 * 128
    p = L.gemm_w8a8_packed
    assert p(A, A, 20, 128, 128, A, A, 64, A, 64, A, need - 1, None) == WS_SMALL
    assert p(A, A, 20, 128, 128, A, A, 64, A, 64, None, need, None) == INVALID
    assert p(A, A, 20, 128, 128, A, A, 64, A, 64, A + 8, need, None) == MISALIGNED
    q = L.gemm_w8a8_packed_i32acc
    assert q(A, 20, 128, 128, A, 64, A, 64, A, need - 1, None) == WS_SMALL
    assert q(A, 20, 128, 128, A, 64, A, 64, None, need, None) == INVALID


def test_linear_validation(L):
    f = L.linear_w8a8
    need = L.linear_w8a8_workspace_bytes(8, 64, 128)
    assert need >= 8 * 128 + 8 * 4
    assert f(A, 8, 128, 128, A, A, 64, 128, A, 64, A, need - 1, None) == WS_SMALL
    assert f(A, 8, 128, 128, A, A, 64, 128, A, 64, None, need, None) == INVALID
    assert f(A, 8, 128, 128, A, A, 64, 128, A, 64, A + 8, need, None) == MISALIGNED


def test_moe_validation(L):
    f = L.moe_w8a8_forward
    need = L.moe_w8a8_workspace_bytes(4, 128, 8, 64, 2)
    assert need > 0
    args = lambda T=4, H=128, E=8, I=64, k=2, ws=A, wsb=need: (
        A, A, T, H, E, I, k, A, A, A, A, A, A, A, ws, wsb, None, None)
    assert f(*args(k=9)) == SHAPE            # topk > E
    assert f(*args(k=17, E=32)) == SHAPE     # topk > 16
    assert f(*args(H=100)) == SHAPE          # H % 64
    assert f(*args(I=96)) == SHAPE           # I % 64
    assert f(*args(E=2048)) == SHAPE
    assert f(*args(wsb=need - 1)) == WS_SMALL
    assert f(*args(ws=None)) == INVALID
    assert f(*args(T=0)) == OK
    assert f(*args(k=0)) == INVALID


def test_hadamard_validation(L):
    assert L.fwht128_quant(A, 2, 200, 208, A, 208, A, None) == SHAPE
    assert L.fwht128_quant(A, 0, 256, 256, A, 256, A, None) == OK
    assert L.fwht128_weight_prep_g256(A, 4, 384, A, A, A, None) == SHAPE
    assert L.gemm_w8a8_g256(A, A, 2, 384, A, A, A, 64, A, 64, None, 0, None) == SHAPE
    assert L.gemm_w8a8_g256(A, A, 2, 512, A, A, A, 40, A, 40, None, 0, None) == SHAPE


def test_stream_read_validation(L):
    f = L.w8a8_stream_read
    assert f(A, 1 << 20, 1000, A, None) == INVALID        # chunk not a multiple of 1 KiB
    assert f(A, (1 << 20) + 1024, 1 << 12, A, None) == INVALID  # bytes not whole chunks
    assert f(A, 0, 1024, A, None) == INVALID
    assert f(None, 1 << 20, 1024, A, None) == INVALID
    assert f(A, 1 << 20, 1024, None, None) == INVALID
    assert f(A + 8, 1 << 20, 1024, A, None) == MISALIGNED


def test_rot_layer_shared_validation(L):
    f = L.moe_w8a8_rot_shared_forward_packed
    ws = L.moe_w8a8_rot_shared_workspace_bytes(1, 256, 8, 128, 2, 128)
    assert ws > L.moe_w8a8_workspace_bytes(1, 256, 8, 128, 2)
    assert L.moe_w8a8_rot_shared_workspace_bytes(1, 256, 8, 128, 2, 0) == 0
    args = lambda **kw: dict(dict(x=A, lg=A, T=1, H=256, E=8, I=128, k=2, Is=128, wsb=ws,
                                  ws=A, su8=A), **kw)
    def call(a):
        return f(a["x"], a["lg"], a["T"], a["H"], a["E"], a["I"], a["k"], A, A, A, A, a["Is"], A,
                 a["su8"], A, A, A, A, A, A, a["ws"], a["wsb"], None, None)
    assert call(args(Is=0)) == INVALID
    assert call(args(Is=100)) == SHAPE            # Is % 128
    assert call(args(Is=4096)) == SHAPE           # Is > 2048
    assert call(args(H=128)) == SHAPE             # H % 256
    assert call(args(su8=None)) == INVALID
    assert call(args(x=A + 2)) == MISALIGNED
    assert call(args(wsb=ws - 1)) == WS_SMALL
    assert call(args(T=0, x=None)) == OK

