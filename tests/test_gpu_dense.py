"""GPU parity of the dense path through the C ABI: per-token quant, the int8
GEMM (decode weight-streaming kernel and LDS-tiled kernel) and the whole
online W8A8 linear, against the CPU oracle on identical seeded inputs.

Bar: int8 codes, fp32 scales and int32 sums bit-exact; bf16 outputs within
1e-3 abs + 1e-2 rel (and, since the GPU evaluates the same fp32 epilogue
operations, expected bit-exact: mismatches are counted and must be zero).
"""
import numpy as np
import pytest
import torch

import moe_quant_token_amd as mq
import synth
from tests._util import (DEV, assert_bf16_close, bf16_dev, bf16_host, dev, host, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mq.lib()


def _inputs(xkey, wkey, M, K, N, n_out, scale):
    x = synth.activations(xkey, M, K, n_out, scale)
    W = synth.weights(wkey, N, K)
    return x, W


# ---------------------------------------------------------------- quant
@pytest.mark.parametrize("M,K", [(16, 512), (1, 5120), (8, 8704), (4096, 5120), (37, 16),
                                 (5, 48), (3, 65536),
                                 # more than 16 rows: one wave per row, every
                                 # register depth (2, 4, 8, 10, 12, 16 chunks)
                                 (17, 1008), (101, 1040), (66, 4096), (35, 5104),
                                 (33, 6000), (20, 8192), (19, 8208)])
def test_quant_bf16_bit_exact(orc, M, K):
    say(f"quant bf16 M={M} K={K}")
    x = synth.activations((7, M, K), M, K, max(1, K // 100), 10.0)
    if M > 2:
        x[1] = 0  # an all-zero row
    q_ref, s_ref = orc.quant_rows(x)
    q, s = mq.quant_per_token_i8(bf16_dev(x))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(q), q_ref)
    np.testing.assert_array_equal(host(s), s_ref)


@pytest.mark.parametrize("N,K", [(256, 512), (17408, 5120), (5120, 8704)])
def test_quant_fp32_weights_bit_exact(orc, N, K):
    say(f"quant fp32 weights N={N} K={K}")
    W = synth.weights((8, N), N, K)
    q_ref, s_ref = orc.quant_rows(W)
    q, s = mq.quant_per_token_i8(dev(W))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(q), q_ref)
    np.testing.assert_array_equal(host(s), s_ref)


def test_quant_tiny_and_huge_rows(orc):
    # rows whose scale falls below 2^-100 (the kernels divide instead of
    # multiplying by the reciprocal), rows at the bf16 extremes, a zero row
    M, K = 24, 320
    x = synth.activations((7, 2), M, K, 3, 10.0).view(np.uint16).copy()
    r = np.random.default_rng(3)
    f = r.standard_normal((3, K)).astype(np.float32)
    x[0] = synth.to_bf16_bits(f[0] * np.float32(1e-35))
    x[1] = synth.to_bf16_bits(f[1] * np.float32(2e-38))
    x[2] = synth.to_bf16_bits(f[2] * np.float32(1e37))
    x[3] = 0
    q_ref, s_ref = orc.quant_rows(x)
    for rows in (M, 8):  # the wave-per-row and the block-per-row kernels
        q, s = mq.quant_per_token_i8(bf16_dev(x[:rows]))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(q), q_ref[:rows])
        np.testing.assert_array_equal(host(s), s_ref[:rows])


def test_quant_strided_rows(orc):
    x = synth.activations((7, 1), 6, 256, 3, 10.0)
    big = np.zeros((6, 384), np.uint16)
    big[:, :256] = x
    xd = bf16_dev(big)[:, :256]
    qbuf = torch.zeros((6, 320), dtype=torch.int8, device=DEV)
    q, s = mq.quant_per_token_i8(xd, q=qbuf[:, :256])
    q_ref, s_ref = orc.quant_rows(x)
    np.testing.assert_array_equal(host(qbuf)[:, :256], q_ref)
    assert not host(qbuf)[:, 256:].any()
    np.testing.assert_array_equal(host(s), s_ref)


# ---------------------------------------------------------------- GEMM
GEMM_SHAPES = [
    (16, 512, 256),     # the small single-linear workload (decode kernel)
    (1, 64, 16),        # smallest legal shape
    (3, 640, 48),
    (17, 512, 64),      # first M served by the tiled kernel
    (300, 640, 272),    # ragged M; packed: 128x64 tiles, two chunks a step
    (64, 1024, 1024),   # packed: 64x64 tiles, two chunks a step
    (160, 4096, 272),   # packed: 128x128 tiles, ragged M and last column tile
    (40, 576, 96),      # K % 128 != 0: 64x64 tiles, one chunk a step
    (2048, 512, 2048),  # 256x256 tiles
    (2100, 256, 2064),  # 256x256 tiles, ragged M and N
    (4096, 64, 4352),   # 256x256 tiles over whole rounds, remaining columns 128x64
    (4000, 128, 4368),  # the same split with ragged M and a ragged last column tile
]


def _packed_ref(qw):
    """The packed tile layout by array reshaping (marshalling only)."""
    N, K = qw.shape
    return np.ascontiguousarray(qw.reshape(N // 16, 16, K // 64, 4, 16)
                                .transpose(0, 2, 3, 1, 4)).reshape(-1)


@pytest.mark.parametrize("N,K", [(16, 64), (48, 640), (17408, 5120)])
def test_pack_weights_layout(N, K):
    r = np.random.default_rng(N)
    qw = r.integers(-127, 128, (N, K)).astype(np.int8)
    big = torch.zeros((N, K + 64), dtype=torch.int8, device=DEV)
    big[:, :K] = dev(qw)
    packed = mq.pack_weights(big[:, :K])
    np.testing.assert_array_equal(host(packed), _packed_ref(qw))


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("M,K,N", GEMM_SHAPES)
def test_gemm_i32_and_bf16(orc, M, K, N, packed):
    say(f"gemm M={M} K={K} N={N} packed={packed}")
    x, W = _inputs((9, M), (9, N), M, K, N, 4, 20.0)
    qa, sa = orc.quant_rows(x)
    qw, sw = orc.quant_rows(W)
    acc_ref = orc.gemm_i32(qa, qw)
    y_ref = orc.gemm_w8a8(qa, sa, qw, sw)
    qa_d, sa_d, qw_d, sw_d = dev(qa), dev(sa), dev(qw), dev(sw)
    if packed:
        qp = mq.pack_weights(qw_d)
        acc = mq.gemm_w8a8_packed_i32acc(qa_d, qp, N)
        y = mq.gemm_w8a8_packed(qa_d, sa_d, qp, sw_d, N)
        y2 = mq.linear_w8a8_packed(bf16_dev(x), qp, sw_d, N)
    else:
        acc = mq.gemm_w8a8_i32acc(qa_d, qw_d)
        y = mq.gemm_w8a8(qa_d, sa_d, qw_d, sw_d)
        y2 = mq.linear_w8a8(bf16_dev(x), qw_d, sw_d)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(acc), acc_ref)
    mism = assert_bf16_close(bf16_host(y), y_ref, "gemm_w8a8")
    assert mism == 0
    np.testing.assert_array_equal(bf16_host(y2), y_ref)


@pytest.mark.parametrize("packed", [False, True])
def test_linear_decode_zero_row_and_stride(orc, packed):
    # the fused decode linear: an all-zero token, a strided activation matrix
    M, K, N = 5, 640, 48
    x, W = _inputs((10, M), (10, N), M, K, N, 4, 20.0)
    x[2] = 0
    qw, sw = orc.quant_rows(W)
    y_ref = orc.linear_w8a8(x, qw, sw)
    big = np.zeros((M, K + 64), np.uint16)
    big[:, :K] = x
    xd = bf16_dev(big)[:, :K]
    qw_d, sw_d = dev(qw), dev(sw)
    if packed:
        y = mq.linear_w8a8_packed(xd, mq.pack_weights(qw_d), sw_d, N)
    else:
        y = mq.linear_w8a8(xd, qw_d, sw_d)
    torch.cuda.synchronize()
    got = bf16_host(y)
    np.testing.assert_array_equal(got, y_ref)
    assert not got[2].any()


@pytest.mark.parametrize("M", [1, 2])
@pytest.mark.parametrize("K,N", [(64, 16), (16384, 32), (640, 8192), (640, 8208)])
def test_linear_one_or_two_tokens(orc, M, K, N):
    # one or two tokens with packed weights: the quantisation runs inside the
    # GEMM launch while the output has at most two 16-channel tiles per CU
    # (N = 8192 on 256 CUs), the two-launch path beyond (N = 8208); strided
    # rows, and an all-zero second token
    say(f"linear one/two tokens M={M} K={K} N={N}")
    x, W = _inputs((11, M, K), (11, N, K), M, K, N, 2, 20.0)
    if M == 2:
        x[1] = 0
    qw, sw = orc.quant_rows(W)
    y_ref = orc.linear_w8a8(x, qw, sw)
    big = np.zeros((M, K + 32), np.uint16)
    big[:, :K] = x
    y = mq.linear_w8a8_packed(bf16_dev(big)[:, :K], mq.pack_weights(dev(qw)), dev(sw), N)
    torch.cuda.synchronize()
    got = bf16_host(y)
    np.testing.assert_array_equal(got, y_ref)
    if M == 2:
        assert not got[1].any()


def test_gemm_extreme_codes_no_overflow():
    # every code +-127 at the largest decode K: |acc| = 127*127*8704
    K, N = 8704, 32
    qa = torch.full((4, K), 127, dtype=torch.int8, device=DEV)
    qa[1] = -127
    qw = torch.full((N, K), 127, dtype=torch.int8, device=DEV)
    qw[1::2, ::2] = -127
    acc = host(mq.gemm_w8a8_i32acc(qa, qw))
    big = 127 * 127 * K
    assert (acc[0, 0::2] == big).all() and (acc[1, 0::2] == -big).all()
    assert (acc[:, 1::2] == 0).all()
    acc2 = host(mq.gemm_w8a8_i32acc(torch.cat([qa] * 8), qw))  # tiled kernel (M = 32)
    np.testing.assert_array_equal(acc2[:4], acc)


@pytest.mark.parametrize("packed", [False, True])
def test_gemm_largest_k_extreme_codes(packed):
    # K = 131072 is the largest K accepted: 127^2 * K = 2,114,060,288 < 2^31
    K, N = 131072, 16
    qa = torch.full((2, K), 127, dtype=torch.int8, device=DEV)
    qa[1] = -127
    qw = torch.full((N, K), 127, dtype=torch.int8, device=DEV)
    qw[1::2] = -127
    big = 127 * 127 * K
    expect = np.array([[big, -big] * (N // 2), [-big, big] * (N // 2)], np.int64)
    if packed:
        qp = mq.pack_weights(qw)
        acc = host(mq.gemm_w8a8_packed_i32acc(qa, qp, N))
        acc17 = host(mq.gemm_w8a8_packed_i32acc(torch.cat([qa] * 9)[:17], qp, N))
    else:
        acc = host(mq.gemm_w8a8_i32acc(qa, qw))
        acc17 = host(mq.gemm_w8a8_i32acc(torch.cat([qa] * 9)[:17], qw))  # tiled kernel
    np.testing.assert_array_equal(acc, expect)
    np.testing.assert_array_equal(acc17[:2], expect)
    np.testing.assert_array_equal(acc17[16], expect[0])


def test_gemm_strided_output_and_inputs(orc):
    M, K, N = 5, 256, 64
    x, W = _inputs((10, 1), (10, 2), M, K, N, 2, 20.0)
    qa, sa = orc.quant_rows(x)
    qw, sw = orc.quant_rows(W)
    y_ref = orc.gemm_w8a8(qa, sa, qw, sw)
    qa_big = torch.zeros((M, K + 64), dtype=torch.int8, device=DEV)
    qa_big[:, :K] = dev(qa)
    ybuf = torch.zeros((M, N + 16), dtype=torch.bfloat16, device=DEV)
    mq.gemm_w8a8(qa_big[:, :K], dev(sa), dev(qw), dev(sw), y=ybuf[:, :N])
    got = bf16_host(ybuf)
    np.testing.assert_array_equal(got[:, :N], y_ref)
    assert not got[:, N:].any()


# ------------------------------------------------------ decode, full size
@pytest.mark.parametrize("shape_idx", [0, 1])
def test_decode_linear_full(orc, shape_idx):
    for M in synth.DECODE_M + [16]:
        cfg = synth.decode_linear(M, shape_idx)
        say(f"decode linear {cfg['name']} M={M} K={cfg['K']} N={cfg['N']}")
        if M == 1:
            W = synth.weights(cfg["wkey"], cfg["N"], cfg["K"])
            qw, sw = orc.quant_rows(W)
            del W
            qw_d, sw_d = dev(qw), dev(sw)
            qp_d = mq.pack_weights(qw_d)
        x = synth.activations(cfg["xkey"], M, cfg["K"], cfg["n_outliers"], cfg["outlier_scale"])
        y_ref = orc.linear_w8a8(x, qw, sw)
        y = mq.linear_w8a8(bf16_dev(x), qw_d, sw_d)
        yp = mq.linear_w8a8_packed(bf16_dev(x), qp_d, sw_d, cfg["N"])
        torch.cuda.synchronize()
        assert assert_bf16_close(bf16_host(y), y_ref, "linear_w8a8") == 0
        assert assert_bf16_close(bf16_host(yp), y_ref, "linear_w8a8_packed") == 0


def test_quant_rows_read_twice(orc):
    # rows too long to hold in registers are read a second time for the codes:
    # bf16 with more than 16 rows and K > 16384 (256-thread kernel), fp32 rows
    # with K > 16384
    xb = synth.activations((7, 30), 20, 16448, 160, 10.0)
    xb[3] = 0
    q_ref, s_ref = orc.quant_rows(xb)
    q, s = mq.quant_per_token_i8(bf16_dev(xb))
    Wf = synth.weights((8, 31), 3, 20000)
    qf_ref, sf_ref = orc.quant_rows(Wf)
    qf, sf = mq.quant_per_token_i8(dev(Wf))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(q), q_ref)
    np.testing.assert_array_equal(host(s), s_ref)
    np.testing.assert_array_equal(host(qf), qf_ref)
    np.testing.assert_array_equal(host(sf), sf_ref)


@pytest.mark.parametrize("M,K", [(40, 8704), (20, 16448)])
def test_packed_linear_long_rows(orc, M, K):
    # packed linear with more than 16 rows and K > 8192: the 256-thread
    # quantiser writes the tile layout (rows held, then read twice)
    say(f"packed linear long rows M={M} K={K}")
    N = 64
    x, W = _inputs((12, M, K), (12, K), M, K, N, max(1, K // 100), 10.0)
    x[1] = 0
    qw, sw = orc.quant_rows(W)
    y_ref = orc.linear_w8a8(x, qw, sw)
    y = mq.linear_w8a8_packed(bf16_dev(x), mq.pack_weights(dev(qw)), dev(sw), N)
    np.testing.assert_array_equal(bf16_host(y), y_ref)


def test_tile_gemm_global_load_feed(orc):
    # an activation row stride so large that a workgroup's operand range
    # spans more than 2 GiB: the tiled kernel feeds LDS with global loads
    # instead of buffer loads (row-major operands only)
    M, K, N = 17, 128, 64
    lda = 35 << 20
    assert 63 * lda + K >= 1 << 31
    r = np.random.default_rng(17)
    qa = r.integers(-127, 128, (M, K)).astype(np.int8)
    sa = (r.random(M) * 0.01).astype(np.float32)
    qw = r.integers(-127, 128, (N, K)).astype(np.int8)
    sw = (r.random(N) * 0.01).astype(np.float32)
    big = torch.zeros((M, lda), dtype=torch.int8, device=DEV)
    big[:, :K] = dev(qa)
    qa_d = big[:, :K]
    acc = mq.gemm_w8a8_i32acc(qa_d, dev(qw))
    y = mq.gemm_w8a8(qa_d, dev(sa), dev(qw), dev(sw))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(acc), orc.gemm_i32(qa, qw))
    np.testing.assert_array_equal(bf16_host(y), orc.gemm_w8a8(qa, sa, qw, sw))
    del big


@pytest.mark.parametrize("packed", [False, True])
def test_tile_256x160_plan_full(orc, packed):
    # 4 x 5 = 20 tiles of 256 x 256 would leave most of a round idle and N is
    # a multiple of 160: the 256 x 160 plan (two workgroups a CU), compared in
    # full
    M, K, N = 1024, 512, 1280
    x, W = _inputs((13, 1), (13, 2), M, K, N, 4, 20.0)
    x[7] = 0
    qa, sa = orc.quant_rows(x)
    qw, sw = orc.quant_rows(W)
    acc_ref = orc.gemm_i32(qa, qw)
    y_ref = orc.epilogue(acc_ref, sa, sw)
    qw_d = mq.pack_weights(dev(qw)) if packed else dev(qw)
    if packed:
        acc = mq.gemm_w8a8_packed_i32acc(dev(qa), qw_d, N)
        y = mq.gemm_w8a8_packed(dev(qa), dev(sa), qw_d, dev(sw), N)
        y2 = mq.linear_w8a8_packed(bf16_dev(x), qw_d, dev(sw), N)
    else:
        acc = mq.gemm_w8a8_i32acc(dev(qa), qw_d)
        y = mq.gemm_w8a8(dev(qa), dev(sa), qw_d, dev(sw))
        y2 = mq.linear_w8a8(bf16_dev(x), qw_d, dev(sw))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(acc), acc_ref)
    np.testing.assert_array_equal(bf16_host(y), y_ref)
    np.testing.assert_array_equal(bf16_host(y2), y_ref)


# ----------------------------------------------------- prefill, full size
@pytest.mark.parametrize("N", [5120, 17408])
def test_prefill_full(orc, N):
    # every output of the prefill workload against the oracle: the int32 sums
    # of the packed GEMM, the GEMM-only call, the linear entry the benchmark
    # times (its quantiser writes the tile layout) and the linear on
    # row-major weights
    cfg = synth.prefill_linear(N)
    M, K = cfg["M"], cfg["K"]
    say(f"prefill full M={M} K={K} N={N}")
    x, W = _inputs(cfg["xkey"], cfg["wkey"], M, K, N, cfg["n_outliers"], cfg["outlier_scale"])
    qa, sa = orc.quant_rows(x)
    qw, sw = orc.quant_rows(W)
    del W
    x_d, qw_d, sw_d = bf16_dev(x), dev(qw), dev(sw)
    q_d, s_d = mq.quant_per_token_i8(x_d)
    qp_d = mq.pack_weights(qw_d)
    acc = host(mq.gemm_w8a8_packed_i32acc(q_d, qp_d, N))
    y = bf16_host(mq.gemm_w8a8_packed(q_d, s_d, qp_d, sw_d, N))
    yl = bf16_host(mq.linear_w8a8_packed(x_d, qp_d, sw_d, N))
    yu = bf16_host(mq.linear_w8a8(x_d, qw_d, sw_d))  # row-major weights
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(q_d), qa)
    np.testing.assert_array_equal(host(s_d), sa)
    say("  oracle GEMM")
    acc_ref = orc.gemm_i32(qa, qw)
    np.testing.assert_array_equal(acc, acc_ref)
    y_ref = orc.epilogue(acc_ref, sa, sw)
    np.testing.assert_array_equal(y, y_ref)
    np.testing.assert_array_equal(yl, y_ref)
    np.testing.assert_array_equal(yu, y_ref)
