"""HIP-graph capture of every entry point, through the C ABI.

The calls enqueue on the caller's stream and never allocate, synchronise or
read device memory on the host, so each can be captured into a graph (the
decode mode of the ATOM pull request's "Performance" section; its "Changes",
linear.py bullet calls the W8A8 GEMM op graph-safe).  Each case captures the
call with preallocated buffers, then replays the graph several times with new
inputs copied into the captured input buffers and eager work in between;
every replay must equal the eager call on the same input bit for bit, and the
eager call must equal the oracle.
"""
import numpy as np
import pytest
import torch

import moe_quant_token_amd as mq
import synth
from tests._util import bf16_dev, bf16_host, dev, host, say

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mq.lib()


def _bits(t):
    return t.contiguous().view(torch.uint8).clone()


def _graph_check(call, static_inputs, input_sets, outputs, oracle_check=None):
    """call(): the entry point on the static buffers; input_sets: a list of
    tuples of host-side tensors to copy into static_inputs before each run."""
    for dst, src in zip(static_inputs, input_sets[0]):
        dst.copy_(src)
    call()  # eager warm-up (device checks are cached before capture)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        for inputs in input_sets:
            for dst, src in zip(static_inputs, inputs):
                dst.copy_(src)
            g.replay()
            torch.cuda.synchronize()
            got = [_bits(o) for o in outputs]
            # eager work between replays, then the eager call on the same input
            for o in outputs:
                o.zero_()
            call()
            torch.cuda.synchronize()
            for a, o in zip(got, outputs):
                assert torch.equal(a, _bits(o)), f"replay {rep} differs from the eager call"
            if oracle_check is not None and rep == 0:
                oracle_check(inputs)


def _dense(orc, M, K, N, seed):
    x = [synth.activations((70, seed, i), M, K, max(1, K // 100), 10.0) for i in range(2)]
    W = synth.weights((70, seed), N, K)
    qw, sw = orc.quant_rows(W)
    return x, qw, sw


@pytest.mark.parametrize("M", [1, 2, 8, 300, 4096])
def test_linear_packed_graph(orc, M):
    K, N = (5120, 17408) if M in (1, 8) else (8704, 5120) if M == 2 else (1024, 1280)
    if M == 4096:
        K, N = 5120, 5120
    say(f"graph linear_w8a8_packed M={M} K={K} N={N}")
    xs, qw, sw = _dense(orc, M, K, N, M)
    qp, sw_d = mq.pack_weights(dev(qw)), dev(sw)
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mq.linear_w8a8_workspace_bytes(M, N, K), dtype=torch.uint8, device="cuda")
    sets = [(bf16_dev(v),) for v in xs]

    def check(inp):
        xh = bf16_host(inp[0])
        ms = np.arange(M) if M <= 300 else np.arange(0, M, 97)
        want = orc.linear_w8a8(np.ascontiguousarray(xh[ms]), qw, sw)
        np.testing.assert_array_equal(bf16_host(y)[ms], want)

    _graph_check(lambda: mq.linear_w8a8_packed(x, qp, sw_d, N, y=y, ws=ws), [x], sets, [y], check)


@pytest.mark.parametrize("M", [8, 300])
def test_gemm_graph(orc, M):
    K, N = 1024, 1280
    xs, qw, sw = _dense(orc, M, K, N, 100 + M)
    q_all = [orc.quant_rows(v) for v in xs]
    qw_d, sw_d = dev(qw), dev(sw)
    qp = mq.pack_weights(qw_d)
    qa = torch.empty((M, K), dtype=torch.int8, device="cuda")
    sa = torch.empty((M,), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    yp = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    accp = torch.empty((M, N), dtype=torch.int32, device="cuda")
    ws = torch.empty(max(1, mq.gemm_w8a8_workspace_bytes(M, N, K)), dtype=torch.uint8,
                     device="cuda")
    sets = [(dev(q), dev(s)) for q, s in q_all]

    def call():
        mq.gemm_w8a8(qa, sa, qw_d, sw_d, y=y)
        mq.gemm_w8a8_packed(qa, sa, qp, sw_d, N, y=yp, ws=ws)
        mq.gemm_w8a8_i32acc(qa, qw_d, acc=acc)
        mq.gemm_w8a8_packed_i32acc(qa, qp, N, acc=accp, ws=ws)

    def check(inp):
        q, s = host(inp[0]), host(inp[1])
        acc_ref = orc.gemm_i32(q, qw)
        np.testing.assert_array_equal(host(acc), acc_ref)
        np.testing.assert_array_equal(host(accp), acc_ref)
        y_ref = orc.epilogue(acc_ref, s, sw)
        np.testing.assert_array_equal(bf16_host(y), y_ref)
        np.testing.assert_array_equal(bf16_host(yp), y_ref)

    _graph_check(call, [qa, sa], sets, [y, yp, acc, accp], check)


def test_quant_and_fwht_graph(orc):
    M, K = 37, 2048
    xs = [synth.activations((71, i), M, K, 20, 10.0, heavy_tail=True) for i in range(2)]
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    q = torch.empty((M, K), dtype=torch.int8, device="cuda")
    s = torch.empty((M,), dtype=torch.float32, device="cuda")
    qh = torch.empty((M, K), dtype=torch.int8, device="cuda")
    sh = torch.empty((M,), dtype=torch.float32, device="cuda")

    def call():
        mq.quant_per_token_i8(x, q=q, s=s)
        mq.fwht128_quant(x, q=qh, s=sh)

    def check(inp):
        xh = bf16_host(inp[0])
        qr, sr = orc.quant_rows(xh)
        np.testing.assert_array_equal(host(q), qr)
        np.testing.assert_array_equal(host(s), sr)
        qr, sr = orc.fwht128_quant(xh)
        np.testing.assert_array_equal(host(qh), qr)
        np.testing.assert_array_equal(host(sh), sr)

    _graph_check(call, [x], [(bf16_dev(v),) for v in xs], [q, s, qh, sh], check)


@pytest.mark.parametrize("M", [1, 256])
def test_hadamard_graph(orc, M):
    K, N = 2048, 8192
    qw, su8, s2 = orc.weight_prep_g256(synth.weights((72, 0), N, K))
    qp, su_d, s2_d, qw_d = mq.pack_weights(dev(qw)), dev(su8), dev(s2), dev(qw)
    xs = [synth.activations((72, M, i), M, K, 20, 10.0, heavy_tail=True) for i in range(2)]
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    qa = torch.empty((M, K), dtype=torch.int8, device="cuda")
    sa = torch.empty((M,), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(256, mq.linear_w8a8_g256_workspace_bytes(M, N, K)), dtype=torch.uint8,
                     device="cuda")
    ws2 = torch.empty(max(256, mq.gemm_w8a8_g256_workspace_bytes(M, N, K)), dtype=torch.uint8,
                      device="cuda")

    def call():
        mq.linear_w8a8_g256_packed(x, qp, su_d, s2_d, y=y, ws=ws)
        mq.fwht128_quant(x, q=qa, s=sa)
        mq.gemm_w8a8_g256(qa, sa, qw_d, su_d, s2_d, y=y2, ws=ws2)

    def check(inp):
        qr, sr = orc.fwht128_quant(bf16_host(inp[0]))
        want = orc.gemm_g256(qr, sr, qw, su8, s2)
        np.testing.assert_array_equal(bf16_host(y), want)
        np.testing.assert_array_equal(bf16_host(y2), want)

    _graph_check(call, [x], [(bf16_dev(v),) for v in xs], [y, y2], check)


def _moe_weights(orc, key, E, H, I):
    q13 = np.empty((E, 2 * I, H), np.int8)
    s13 = np.empty((E, 2 * I), np.float32)
    q2 = np.empty((E, H, I), np.int8)
    s2 = np.empty((E, H), np.float32)
    for e in range(E):
        q13[e], s13[e] = orc.quant_rows(synth.expert_weights(key, e, 2 * I, H, synth.T_W))
        q2[e], s2[e] = orc.quant_rows(synth.expert_weights(key, e, H, I, synth.T_W2))
    return q13, s13, q2, s2


@pytest.mark.parametrize("T", [1, 5, 40, 700])
def test_moe_graph(orc, T):
    # the four batch paths: single token, one-workgroup prep, wave-per-token
    # routing with the one-workgroup sort, and the large-batch kernels
    E, H, I, k = 16, 256, 128, 4
    say(f"graph moe T={T}")
    key = (73, T)
    W = _moe_weights(orc, key, E, H, I)
    w13, w2 = mq.pack_moe_weights(dev(W[0]), dev(W[2]))
    s13, s2 = dev(W[1]), dev(W[3])
    sets_h = []
    for i in range(2):
        xh = synth.activations((*key, i), T, H, 0, 1.0)
        lh = synth.router_logits((*key, i), T, E)
        sets_h.append((xh, lh))
    x = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wt = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ws = torch.empty(mq.moe_w8a8_workspace_bytes(T, H, E, I, k), dtype=torch.uint8, device="cuda")

    def call():
        mq.moe_w8a8_forward(x, lg, w13, s13, w2, s2, topk=k, topk_ids=ids, topk_w=wt, out=out,
                            ws=ws, packed=True)

    def check(inp):
        xh, lh = bf16_host(inp[0]), host(inp[1])
        ids_ref, w_ref = orc.route_topk(lh, k)
        np.testing.assert_array_equal(host(ids), ids_ref)
        want = orc.moe_forward(xh, ids_ref, w_ref, *W)
        got = bf16_host(out)
        g = orc.bf16_to_f32(got).astype(np.float64)
        r = orc.bf16_to_f32(want).astype(np.float64)
        assert np.all(np.abs(g - r) <= 1e-3 + 1e-2 * np.abs(r))

    _graph_check(call, [x, lg], [(bf16_dev(a), dev(b)) for a, b in sets_h], [out, ids, wt], check)


@pytest.mark.parametrize("M", [2, 100])
def test_mlp_graph(orc, M):
    K, I, N = 512, 192, 128
    key = (74, M)
    qgu, sgu = orc.quant_rows(synth.weights(key, 2 * I, K))
    qd, sd = orc.quant_rows(synth.weights(key, N, I, tensor_id=synth.T_W2))
    wgu_d, wd_d = mq.pack_weights(dev(qgu)), mq.pack_weights(dev(qd))
    sgu_d, sd_d = dev(sgu), dev(sd)
    sets_h = [synth.activations((*key, i), M, K, 4, 20.0) for i in range(2)]
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mq.mlp_w8a8_workspace_bytes(M, K, I, N), dtype=torch.uint8, device="cuda")

    def call():
        mq.mlp_w8a8_packed(x, wgu_d, sgu_d, wd_d, sd_d, I, N, y=y, ws=ws)

    def check(inp):
        want = orc.mlp_forward(bf16_host(inp[0]), qgu, sgu, qd, sd)
        g = orc.bf16_to_f32(bf16_host(y)).astype(np.float64)
        r = orc.bf16_to_f32(want).astype(np.float64)
        assert np.all(np.abs(g - r) <= 1e-3 + 1e-2 * np.abs(r))

    _graph_check(call, [x], [(bf16_dev(a),) for a in sets_h], [y], check)


def test_kv_quant_graph(orc):
    T, Hk, D, rows = 9, 4, 256, 64
    sets_h = [synth.activations((75, i), T, Hk * D, 10, 10.0).reshape(T, Hk, D)
              for i in range(2)]
    slots_h = np.random.default_rng(75).permutation(rows)[:T].astype(np.int32)
    x = torch.empty((T, Hk, D), dtype=torch.bfloat16, device="cuda")
    slots = dev(slots_h)
    q = torch.zeros((rows, Hk, D), dtype=torch.int8, device="cuda")
    s = torch.zeros((rows, Hk), dtype=torch.float16, device="cuda")

    def call():
        mq.kv_quant_i8(x, q, s, slots=slots)

    def check(inp):
        q_ref, s_ref = orc.kv_quant_i8(bf16_host(inp[0]).reshape(T, Hk, D), slots_h, rows)
        np.testing.assert_array_equal(host(q)[slots_h], q_ref[slots_h])
        np.testing.assert_array_equal(host(s).view(np.uint16)[slots_h], s_ref[slots_h])

    _graph_check(call, [x], [(bf16_dev(a),) for a in sets_h], [q, s], check)


def test_stream_read_probe():
    # the measurement helper reads its 481 KiB buffer and leaves the sink
    # alone for zeros (eager and graph-replayed): 37, 13 and 1 chunks, the
    # last with 481 pieces (several rounds of loads, the final one partial)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    buf = torch.zeros(37 * 13 * 1024, dtype=torch.int8, device="cuda")
    for chunk in (13 * 1024, 37 * 1024, 481 * 1024):
        mq.stream_read(buf, chunk, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mq.stream_read(buf, 13 * 1024, sink)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    assert int(sink.item()) == 0


def test_router_and_g128_prep_graph(orc):
    T, H, E = 20, 512, 32
    wg_h = synth.to_bf16_bits(synth.weights((76, 0), E, H))
    wg = bf16_dev(wg_h)
    sets_h = [(synth.activations((76, i), T, H, 4, 10.0), synth.weights((76, i + 1), 24, H))
              for i in range(2)]
    x = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    W = torch.empty((24, H), dtype=torch.float32, device="cuda")
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    qw = torch.empty((24, H), dtype=torch.int8, device="cuda")
    sw = torch.empty((24, H // 128), dtype=torch.bfloat16, device="cuda")
    L = mq.lib()

    def call():
        mq.router_gate_bf16(x, wg, logits=lg)
        st = L.fwht128_weight_prep_g128(W.data_ptr(), 24, H, qw.data_ptr(), sw.data_ptr(),
                                        torch.cuda.current_stream().cuda_stream)
        assert st == 0

    def check(inp):
        ref = orc.router_gate_bf16(bf16_host(inp[0]), wg_h)
        xf = orc.bf16_to_f32(bf16_host(inp[0])).astype(np.float64)
        bound = H * 2.0 ** -24 * (np.abs(xf) @ np.abs(orc.bf16_to_f32(wg_h)).astype(
            np.float64).T)
        assert np.all(np.abs(host(lg) - ref) <= bound + 1e-30)
        q_ref, s_ref = orc.weight_prep_g128(host(inp[1]))
        np.testing.assert_array_equal(host(qw), q_ref)
        np.testing.assert_array_equal(bf16_host(sw), s_ref)

    _graph_check(call, [x, W], [(bf16_dev(a), dev(b)) for a, b in sets_h], [lg, qw, sw], check)


@pytest.mark.parametrize("T", [2, 40, 200])
def test_rot_moe_and_shared_graph(orc, T):
    # split-K forms (2 and 40 tokens) and, at 200 tokens (800 pairs), the
    # one-wave-per-tile GEMMs of the routed experts and of the shared expert
    E, H, I, k, Is = 8, 256, 128, 4, 128
    key = (77, T)
    q13 = np.empty((E, 2 * I, H), np.int8)
    s13 = np.empty((E, 2 * I, H // 128), np.uint16)
    q2 = np.empty((E, H, I), np.int8)
    s2 = np.empty((E, H, I // 128), np.uint16)
    for e in range(E):
        q13[e], s13[e] = orc.weight_prep_g128(synth.expert_weights(key, e, 2 * I, H, synth.T_W))
        q2[e], s2[e] = orc.weight_prep_g128(synth.expert_weights(key, e, H, I, synth.T_W2))
    S = (*orc.weight_prep_g256(synth.weights(key, 2 * Is, H)),
         *orc.weight_prep_g128(synth.weights(key, H, Is, tensor_id=synth.T_W2)))
    w13, w2 = mq.pack_moe_weights(dev(q13), dev(q2))
    Wd = (w13, bf16_dev(s13), w2, bf16_dev(s2))
    Sd = (mq.pack_weights(dev(S[0])), dev(S[1]), bf16_dev(S[2]), mq.pack_weights(dev(S[3])),
          bf16_dev(S[4]))
    sets_h = [(synth.activations((*key, i), T, H, 0, 1.0), synth.router_logits((*key, i), T, E))
              for i in range(2)]
    x = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wt = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ws = torch.empty(mq.moe_w8a8_workspace_bytes(T, H, E, I, k), dtype=torch.uint8, device="cuda")
    wss = torch.empty(mq.shared_expert_w8a8_rot_workspace_bytes(T, H, Is), dtype=torch.uint8,
                      device="cuda")

    def call():
        mq.shared_expert_w8a8_rot(x, *Sd, y=y, ws=wss)
        mq.moe_w8a8_rot_forward(x, lg, *Wd, topk=k, shared=y, topk_ids=ids, topk_w=wt, out=out,
                                ws=ws)

    def check(inp):
        xh, lh = bf16_host(inp[0]), host(inp[1])
        y_ref = orc.shared_expert(xh, *S)
        ids_ref, w_ref = orc.route_topk(lh, k)
        np.testing.assert_array_equal(host(ids), ids_ref)
        want = orc.moe_rot_forward(xh, ids_ref, w_ref, q13, s13, q2, s2, shared=y_ref)
        g = orc.bf16_to_f32(bf16_host(out)).astype(np.float64)
        r = orc.bf16_to_f32(want).astype(np.float64)
        assert np.all(np.abs(g - r) <= 1e-3 + 1e-2 * np.abs(r))

    _graph_check(call, [x, lg], [(bf16_dev(a), dev(b)) for a, b in sets_h], [y, out, ids, wt],
                 check)


@pytest.mark.parametrize("T", [1, 2])
def test_rot_layer_with_shared_graph(orc, T):
    # the one-call layer: one token with the shared expert inside the two
    # routed launches, two tokens composed
    E, H, I, k, Is = 8, 256, 128, 4, 256
    key = (78, T)
    q13 = np.empty((E, 2 * I, H), np.int8)
    s13 = np.empty((E, 2 * I, H // 128), np.uint16)
    q2 = np.empty((E, H, I), np.int8)
    s2 = np.empty((E, H, I // 128), np.uint16)
    for e in range(E):
        q13[e], s13[e] = orc.weight_prep_g128(synth.expert_weights(key, e, 2 * I, H, synth.T_W))
        q2[e], s2[e] = orc.weight_prep_g128(synth.expert_weights(key, e, H, I, synth.T_W2))
    S = (*orc.weight_prep_g256(synth.weights(key, 2 * Is, H)),
         *orc.weight_prep_g128(synth.weights(key, H, Is, tensor_id=synth.T_W2)))
    w13, w2 = mq.pack_moe_weights(dev(q13), dev(q2))
    Wd = (w13, bf16_dev(s13), w2, bf16_dev(s2))
    Sd = (mq.pack_weights(dev(S[0])), dev(S[1]), bf16_dev(S[2]), mq.pack_weights(dev(S[3])),
          bf16_dev(S[4]))
    sets_h = [(synth.activations((*key, i), T, H, 0, 1.0), synth.router_logits((*key, i), T, E))
              for i in range(2)]
    x = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wt = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ws = torch.empty(mq.lib().moe_w8a8_rot_shared_workspace_bytes(T, H, E, I, k, Is),
                     dtype=torch.uint8, device="cuda")

    def call():
        mq.moe_w8a8_rot_shared_forward(x, lg, *Wd, topk=k, shared_w=Sd, topk_ids=ids, topk_w=wt,
                                       out=out, ws=ws)

    def check(inp):
        xh, lh = bf16_host(inp[0]), host(inp[1])
        y_ref = orc.shared_expert(xh, *S)
        ids_ref, w_ref = orc.route_topk(lh, k)
        np.testing.assert_array_equal(host(ids), ids_ref)
        want = orc.moe_rot_forward(xh, ids_ref, w_ref, q13, s13, q2, s2, shared=y_ref)
        g = orc.bf16_to_f32(bf16_host(out)).astype(np.float64)
        r = orc.bf16_to_f32(want).astype(np.float64)
        assert np.all(np.abs(g - r) <= 1e-3 + 1e-2 * np.abs(r))

    _graph_check(call, [x, lg], [(bf16_dev(a), dev(b)) for a, b in sets_h], [out, ids, wt], check)


@pytest.mark.parametrize("M", [3, 300])
def test_unpacked_linear_pack_and_noalloc_graph(orc, M):
    # linear_w8a8 (row-major weights), w8a8_pack_weights, the allocation-free
    # linear and the g256 preparation + packed g256 GEMM, in one graph
    K, N = 1024, 1280
    xs, qw, sw = _dense(orc, M, K, N, 200 + M)
    Wg = synth.weights((78, M), 256, K)
    qg_ref, su_ref, s2_ref = orc.weight_prep_g256(Wg)
    qw_d, sw_d, Wg_d = dev(qw), dev(sw), dev(Wg)
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    yg = torch.empty((M, 256), dtype=torch.bfloat16, device="cuda")
    qp = torch.empty((N * K,), dtype=torch.int8, device="cuda")
    qg = torch.empty((256, K), dtype=torch.int8, device="cuda")
    su = torch.empty((256, K // 256), dtype=torch.uint8, device="cuda")
    s2 = torch.empty((256,), dtype=torch.bfloat16, device="cuda")
    qgp = torch.empty((256 * K,), dtype=torch.int8, device="cuda")
    qa = torch.empty((M, K), dtype=torch.int8, device="cuda")
    sa = torch.empty((M,), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(256, mq.linear_w8a8_workspace_bytes(M, N, K)), dtype=torch.uint8,
                     device="cuda")
    wsg = torch.empty(max(256, mq.gemm_w8a8_g256_workspace_bytes(M, 256, K)), dtype=torch.uint8,
                      device="cuda")
    L = mq.lib()

    def call():
        st = torch.cuda.current_stream().cuda_stream
        mq.linear_w8a8(x, qw_d, sw_d, y=y, ws=ws)
        assert L.w8a8_pack_weights(qw_d.data_ptr(), N, K, K, qp.data_ptr(), st) == 0
        mq.linear_w8a8_packed_noalloc(x, qp, sw_d, N, y=y2)
        assert L.fwht128_weight_prep_g256(Wg_d.data_ptr(), 256, K, qg.data_ptr(), su.data_ptr(),
                                          s2.data_ptr(), st) == 0
        assert L.w8a8_pack_weights(qg.data_ptr(), 256, K, K, qgp.data_ptr(), st) == 0
        mq.fwht128_quant(x, q=qa, s=sa)
        mq.gemm_w8a8_g256(qa, sa, qgp, su, s2, y=yg, ws=wsg, packed=True)

    def check(inp):
        xh = bf16_host(inp[0])
        want = orc.linear_w8a8(xh, qw, sw)
        np.testing.assert_array_equal(bf16_host(y), want)
        np.testing.assert_array_equal(bf16_host(y2), want)
        np.testing.assert_array_equal(host(qg), qg_ref)
        np.testing.assert_array_equal(host(su), su_ref)
        np.testing.assert_array_equal(bf16_host(s2), s2_ref)
        qr, sr = orc.fwht128_quant(xh)
        np.testing.assert_array_equal(bf16_host(yg), orc.gemm_g256(qr, sr, qg_ref, su_ref,
                                                                    s2_ref))

    _graph_check(call, [x], [(bf16_dev(v),) for v in xs], [y, y2, qp, qg, su, s2, qgp, yg],
                 check)
