"""Pins for the oracle's Hadamard-domain expert formats and layers: the g128
weight preparation (O16), the g128 GEMM (O17), the rotated requant (O18), the
routed experts on the rotated grid (O19), the shared expert (O20) and the bf16
router gate (O21).

What pins them:
  - g128 prep: hand-worked rows (tests/golden/g128_prep_worked.txt; a bf16
    scale tie, code ties, zero groups), and each plausible misreading planted
    in a copy of the oracle's C source must fail them;
  - g128 GEMM: a closed form (single-column rows whose rotation and codes are
    exact give exactly x . w, which pins the 2^-7 and where the scales go) and
    a special case that reduces to the already pinned int32 GEMM;
  - rotated requant = the pinned fwht128 followed by the pinned row quant;
  - routed layer: one expert, top-1, weight 1 equals a chain built from the
    pinned pieces and torch's float64 SiLU; the shared term is added after the
    slot-order fp32 sum; token permutation and batch invariance;
  - shared expert: its gate/up projection rounded to bf16 equals the pinned
    g256 GEMM's output, the rest is the pinned chain;
  - router gate: unit vectors give weight columns exactly, integer operands
    are exact, and float64 BLAS agrees to one fp32 ulp.
Sources: "Qwen3.6-35B-A3B IQ8R - radiance container" (Experts and Activations
rows, the recipe's ffn_*_exps / ffn_*_shexp lines); "[gfx1151] Online INT8
W8A8 ..." (ATOM pull request): intro (router gate BF16) and Changes,
fused_moe_triton.py bullet (the routed order).
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))
U = 2.0 ** -10


def _golden():
    rows, scales, codes = [], [], []
    for line in open(os.path.join(HERE, "golden", "g128_prep_worked.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        ent, st, ct = [p.strip() for p in line.split("|")]
        w = np.zeros(256, np.float32)
        if ent != "-":
            for e in ent.split():
                k, v = e.split(":")
                w[int(k)] = np.float32(float(v) * U)
        rows.append(w)
        scales.append([float(v) * U for v in st.split()])
        q = np.zeros(256, np.int8)
        for b, blk in enumerate(ct.split()):
            for i, c in enumerate(int(v) for v in blk.split(",")):
                q[b * 128 + i:(b + 1) * 128:4] = c
        codes.append(q)
    return np.stack(rows), np.array(scales), np.stack(codes)


def _matches(prep):
    W, s_ref, q_ref = _golden()
    q, s = prep(W)
    return (np.array_equal(oracle.bf16_to_f32(s).astype(np.float64), s_ref)
            and np.array_equal(q, q_ref))


def test_g128_worked_cases():
    W, s_ref, q_ref = _golden()
    q, s = oracle.weight_prep_g128(W)
    np.testing.assert_array_equal(oracle.bf16_to_f32(s).astype(np.float64), s_ref)
    np.testing.assert_array_equal(q, q_ref)


G128_MUTANTS = {
    "codes against the unrounded scale": ("float sf = bf16_to_f32(sb);", "float sf = a / 127.0f;"),
    "scale over 128": ("f32_to_bf16(a / 127.0f)", "f32_to_bf16(a / 128.0f)"),
    "codes round half away": ("nearbyintf(row[k] / sf)", "roundf(row[k] / sf)"),
}


@pytest.mark.parametrize("name", sorted(G128_MUTANTS))
def test_g128_worked_cases_reject_misreadings(tmp_path, name):
    old, new = G128_MUTANTS[name]
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    assert src.count(old) == 1, f"mutation site not unique: {old!r}"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", *oracle.CFLAGS, "-o", str(so), str(path), "-lm"])
    lib = ctypes.CDLL(str(so))

    def prep(W):
        W = np.ascontiguousarray(W, np.float32)
        N, K = W.shape
        q = np.empty((N, K), np.int8)
        s = np.empty((N, K // 128), np.uint16)
        lib.orc_weight_prep_g128(ctypes.c_void_p(W.ctypes.data), ctypes.c_int64(N),
                                 ctypes.c_int64(K), ctypes.c_void_p(q.ctypes.data),
                                 ctypes.c_void_p(s.ctypes.data))
        return q, s

    assert _matches(oracle.weight_prep_g128)
    assert not _matches(prep), f"the worked cases accept the mutant: {name}"


def test_g128_gemm_closed_form():
    # x row: 127 at position i of each block (its rotation is +-127 everywhere:
    # scale 1, codes +-127 exactly); w row: d * 2^-3 * 127 at position j of
    # each block with d in {1, -1} (scale 2^-3, codes +-127).  Then
    # <Hx, Hw> = 128 <x, w> makes y = x . w exactly.
    K = 256
    r = np.random.default_rng(0)
    xs, ws = [], []
    for _ in range(5):
        x = np.zeros(K, np.float32)
        for b in range(2):
            x[b * 128 + r.integers(128)] = 127.0
        xs.append(x)
    for _ in range(6):
        w = np.zeros(K, np.float32)
        for b in range(2):
            w[b * 128 + r.integers(128)] = 127.0 / 8 * (1 if r.random() < 0.5 else -1)
        ws.append(w)
    X, W = np.stack(xs), np.stack(ws)
    qa, sa = oracle.fwht128_quant(synth.to_bf16_bits(X))
    assert np.all(sa == 1.0)
    qw, s = oracle.weight_prep_g128(W)
    assert np.all(oracle.bf16_to_f32(s) == 0.125)
    y = oracle.gemm_g128(qa, sa, qw, s)
    np.testing.assert_array_equal(y, (X.astype(np.float64) @ W.astype(np.float64).T).astype(
        np.float32))


def test_g128_gemm_reduces_to_int32_gemm():
    # every group scale 1 and a row scale of 128: y = sum of the exact int32
    # group sums (the pinned int32 GEMM) times 128 * 2^-7 = 1
    r = np.random.default_rng(1)
    M, N, K = 5, 7, 512
    qa = r.integers(-127, 128, (M, K)).astype(np.int8)
    qw = r.integers(-127, 128, (N, K)).astype(np.int8)
    s = synth.to_bf16_bits(np.ones((N, K // 128), np.float32))
    y = oracle.gemm_g128(qa, np.full(M, 128.0, np.float32), qw, s)
    np.testing.assert_array_equal(y, oracle.gemm_i32(qa, qw).astype(np.float32))


def test_rot_quant_is_fwht_then_row_quant():
    x = np.random.default_rng(2).standard_normal((6, 512)).astype(np.float32)
    x[2] = 0
    q, s = oracle.rot_quant_rows(x)
    q2, s2 = oracle.quant_rows(oracle.fwht128_rows(x))
    np.testing.assert_array_equal(q, q2)
    np.testing.assert_array_equal(s, s2)


def _rot_layer(T, E, H, I, k, seed):
    key = (92, seed)
    x = synth.activations(key, T, H, 0, 1.0)
    w13 = np.empty((E, 2 * I, H), np.int8)
    s13 = np.empty((E, 2 * I, H // 128), np.uint16)
    w2 = np.empty((E, H, I), np.int8)
    s2 = np.empty((E, H, I // 128), np.uint16)
    for e in range(E):
        w13[e], s13[e] = oracle.weight_prep_g128(synth.expert_weights(key, e, 2 * I, H, synth.T_W))
        w2[e], s2[e] = oracle.weight_prep_g128(synth.expert_weights(key, e, H, I, synth.T_W2))
    ids, w = oracle.route_topk(synth.router_logits(key, T, E), k)
    return x, ids, w, w13, s13, w2, s2


def _chain(x_row, e, w13, s13, w2, s2):
    qx, sx = oracle.fwht128_quant(x_row[None])
    h = oracle.gemm_g128(qx, sx, w13[e], s13[e])
    g, u = h[:, 0::2], h[:, 1::2]
    silu = torch.nn.functional.silu(torch.from_numpy(g.astype(np.float64))).numpy()
    act = silu.astype(np.float32) * u
    return act[0], qx, sx


def test_rot_layer_single_expert_chain():
    T, E, H, I, k = 4, 2, 256, 128, 1
    x, ids, w, w13, s13, w2, s2 = _rot_layer(T, E, H, I, k, 1)
    w[:] = 1.0
    out, d = oracle.moe_rot_forward(x, ids, w, w13, s13, w2, s2, debug=True)
    for t in range(T):
        e = ids[t, 0]
        act, qx, sx = _chain(x[t], e, w13, s13, w2, s2)
        np.testing.assert_array_equal(d["qx"][t], qx[0])
        assert d["sx"][t] == sx[0]
        np.testing.assert_allclose(d["act"][t], act, rtol=2 ** -22, atol=1e-30)
        qa, sa = oracle.rot_quant_rows(d["act"][t:t + 1])
        np.testing.assert_array_equal(d["qa"][t], qa[0])
        assert d["sa2"][t] == sa[0]
        y2 = oracle.gemm_g128(qa, sa, w2[e], s2[e])[0]
        np.testing.assert_array_equal(d["y2"][t], y2)
        np.testing.assert_array_equal(out[t], oracle.bf16_round(y2))


def test_rot_layer_shared_term_and_invariances():
    T, E, H, I, k = 6, 8, 256, 128, 4
    x, ids, w, w13, s13, w2, s2 = _rot_layer(T, E, H, I, k, 2)
    shared = np.random.default_rng(3).standard_normal((T, H)).astype(np.float32)
    out, d = oracle.moe_rot_forward(x, ids, w, w13, s13, w2, s2, shared=shared, debug=True)
    y2 = d["y2"].reshape(T, k, H)
    acc = np.zeros((T, H), np.float32)
    for j in range(k):
        acc = acc + w[:, j:j + 1] * y2[:, j]
    np.testing.assert_array_equal(out, oracle.bf16_round(acc + shared))
    out0 = oracle.moe_rot_forward(x, ids, w, w13, s13, w2, s2)
    np.testing.assert_array_equal(out0, oracle.bf16_round(acc))
    perm = np.random.default_rng(4).permutation(T)
    outp = oracle.moe_rot_forward(np.ascontiguousarray(x[perm]), np.ascontiguousarray(ids[perm]),
                                  np.ascontiguousarray(w[perm]), w13, s13, w2, s2,
                                  shared=np.ascontiguousarray(shared[perm]))
    np.testing.assert_array_equal(outp, out[perm])


def test_shared_expert_chain():
    T, H, Is = 3, 512, 128
    key = (93, 1)
    x = synth.activations(key, T, H, 5, 10.0, heavy_tail=True)
    wgu, su8, s2 = oracle.weight_prep_g256(synth.weights(key, 2 * Is, H))
    wd, sd = oracle.weight_prep_g128(synth.weights(key, H, Is, tensor_id=synth.T_W2))
    y, act = oracle.shared_expert(x, wgu, su8, s2, wd, sd, debug=True)
    qx, sx = oracle.fwht128_quant(x)
    hb = oracle.gemm_g256(qx, sx, wgu, su8, s2)  # the pinned g256 GEMM, bf16 out
    _, ts = oracle.gemm_g256(qx, sx, wgu, su8, s2, return_tsum=True)
    h = ((ts.astype(np.float64) * sx[:, None].astype(np.float64))
         * oracle.bf16_to_f32(s2)[None, :].astype(np.float64) / 128.0).astype(np.float32)
    np.testing.assert_array_equal(oracle.bf16_round(h), hb)
    g, u = h[:, 0::2], h[:, 1::2]
    ref_act = torch.nn.functional.silu(torch.from_numpy(g.astype(np.float64))).numpy().astype(
        np.float32) * u
    np.testing.assert_allclose(act, ref_act, rtol=2 ** -22, atol=1e-30)
    qa, sa = oracle.rot_quant_rows(act)
    np.testing.assert_array_equal(y, oracle.gemm_g128(qa, sa, wd, sd))


def test_router_gate_exact_cases():
    r = np.random.default_rng(6)
    T, H, E = 5, 256, 16
    wg = synth.to_bf16_bits(r.standard_normal((E, H)).astype(np.float32))
    # unit vectors pick weight columns exactly
    X = np.zeros((T, H), np.float32)
    cols = r.integers(0, H, T)
    X[np.arange(T), cols] = 1.0
    lg = oracle.router_gate_bf16(synth.to_bf16_bits(X), wg)
    np.testing.assert_array_equal(lg, oracle.bf16_to_f32(wg)[:, cols].T)
    # small integers: every partial sum exact
    xi = r.integers(-8, 9, (T, H)).astype(np.float32)
    wi = r.integers(-8, 9, (E, H)).astype(np.float32)
    lg = oracle.router_gate_bf16(synth.to_bf16_bits(xi), synth.to_bf16_bits(wi))
    np.testing.assert_array_equal(lg, (xi.astype(np.int64) @ wi.astype(np.int64).T).astype(
        np.float32))
    # float64 BLAS on the same bf16 values: one fp32 ulp
    xb = synth.activations((94, 1), T, H, 0, 1.0)
    lg = oracle.router_gate_bf16(xb, wg)
    ref = oracle.bf16_to_f32(xb).astype(np.float64) @ oracle.bf16_to_f32(wg).astype(np.float64).T
    np.testing.assert_allclose(lg, ref.astype(np.float32), rtol=2 ** -23, atol=1e-6)
