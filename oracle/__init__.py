"""CPU oracle for online INT8 W8A8 (dense, routed MoE, fwht128 / g256).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the product package.  The oracle
is the plain C file ``oracle.c`` (built into ``liboracle.so``) and these ctypes
wrappers, which only marshal numpy arrays.  It shares no code with the HIP
library.

Every function cites the passage of the source pages it follows; see the
header of ``oracle.c`` for the page titles and the numeric conventions.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no -march, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        _lib = ctypes.CDLL(_LIB_PATH)
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return ctypes.c_void_p(0)
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


_i64 = ctypes.c_int64


def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().orc_threads())


def set_threads(n: int) -> None:
    """OpenMP threads for the oracle's parallel loops (results do not depend on it)."""
    _load().orc_set_threads(ctypes.c_int(int(n)))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, np.uint16)
    _load().orc_bf16_round(_p(x), _i64(x.size), _p(y))
    return y


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp32 values (exact)."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def quant_rows(x: np.ndarray):
    """O1 / O2: symmetric per-row int8 quantisation.

    "Qwen3.6-27B-Quark-W8A8-INT8", Quantization Scheme table: per-token
    (activations) and per-channel (weights) symmetric INT8.  scale = amax/127
    (fp32), code = round-half-even(x / scale) clamped to [-127, 127].
    ``x`` is fp32 [M, K] or bf16 bit patterns (uint16) [M, K].
    Returns (q int8 [M, K], s fp32 [M]).
    """
    x = np.ascontiguousarray(x)
    M, K = x.shape
    q = np.empty((M, K), np.int8)
    s = np.empty((M,), np.float32)
    lib = _load()
    if x.dtype == np.uint16:
        lib.orc_quant_rows_bf16(_p(x), _i64(M), _i64(K), _i64(K), _p(q), _i64(K), _p(s))
    elif x.dtype == np.float32:
        lib.orc_quant_rows_f32(_p(x), _i64(M), _i64(K), _i64(K), _p(q), _i64(K), _p(s))
    else:
        raise TypeError(f"quant_rows: unsupported dtype {x.dtype}")
    return q, s


def gemm_i32(qa: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """O3 step 1: acc[m, n] = sum_k qa[m, k] * qw[n, k], exact (int32 result)."""
    qa = np.ascontiguousarray(qa, np.int8)
    qw = np.ascontiguousarray(qw, np.int8)
    M, K = qa.shape
    N, K2 = qw.shape
    assert K == K2
    acc = np.empty((M, N), np.int32)
    _load().orc_gemm_i32(_p(qa), _i64(K), _p(qw), _i64(K), _i64(M), _i64(N), _i64(K),
                         _p(acc), _i64(N))
    return acc


def epilogue(acc: np.ndarray, sa: np.ndarray, sw: np.ndarray) -> np.ndarray:
    """O3 step 2: y = bf16((float(acc) * sa[m]) * sw[n]), fp32, no FMA."""
    acc = np.ascontiguousarray(acc, np.int32)
    sa = np.ascontiguousarray(sa, np.float32)
    sw = np.ascontiguousarray(sw, np.float32)
    M, N = acc.shape
    y = np.empty((M, N), np.uint16)
    _load().orc_epilogue(_p(acc), _i64(N), _p(sa), _p(sw), _i64(M), _i64(N), _p(y), _i64(N))
    return y


def gemm_w8a8(qa, sa, qw, sw) -> np.ndarray:
    """O3: int8 GEMM plus the per-token x per-channel fp32 epilogue, bf16 out.

    "[gfx1151] Online INT8 W8A8 ..." (ATOM pull request), Changes: per-token
    int8 activations against int8 weights with per-channel fp32 scales.
    """
    qa = np.ascontiguousarray(qa, np.int8)
    qw = np.ascontiguousarray(qw, np.int8)
    sa = np.ascontiguousarray(sa, np.float32)
    sw = np.ascontiguousarray(sw, np.float32)
    M, K = qa.shape
    N = qw.shape[0]
    y = np.empty((M, N), np.uint16)
    _load().orc_gemm_w8a8(_p(qa), _p(sa), _i64(K), _p(qw), _p(sw), _i64(K), _i64(M), _i64(N),
                          _i64(K), _p(y), _i64(N))
    return y


def gemm_w8a8_points(qa, sa, qw, sw, ms, ns):
    """O3 at selected outputs (ms[p], ns[p]); returns (acc int32 [P], y bf16 [P])."""
    qa = np.ascontiguousarray(qa, np.int8)
    qw = np.ascontiguousarray(qw, np.int8)
    sa = np.ascontiguousarray(sa, np.float32)
    sw = np.ascontiguousarray(sw, np.float32)
    ms = np.ascontiguousarray(ms, np.int64)
    ns = np.ascontiguousarray(ns, np.int64)
    K = qa.shape[1]
    P = ms.size
    acc = np.empty((P,), np.int32)
    y = np.empty((P,), np.uint16)
    _load().orc_gemm_w8a8_points(_p(qa), _p(sa), _i64(K), _p(qw), _p(sw), _i64(K), _i64(K),
                                 _p(ms), _p(ns), _i64(P), _p(acc), _p(y))
    return acc, y


def linear_w8a8(x_bf16, qw, sw) -> np.ndarray:
    """O1 then O3: bf16 activations -> per-token int8 -> GEMM -> bf16."""
    x_bf16 = np.ascontiguousarray(x_bf16, np.uint16)
    qw = np.ascontiguousarray(qw, np.int8)
    sw = np.ascontiguousarray(sw, np.float32)
    M, K = x_bf16.shape
    N = qw.shape[0]
    y = np.empty((M, N), np.uint16)
    _load().orc_linear_w8a8(_p(x_bf16), _i64(M), _i64(K), _p(qw), _p(sw), _i64(N), _p(y))
    return y


def route_topk(logits: np.ndarray, k: int):
    """O4: softmax over experts, top-k, renormalise (fp64, rounded to fp32).

    "[gfx1151] Online INT8 W8A8 ..." (ATOM pull request), Changes: routing is
    the first step of the int8 MoE forward.  Slot j = j-th largest logit,
    ties to the lower expert index.  Returns (ids int32 [T, k], w fp32 [T, k]).
    """
    logits = np.ascontiguousarray(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    _load().orc_route_topk(_p(logits), _i64(T), _i64(E), _i64(k), _p(ids), _p(w))
    return ids, w


def expert_counts(ids: np.ndarray, E: int) -> np.ndarray:
    """O5: number of routed (token, slot) pairs per expert."""
    ids = np.ascontiguousarray(ids, np.int32)
    counts = np.empty((E,), np.int32)
    _load().orc_expert_counts(_p(ids), _i64(ids.size), _i64(E), _p(counts))
    return counts


def moe_forward(x_bf16, ids, w, w13, s13, w2, s2, debug: bool = False):
    """O6..O10: routed int8 MoE forward for given routing (ids, w).

    "[gfx1151] Online INT8 W8A8 ..." (ATOM pull request), Changes,
    fused_moe_triton.py bullet: per-token int8 quant -> gemm1 with gated SiLU
    over interleaved w13 rows (2i = gate, 2i+1 = up) -> per-token int8 requant
    -> gemm2 -> weighted scatter/combine.  Shapes: x [T, H] bf16, ids/w [T, k],
    w13 [E, 2I, H] int8, s13 [E, 2I] fp32, w2 [E, H, I] int8, s2 [E, H] fp32.
    Returns out bf16 [T, H], plus a dict of intermediates when ``debug``.
    """
    x_bf16 = np.ascontiguousarray(x_bf16, np.uint16)
    ids = np.ascontiguousarray(ids, np.int32)
    w = np.ascontiguousarray(w, np.float32)
    w13 = np.ascontiguousarray(w13, np.int8)
    s13 = np.ascontiguousarray(s13, np.float32)
    w2 = np.ascontiguousarray(w2, np.int8)
    s2 = np.ascontiguousarray(s2, np.float32)
    T, H = x_bf16.shape
    k = ids.shape[1]
    E, I2, H2 = w13.shape
    I = I2 // 2
    assert H2 == H and w2.shape == (E, H, I) and s13.shape == (E, I2) and s2.shape == (E, H)
    out = np.empty((T, H), np.uint16)
    dbg = None
    if debug:
        R = T * k
        dbg = dict(qx=np.empty((T, H), np.int8), sx=np.empty((T,), np.float32),
                   acc1=np.empty((R, I2), np.int32), act=np.empty((R, I), np.float32),
                   qa=np.empty((R, I), np.int8), sa2=np.empty((R,), np.float32),
                   acc2=np.empty((R, H), np.int32), y2=np.empty((R, H), np.float32))
    g = (lambda name: _p(dbg[name])) if debug else (lambda name: ctypes.c_void_p(0))
    _load().orc_moe_forward(_p(x_bf16), _p(ids), _p(w), _p(w13), _p(s13), _p(w2), _p(s2),
                            _i64(T), _i64(H), _i64(E), _i64(I), _i64(k), _p(out),
                            g("qx"), g("sx"), g("acc1"), g("act"), g("qa"), g("sa2"),
                            g("acc2"), g("y2"))
    return (out, dbg) if debug else out


def mlp_forward(x_bf16, wgu, sgu, wd, sd, debug: bool = False):
    """O14: dense W8A8 MLP block.

    "[gfx1151] Online INT8 W8A8 ..." (ATOM pull request): A8W8 for all dense
    GEMMs (intro); the gated-SiLU and requant order of its Changes,
    fused_moe_triton.py bullet, on the dense gate_up and down linears:
    per-token int8 quant -> gate_up GEMM (rows 2i = gate, 2i+1 = up) ->
    SiLU(gate) * up in fp32 -> per-token int8 requant -> down GEMM -> bf16.
    Shapes: x [M, K] bf16, wgu [2I, K] int8, sgu [2I] fp32, wd [N, I] int8,
    sd [N] fp32.  Returns y bf16 [M, N], plus a dict of intermediates when
    ``debug``.
    """
    x_bf16 = np.ascontiguousarray(x_bf16, np.uint16)
    wgu = np.ascontiguousarray(wgu, np.int8)
    sgu = np.ascontiguousarray(sgu, np.float32)
    wd = np.ascontiguousarray(wd, np.int8)
    sd = np.ascontiguousarray(sd, np.float32)
    M, K = x_bf16.shape
    I2, K2 = wgu.shape
    I = I2 // 2
    N = wd.shape[0]
    assert K2 == K and wd.shape == (N, I) and sgu.shape == (I2,) and sd.shape == (N,)
    y = np.empty((M, N), np.uint16)
    dbg = None
    if debug:
        dbg = dict(qx=np.empty((M, K), np.int8), sx=np.empty((M,), np.float32),
                   acc1=np.empty((M, I2), np.int32), act=np.empty((M, I), np.float32),
                   qa=np.empty((M, I), np.int8), sa=np.empty((M,), np.float32),
                   acc2=np.empty((M, N), np.int32))
    g = (lambda name: _p(dbg[name])) if debug else (lambda name: ctypes.c_void_p(0))
    _load().orc_mlp_forward(_p(x_bf16), _i64(M), _i64(K), _p(wgu), _p(sgu), _i64(I), _p(wd),
                            _p(sd), _i64(N), _p(y), g("qx"), g("sx"), g("acc1"), g("act"),
                            g("qa"), g("sa"), g("acc2"))
    return (y, dbg) if debug else y


def f32_to_f16(x: np.ndarray) -> np.ndarray:
    """fp32 -> IEEE binary16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, np.uint16)
    _load().orc_f32_to_f16(_p(x), _i64(x.size), _p(y))
    return y


def kv_quant_i8(x_bf16: np.ndarray, slots: np.ndarray | None = None, rows: int | None = None):
    """O15: int8 KV-cache quantisation with an f16 scale per token and head.

    "Qwen3.6-35B-A3B IQ8R - radiance container", Serve: kv-cache-dtype i8
    stores the attention cache as int8 with an f16 scale per token and head.
    s = f16(amax / 127), code = round-half-even(x / s) clamped to +-127 (0 for
    a zero scale).  ``x_bf16`` [T, Hk, D] (uint16 bf16 bits); token t goes to
    cache row ``slots[t]`` (row t without slots; negative skips), ``rows``
    cache rows (default T).  Returns (q int8 [rows, Hk, D], s f16 bits
    uint16 [rows, Hk]); rows no token writes stay zero.
    """
    x_bf16 = np.ascontiguousarray(x_bf16, np.uint16)
    T, Hk, D = x_bf16.shape
    rows = T if rows is None else rows
    q = np.zeros((rows, Hk, D), np.int8)
    s = np.zeros((rows, Hk), np.uint16)
    sl = None if slots is None else np.ascontiguousarray(slots, np.int32)
    _load().orc_kv_quant_i8(_p(x_bf16), _i64(T), _i64(Hk), _i64(D), _i64(Hk * D), _p(sl),
                            _p(q), _i64(Hk * D), _p(s), _i64(Hk))
    return q, s


def fwht128_rows(v: np.ndarray) -> np.ndarray:
    """O11: fp32 fast Walsh-Hadamard transform of every 128-block of each row.

    "Qwen3.6-35B-A3B IQ8R - radiance container", Trunk row: each 128 of K
    rotated by the unnormalised Hadamard.  Natural (Sylvester) order, stages
    h = 1..64, pair (i, i+h) -> (a + b, a - b).  Returns a new array.
    """
    v = np.array(v, dtype=np.float32, order="C", copy=True)
    if v.ndim == 1:
        v = v[None, :]
        squeeze = True
    else:
        squeeze = False
    M, K = v.shape
    assert K % 128 == 0
    _load().orc_fwht128_rows(_p(v), _i64(M), _i64(K), _i64(K))
    return v[0] if squeeze else v


def fwht128_quant(x_bf16: np.ndarray):
    """O11 then O1: rotate each 128-block of the bf16 row, quantise the row.

    "Qwen3.6-35B-A3B IQ8R - radiance container", Activations row: int8
    activations under the same rotation.  Returns (q int8 [M, K], s fp32 [M]).
    """
    x_bf16 = np.ascontiguousarray(x_bf16, np.uint16)
    M, K = x_bf16.shape
    q = np.empty((M, K), np.int8)
    s = np.empty((M,), np.float32)
    _load().orc_fwht128_quant(_p(x_bf16), _i64(M), _i64(K), _i64(K), _p(q), _i64(K), _p(s))
    return q, s


def weight_prep_g256(W: np.ndarray):
    """O12: rotated int8 weights, u8 scale per row per 256 of K, bf16 row scale.

    "Qwen3.6-35B-A3B IQ8R - radiance container", Trunk row and the recipe
    (group=256 scale=u8 scale2=bf16 block2=1x* transform=fwht128 clamp=sym).
    Returns (qw int8 [N, K], su8 uint8 [N, K/256], s2 bf16 bits uint16 [N]).
    """
    W = np.ascontiguousarray(W, np.float32)
    N, K = W.shape
    assert K % 256 == 0
    qw = np.empty((N, K), np.int8)
    su8 = np.empty((N, K // 256), np.uint8)
    s2 = np.empty((N,), np.uint16)
    _load().orc_weight_prep_g256(_p(W), _i64(N), _i64(K), _p(qw), _p(su8), _p(s2))
    return qw, su8, s2


def weight_prep_g128(W: np.ndarray):
    """O16: rotated int8 weights with a bf16 scale per row per 128 of K.

    "Qwen3.6-35B-A3B IQ8R - radiance container", Experts row and the recipe
    (group=128 scale=bf16 transform=fwht128 clamp=sym).  s = bf16(amax/127)
    per 128-block of the rotated row, codes against the stored bf16 scale.
    Returns (qw int8 [N, K], s bf16 bits uint16 [N, K/128]).
    """
    W = np.ascontiguousarray(W, np.float32)
    N, K = W.shape
    assert K % 128 == 0
    qw = np.empty((N, K), np.int8)
    s = np.empty((N, K // 128), np.uint16)
    _load().orc_weight_prep_g128(_p(W), _i64(N), _i64(K), _p(qw), _p(s))
    return qw, s


def gemm_g128(qa, sa, qw, s):
    """O17: rotated-domain GEMM with a bf16 scale per row per 128 of K, fp32 out.

    y = float(((sum over groups, in order, of acc_g * s_g) * sa) * 2^-7) in
    fp64 (acc_g the exact int32 group sums)."""
    qa = np.ascontiguousarray(qa, np.int8)
    sa = np.ascontiguousarray(sa, np.float32)
    qw = np.ascontiguousarray(qw, np.int8)
    s = np.ascontiguousarray(s, np.uint16)
    M, K = qa.shape
    N = qw.shape[0]
    y = np.empty((M, N), np.float32)
    _load().orc_gemm_g128(_p(qa), _p(sa), _i64(M), _i64(K), _p(qw), _p(s), _i64(N), _p(y))
    return y


def rot_quant_rows(x: np.ndarray):
    """O18: fwht128 of each 128-block of fp32 rows, then per-row int8 quant."""
    x = np.ascontiguousarray(x, np.float32)
    M, K = x.shape
    q = np.empty((M, K), np.int8)
    s = np.empty((M,), np.float32)
    _load().orc_rot_quant_rows_f32(_p(x), _i64(M), _i64(K), _p(q), _p(s))
    return q, s


def moe_rot_forward(x_bf16, ids, w, w13, s13, w2, s2, shared=None, debug: bool = False):
    """O19: routed int8 MoE with the experts on the rotated grid (g128 bf16).

    "Qwen3.6-35B-A3B IQ8R - radiance container", Experts and Activations rows:
    experts int8 on the rotated grid with a bf16 scale per row and 128 of K,
    reading the trunk quantiser's codes; the routed order of the ATOM pull
    request's fused_moe_triton.py bullet.  w13 [E, 2I, H] int8 with s13 bf16
    [E, 2I, H/128]; w2 [E, H, I] with s2 [E, H, I/128]; ``shared`` fp32
    [T, H] (the shared expert's output) is added to the fp32 combine.
    """
    x_bf16 = np.ascontiguousarray(x_bf16, np.uint16)
    ids = np.ascontiguousarray(ids, np.int32)
    w = np.ascontiguousarray(w, np.float32)
    w13 = np.ascontiguousarray(w13, np.int8)
    s13 = np.ascontiguousarray(s13, np.uint16)
    w2 = np.ascontiguousarray(w2, np.int8)
    s2 = np.ascontiguousarray(s2, np.uint16)
    T, H = x_bf16.shape
    k = ids.shape[1]
    E, I2, _ = w13.shape
    I = I2 // 2
    assert w2.shape == (E, H, I) and s13.shape == (E, I2, H // 128) and s2.shape == (E, H, I // 128)
    sh = None if shared is None else np.ascontiguousarray(shared, np.float32)
    out = np.empty((T, H), np.uint16)
    dbg = None
    if debug:
        R = T * k
        dbg = dict(qx=np.empty((T, H), np.int8), sx=np.empty((T,), np.float32),
                   act=np.empty((R, I), np.float32), qa=np.empty((R, I), np.int8),
                   sa2=np.empty((R,), np.float32), y2=np.empty((R, H), np.float32))
    g = (lambda name: _p(dbg[name])) if debug else (lambda name: ctypes.c_void_p(0))
    _load().orc_moe_rot_forward(_p(x_bf16), _p(ids), _p(w), _p(w13), _p(s13), _p(w2), _p(s2),
                                _i64(T), _i64(H), _i64(E), _i64(I), _i64(k), _p(sh), _p(out),
                                g("qx"), g("sx"), g("act"), g("qa"), g("sa2"), g("y2"))
    return (out, dbg) if debug else out


def shared_expert(x_bf16, wgu, su8, s2, wd, sd, debug: bool = False):
    """O20: the shared expert in the Hadamard domain, fp32 out [T, H].

    "Qwen3.6-35B-A3B IQ8R - radiance container", Experts row and recipe:
    gate/up as the trunk's linears (g256: wgu [2Is, H] int8, su8 [2Is, H/256],
    s2 bf16 [2Is], rows 2i = gate_i), down g128 bf16 (wd [H, Is], sd [H, Is/128]).
    """
    x_bf16 = np.ascontiguousarray(x_bf16, np.uint16)
    T, H = x_bf16.shape
    I2 = wgu.shape[0]
    Is = I2 // 2
    args = [np.ascontiguousarray(a, dt) for a, dt in ((wgu, np.int8), (su8, np.uint8),
                                                     (s2, np.uint16), (wd, np.int8),
                                                     (sd, np.uint16))]
    assert args[0].shape == (I2, H) and args[3].shape == (H, Is)
    y = np.empty((T, H), np.float32)
    act = np.empty((T, Is), np.float32) if debug else None
    _load().orc_shared_expert(_p(x_bf16), _i64(T), _i64(H), _i64(Is), *[_p(a) for a in args],
                              _p(y), _p(act))
    return (y, act) if debug else y


def router_gate_bf16(x_bf16, wg_bf16) -> np.ndarray:
    """O21: router logits from the bf16 gate: fp64 sums of exact products,
    rounded once to fp32.  "[gfx1151] Online INT8 W8A8 ..." (ATOM pull
    request), intro: the router gate stays BF16."""
    x_bf16 = np.ascontiguousarray(x_bf16, np.uint16)
    wg_bf16 = np.ascontiguousarray(wg_bf16, np.uint16)
    T, H = x_bf16.shape
    E = wg_bf16.shape[0]
    out = np.empty((T, E), np.float32)
    _load().orc_router_gate_bf16(_p(x_bf16), _p(wg_bf16), _i64(T), _i64(H), _i64(E), _p(out))
    return out


def gemm_g256(qa, sa, qw, su8, s2, return_tsum: bool = False):
    """O13: rotated-domain GEMM with per-256 u8 group scales and a bf16 row scale.

    y[m, n] = bf16(float(sum_g su8[n,g] * acc_g * sa[m] * s2[n] * 2^-7)), the
    group sum exact in int64 and the product in fp64.
    """
    qa = np.ascontiguousarray(qa, np.int8)
    sa = np.ascontiguousarray(sa, np.float32)
    qw = np.ascontiguousarray(qw, np.int8)
    su8 = np.ascontiguousarray(su8, np.uint8)
    s2 = np.ascontiguousarray(s2, np.uint16)
    M, K = qa.shape
    N = qw.shape[0]
    y = np.empty((M, N), np.uint16)
    ts = np.empty((M, N), np.int64) if return_tsum else None
    _load().orc_gemm_g256(_p(qa), _p(sa), _i64(M), _i64(K), _p(qw), _p(su8), _p(s2), _i64(N),
                          _p(y), _p(ts))
    return (y, ts) if return_tsum else y


def gemm_g256_points(qa, sa, qw, su8, s2, ms, ns):
    """O13 at selected outputs; returns (y bf16 [P], tsum int64 [P])."""
    qa = np.ascontiguousarray(qa, np.int8)
    sa = np.ascontiguousarray(sa, np.float32)
    qw = np.ascontiguousarray(qw, np.int8)
    su8 = np.ascontiguousarray(su8, np.uint8)
    s2 = np.ascontiguousarray(s2, np.uint16)
    ms = np.ascontiguousarray(ms, np.int64)
    ns = np.ascontiguousarray(ns, np.int64)
    K = qa.shape[1]
    P = ms.size
    y = np.empty((P,), np.uint16)
    ts = np.empty((P,), np.int64)
    _load().orc_gemm_g256_points(_p(qa), _p(sa), _i64(K), _p(qw), _p(su8), _p(s2), _p(ms),
                                 _p(ns), _i64(P), _p(y), _p(ts))
    return y, ts
