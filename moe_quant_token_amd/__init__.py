"""Online INT8 W8A8 (dense, routed MoE, fwht128 / g256) on MI355X.

Thin ctypes binding of ``libw8a8.so`` (hand-written gfx950 HIP kernels behind
the C ABI of ``include/w8a8.h``).  The functions here only marshal torch
tensors (device memory) and the current HIP stream into the C calls; every
step of the computation runs in the library's kernels.  There is no CPU or
PyTorch fallback: if the library is missing or the device is not gfx950 the
calls raise.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libw8a8.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "w8a8.h")

_lib = None

W8A8_OK = 0
STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported shape", -3: "misaligned",
          -4: "workspace too small", -5: "HIP error", -6: "unsupported device"}


class W8A8Error(RuntimeError):
    def __init__(self, fn: str, status: int, hip_err: int = 0):
        self.status = status
        msg = f"{fn} failed: {STATUS.get(status, status)}"
        if status == -5:
            msg += f" (hipError {hip_err})"
        super().__init__(msg)


_i64, _i32, _sz, _vp = ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p


class MoeDebug(ctypes.Structure):
    _fields_ = [("qx", _vp), ("sx", _vp), ("acc1", _vp), ("act", _vp), ("qa", _vp),
                ("sa2", _vp), ("acc2", _vp)]


class MlpDebug(ctypes.Structure):
    _fields_ = [("act", _vp), ("qa", _vp), ("sa", _vp)]


class SharedDebug(ctypes.Structure):
    _fields_ = [("act", _vp), ("qa", _vp), ("sa", _vp)]


_SIGS = {
    "w8a8_status_string": ([_i32], ctypes.c_char_p),
    "w8a8_last_hip_error": ([], _i32),
    "w8a8_version": ([], _i32),
    "w8a8_stream_read": ([_vp, _i64, _i64, _vp, _vp], _i32),
    "quant_per_token_i8": ([_vp, _i32, _i64, _i64, _i64, _vp, _i64, _vp, _vp], _i32),
    "gemm_w8a8_workspace_bytes": ([_i64, _i64, _i64], _sz),
    "gemm_w8a8": ([_vp, _vp, _i64, _i64, _i64, _vp, _vp, _i64, _i64, _vp, _i64, _vp, _sz, _vp],
                  _i32),
    "gemm_w8a8_i32acc": ([_vp, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _vp, _sz, _vp],
                         _i32),
    "linear_w8a8_workspace_bytes": ([_i64, _i64, _i64], _sz),
    "linear_w8a8": ([_vp, _i64, _i64, _i64, _vp, _vp, _i64, _i64, _vp, _i64, _vp, _sz, _vp],
                    _i32),
    "w8a8_pack_weights": ([_vp, _i64, _i64, _i64, _vp, _vp], _i32),
    "gemm_w8a8_packed": ([_vp, _vp, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _i64, _vp, _sz, _vp],
                         _i32),
    "gemm_w8a8_packed_i32acc": ([_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _sz, _vp],
                                _i32),
    "linear_w8a8_packed": ([_vp, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _i64, _vp, _sz, _vp],
                           _i32),
    "linear_w8a8_packed_noalloc": ([_vp, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _i64, _vp],
                                   _i32),
    "mlp_w8a8_workspace_bytes": ([_i64, _i64, _i64, _i64], _sz),
    "mlp_w8a8_packed": ([_vp, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _i64, _vp, _i64, _vp,
                         _sz, ctypes.POINTER(MlpDebug), _vp], _i32),
    "kv_quant_i8": ([_vp, _i64, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp], _i32),
    "moe_w8a8_workspace_bytes": ([_i64, _i64, _i64, _i64, _i32], _sz),
    "moe_w8a8_forward": ([_vp, _vp, _i64, _i64, _i64, _i64, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                          _vp, _vp, _sz, ctypes.POINTER(MoeDebug), _vp], _i32),
    "moe_w8a8_forward_packed": ([_vp, _vp, _i64, _i64, _i64, _i64, _i32, _vp, _vp, _vp, _vp,
                                 _vp, _vp, _vp, _vp, _sz, ctypes.POINTER(MoeDebug), _vp], _i32),
    "fwht128_quant": ([_vp, _i64, _i64, _i64, _vp, _i64, _vp, _vp], _i32),
    "fwht128_weight_prep_g256": ([_vp, _i64, _i64, _vp, _vp, _vp, _vp], _i32),
    "gemm_w8a8_g256_workspace_bytes": ([_i64, _i64, _i64], _sz),
    "linear_w8a8_g256_workspace_bytes": ([_i64, _i64, _i64], _sz),
    "linear_w8a8_g256_packed": ([_vp, _i64, _i64, _i64, _vp, _vp, _vp, _i64, _vp, _i64, _vp,
                                 _sz, _vp], _i32),
    "gemm_w8a8_g256_packed": ([_vp, _vp, _i64, _i64, _vp, _vp, _vp, _i64, _vp, _i64, _vp, _sz,
                               _vp], _i32),
    "gemm_w8a8_g256": ([_vp, _vp, _i64, _i64, _vp, _vp, _vp, _i64, _vp, _i64, _vp, _sz, _vp],
                       _i32),
    "fwht128_weight_prep_g128": ([_vp, _i64, _i64, _vp, _vp, _vp], _i32),
    "router_gate_bf16": ([_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp], _i32),
    "moe_w8a8_rot_forward_packed": ([_vp, _vp, _i64, _i64, _i64, _i64, _i32, _vp, _vp, _vp, _vp,
                                     _vp, _vp, _vp, _vp, _vp, _sz, ctypes.POINTER(MoeDebug),
                                     _vp], _i32),
    "shared_expert_w8a8_rot_workspace_bytes": ([_i64, _i64, _i64], _sz),
    "moe_w8a8_rot_shared_workspace_bytes": ([_i64, _i64, _i64, _i64, _i32, _i64], _sz),
    "moe_w8a8_rot_shared_forward_packed": ([_vp, _vp, _i64, _i64, _i64, _i64, _i32, _vp, _vp,
                                            _vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                            _vp, _vp, _sz, ctypes.POINTER(MoeDebug), _vp], _i32),
    "shared_expert_w8a8_rot_packed": ([_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       _sz, ctypes.POINTER(SharedDebug), _vp], _i32),
}


def header_functions() -> list[str]:
    """Names of the functions include/w8a8.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(",
                                 text, flags=re.M)))


def lib() -> ctypes.CDLL:
    """Load libw8a8.so (built by ``moe_quant_token_amd.build``); raise if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run moe_quant_token_amd/build.py "
                               "(or __graft_entry__.build()) first")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check(fn: str, status: int):
    if status != W8A8_OK:
        raise W8A8Error(fn, status, lib().w8a8_last_hip_error())


def _ptr(t: torch.Tensor | None):
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _req(t: torch.Tensor, dtype, name: str):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name}: expected a device tensor")
    if t.stride(-1) != 1:
        raise ValueError(f"{name}: last dimension must be contiguous")


def _workspace(nbytes: int, device, ws: torch.Tensor | None):
    if nbytes == 0:
        return ws, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


# --------------------------------------------------------------------------
def quant_per_token_i8(x: torch.Tensor, q: torch.Tensor | None = None,
                       s: torch.Tensor | None = None):
    """Per-row symmetric int8 quantisation of bf16 or fp32 rows -> (q int8, s fp32)."""
    dt = {torch.bfloat16: 0, torch.float32: 1}.get(x.dtype)
    if dt is None:
        raise TypeError("quant_per_token_i8: x must be bfloat16 or float32")
    _req(x, x.dtype, "x")
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.int8, device=x.device) if q is None else q
    s = torch.empty((M,), dtype=torch.float32, device=x.device) if s is None else s
    _check("quant_per_token_i8",
           lib().quant_per_token_i8(_ptr(x), dt, M, K, x.stride(0), _ptr(q), q.stride(0),
                                    _ptr(s), _stream(x.device)))
    return q, s


def gemm_w8a8(qa, sa, qw, sw, y: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """y[m, n] = bf16((float(sum_k qa[m,k] qw[n,k]) * sa[m]) * sw[n])."""
    _req(qa, torch.int8, "qa")
    _req(qw, torch.int8, "qw")
    M, K = qa.shape
    N = qw.shape[0]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=qa.device) if y is None else y
    ws, wsb = _workspace(0, qa.device, ws)  # row-major weights: no workspace
    _check("gemm_w8a8",
           lib().gemm_w8a8(_ptr(qa), _ptr(sa), M, K, qa.stride(0), _ptr(qw), _ptr(sw), N,
                           qw.stride(0), _ptr(y), y.stride(0), _ptr(ws), wsb,
                           _stream(qa.device)))
    return y


def gemm_w8a8_i32acc(qa, qw, acc: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """The exact int32 sums of gemm_w8a8 (same kernels, int32 store)."""
    _req(qa, torch.int8, "qa")
    _req(qw, torch.int8, "qw")
    M, K = qa.shape
    N = qw.shape[0]
    acc = torch.empty((M, N), dtype=torch.int32, device=qa.device) if acc is None else acc
    ws, wsb = _workspace(0, qa.device, ws)  # row-major weights: no workspace
    _check("gemm_w8a8_i32acc",
           lib().gemm_w8a8_i32acc(_ptr(qa), M, K, qa.stride(0), _ptr(qw), N, qw.stride(0),
                                  _ptr(acc), acc.stride(0), _ptr(ws), wsb, _stream(qa.device)))
    return acc


def gemm_w8a8_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().gemm_w8a8_workspace_bytes(M, N, K))


def linear_w8a8_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().linear_w8a8_workspace_bytes(M, N, K))


def linear_w8a8(x, qw, sw, y: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """bf16 x -> per-token int8 -> W8A8 GEMM + epilogue -> bf16 y."""
    _req(x, torch.bfloat16, "x")
    _req(qw, torch.int8, "qw")
    M, K = x.shape
    N = qw.shape[0]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device) if y is None else y
    ws, wsb = _workspace(linear_w8a8_workspace_bytes(M, N, K), x.device, ws)
    _check("linear_w8a8",
           lib().linear_w8a8(_ptr(x), M, K, x.stride(0), _ptr(qw), _ptr(sw), N, qw.stride(0),
                             _ptr(y), y.stride(0), _ptr(ws), wsb, _stream(x.device)))
    return y


def pack_weights(qw: torch.Tensor) -> torch.Tensor:
    """Row-major int8 [N, K] weights -> the packed MFMA tile layout (same bytes, permuted)."""
    _req(qw, torch.int8, "qw")
    N, K = qw.shape
    out = torch.empty((N * K,), dtype=torch.int8, device=qw.device)
    _check("w8a8_pack_weights",
           lib().w8a8_pack_weights(_ptr(qw), N, K, qw.stride(0), _ptr(out), _stream(qw.device)))
    return out


def gemm_w8a8_packed(qa, sa, qw_packed, sw, N: int, y: torch.Tensor | None = None,
                     ws: torch.Tensor | None = None):
    """gemm_w8a8 with packed weights (``pack_weights``); N = output channels."""
    _req(qa, torch.int8, "qa")
    M, K = qa.shape
    y = torch.empty((M, N), dtype=torch.bfloat16, device=qa.device) if y is None else y
    ws, wsb = _workspace(lib().gemm_w8a8_workspace_bytes(M, N, K), qa.device, ws)
    _check("gemm_w8a8_packed",
           lib().gemm_w8a8_packed(_ptr(qa), _ptr(sa), M, K, qa.stride(0), _ptr(qw_packed),
                                  _ptr(sw), N, _ptr(y), y.stride(0), _ptr(ws), wsb,
                                  _stream(qa.device)))
    return y


def gemm_w8a8_packed_i32acc(qa, qw_packed, N: int, acc: torch.Tensor | None = None,
                            ws: torch.Tensor | None = None):
    _req(qa, torch.int8, "qa")
    M, K = qa.shape
    acc = torch.empty((M, N), dtype=torch.int32, device=qa.device) if acc is None else acc
    ws, wsb = _workspace(lib().gemm_w8a8_workspace_bytes(M, N, K), qa.device, ws)
    _check("gemm_w8a8_packed_i32acc",
           lib().gemm_w8a8_packed_i32acc(_ptr(qa), M, K, qa.stride(0), _ptr(qw_packed), N,
                                         _ptr(acc), acc.stride(0), _ptr(ws), wsb,
                                         _stream(qa.device)))
    return acc


def linear_w8a8_packed(x, qw_packed, sw, N: int, y: torch.Tensor | None = None,
                       ws: torch.Tensor | None = None):
    _req(x, torch.bfloat16, "x")
    M, K = x.shape
    y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device) if y is None else y
    ws, wsb = _workspace(linear_w8a8_workspace_bytes(M, N, K), x.device, ws)
    _check("linear_w8a8_packed",
           lib().linear_w8a8_packed(_ptr(x), M, K, x.stride(0), _ptr(qw_packed), _ptr(sw), N,
                                    _ptr(y), y.stride(0), _ptr(ws), wsb, _stream(x.device)))
    return y


NOALLOC_SCRATCH_BYTES = 32 << 20


def linear_w8a8_packed_noalloc(x, qw_packed, sw, N: int, y: torch.Tensor | None = None):
    """linear_w8a8_packed with the library's own static scratch (no workspace)."""
    _req(x, torch.bfloat16, "x")
    M, K = x.shape
    y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device) if y is None else y
    _check("linear_w8a8_packed_noalloc",
           lib().linear_w8a8_packed_noalloc(_ptr(x), M, K, x.stride(0), _ptr(qw_packed),
                                            _ptr(sw), N, _ptr(y), y.stride(0),
                                            _stream(x.device)))
    return y


def mlp_w8a8_workspace_bytes(M: int, K: int, I: int, N: int) -> int:
    return int(lib().mlp_w8a8_workspace_bytes(M, K, I, N))


def mlp_w8a8_packed(x, wgu_packed, sgu, wd_packed, sd, I: int, N: int,
                    y: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                    debug: bool = False):
    """Dense W8A8 MLP block: gate_up (interleaved rows) -> SiLU(gate)*up ->
    per-token requant -> down, weights from ``pack_weights``.  Returns y
    (bf16 [M, N]) and, with ``debug``, a dict of intermediates."""
    _req(x, torch.bfloat16, "x")
    M, K = x.shape
    dev = x.device
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if y is None else y
    ws, wsb = _workspace(mlp_w8a8_workspace_bytes(M, K, I, N), dev, ws)
    dbg_t = dbg_p = None
    if debug:
        dbg_t = dict(act=torch.empty((M, I), dtype=torch.float32, device=dev),
                     qa=torch.empty((M, I), dtype=torch.int8, device=dev),
                     sa=torch.empty((M,), dtype=torch.float32, device=dev))
        dbg_p = ctypes.pointer(MlpDebug(**{k: v.data_ptr() for k, v in dbg_t.items()}))
    _check("mlp_w8a8_packed",
           lib().mlp_w8a8_packed(_ptr(x), M, K, x.stride(0), _ptr(wgu_packed), _ptr(sgu), I,
                                 _ptr(wd_packed), _ptr(sd), N, _ptr(y), y.stride(0), _ptr(ws),
                                 wsb, dbg_p, _stream(dev)))
    return (y, dbg_t) if debug else y


def kv_quant_i8(x, q_cache: torch.Tensor | None = None, s_cache: torch.Tensor | None = None,
                slots: torch.Tensor | None = None):
    """int8 KV-cache quant with an f16 scale per token and head.

    ``x`` bf16 [T, Hk, D]; token t goes to cache row ``slots[t]`` (row t
    without slots).  Returns (q_cache int8 [rows, Hk, D], s_cache f16
    [rows, Hk])."""
    _req(x, torch.bfloat16, "x")
    T, Hk, D = x.shape
    if x.stride(1) != D:
        raise ValueError("x: heads must be contiguous within a token")
    if q_cache is None:
        q_cache = torch.zeros((T, Hk, D), dtype=torch.int8, device=x.device)
    if s_cache is None:
        s_cache = torch.zeros((q_cache.shape[0], Hk), dtype=torch.float16, device=x.device)
    if slots is not None and slots.dtype != torch.int32:
        raise TypeError("slots: expected int32")
    _check("kv_quant_i8",
           lib().kv_quant_i8(_ptr(x), T, Hk, D, x.stride(0), _ptr(slots), q_cache.shape[0],
                             _ptr(q_cache), q_cache.stride(0), _ptr(s_cache), s_cache.stride(0),
                             _stream(x.device)))
    return q_cache, s_cache


def stream_read(buf: torch.Tensor, chunk: int, sink: torch.Tensor) -> None:
    """Measurement helper: read ``buf`` (any dtype, contiguous) once, one
    workgroup per ``chunk`` bytes (see w8a8_stream_read); ``sink`` int32 [1]."""
    if not buf.is_contiguous():
        raise ValueError("buf: must be contiguous")
    _req(sink, torch.int32, "sink")
    _check("w8a8_stream_read",
           lib().w8a8_stream_read(_ptr(buf), buf.numel() * buf.element_size(), chunk,
                                  _ptr(sink), _stream(buf.device)))


def moe_w8a8_workspace_bytes(T: int, H: int, E: int, I: int, topk: int) -> int:
    return int(lib().moe_w8a8_workspace_bytes(T, H, E, I, topk))


def pack_moe_weights(w13: torch.Tensor, w2: torch.Tensor):
    """Pack [E, 2I, H] and [E, H, I] int8 expert weights into the tile layout."""
    E, I2, H = w13.shape
    return (pack_weights(w13.reshape(E * I2, H)).reshape(E, I2, H),
            pack_weights(w2.reshape(E * H, w2.shape[2])).reshape(w2.shape))


def moe_w8a8_forward(x, logits, w13, s13, w2, s2, topk: int, topk_ids=None, topk_w=None,
                     out=None, ws=None, debug: bool = False, packed: bool = False):
    """Routed int8 MoE layer.  ``logits`` None -> ``topk_ids``/``topk_w`` are inputs.

    ``packed``: w13/w2 come from ``pack_moe_weights`` (shapes unchanged).
    Returns ``out`` (bf16 [T, H]) and, with ``debug``, a dict of intermediates.
    """
    _req(x, torch.bfloat16, "x")
    T, H = x.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    dev = x.device
    if topk_ids is None:
        topk_ids = torch.empty((T, topk), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, topk), dtype=torch.float32, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev) if out is None else out
    ws, wsb = _workspace(moe_w8a8_workspace_bytes(T, H, E, I, topk), dev, ws)
    dbg_t = None
    dbg_p = None
    if debug:
        R = T * topk
        dbg_t = dict(qx=torch.empty((T, H), dtype=torch.int8, device=dev),
                     sx=torch.empty((T,), dtype=torch.float32, device=dev),
                     acc1=torch.empty((R, I2), dtype=torch.int32, device=dev),
                     act=torch.empty((R, I), dtype=torch.float32, device=dev),
                     qa=torch.empty((R, I), dtype=torch.int8, device=dev),
                     sa2=torch.empty((R,), dtype=torch.float32, device=dev),
                     acc2=torch.empty((R, H), dtype=torch.int32, device=dev))
        dbg_p = ctypes.pointer(MoeDebug(**{k: v.data_ptr() for k, v in dbg_t.items()}))
    fn = lib().moe_w8a8_forward_packed if packed else lib().moe_w8a8_forward
    _check("moe_w8a8_forward", fn(_ptr(x), _ptr(logits), T, H, E, I, topk, _ptr(w13), _ptr(s13),
                                  _ptr(w2), _ptr(s2), _ptr(topk_ids), _ptr(topk_w), _ptr(out),
                                  _ptr(ws), wsb, dbg_p, _stream(dev)))
    if debug:
        return out, topk_ids, topk_w, dbg_t
    return out, topk_ids, topk_w


def fwht128_quant(x, q: torch.Tensor | None = None, s: torch.Tensor | None = None):
    """fwht128 of each 128-block of every bf16 row, then per-row int8 quant."""
    _req(x, torch.bfloat16, "x")
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.int8, device=x.device) if q is None else q
    s = torch.empty((M,), dtype=torch.float32, device=x.device) if s is None else s
    _check("fwht128_quant",
           lib().fwht128_quant(_ptr(x), M, K, x.stride(0), _ptr(q), q.stride(0), _ptr(s),
                               _stream(x.device)))
    return q, s


def fwht128_weight_prep_g256(W):
    """Rotated int8 weights with u8 scales per 256 of K under a bf16 row scale."""
    _req(W, torch.float32, "W")
    W = W.contiguous()
    N, K = W.shape
    qw = torch.empty((N, K), dtype=torch.int8, device=W.device)
    su8 = torch.empty((N, K // 256), dtype=torch.uint8, device=W.device)
    s2 = torch.empty((N,), dtype=torch.bfloat16, device=W.device)
    _check("fwht128_weight_prep_g256",
           lib().fwht128_weight_prep_g256(_ptr(W), N, K, _ptr(qw), _ptr(su8), _ptr(s2),
                                          _stream(W.device)))
    return qw, su8, s2


def gemm_w8a8_g256(qa, sa, qw, su8, s2, y: torch.Tensor | None = None,
                   ws: torch.Tensor | None = None, packed: bool = False):
    """Hadamard-domain GEMM with per-256 u8 group scales and a bf16 row scale.

    With ``packed`` the codes ``qw`` are in the packed tile layout
    (``pack_weights`` of the prepared codes); ``N`` is then ``su8.shape[0]``."""
    _req(qa, torch.int8, "qa")
    _req(qw, torch.int8, "qw")
    M, K = qa.shape
    N = su8.shape[0]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=qa.device) if y is None else y
    ws, wsb = _workspace(lib().gemm_w8a8_g256_workspace_bytes(M, N, K), qa.device, ws)
    fn = "gemm_w8a8_g256_packed" if packed else "gemm_w8a8_g256"
    _check(fn, getattr(lib(), fn)(_ptr(qa), _ptr(sa), M, K, _ptr(qw), _ptr(su8), _ptr(s2), N,
                                  _ptr(y), y.stride(0), _ptr(ws), wsb, _stream(qa.device)))
    return y


def gemm_w8a8_g256_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().gemm_w8a8_g256_workspace_bytes(M, N, K))


def linear_w8a8_g256_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().linear_w8a8_g256_workspace_bytes(M, N, K))


def linear_w8a8_g256_packed(x, qw_packed, su8, s2, y: torch.Tensor | None = None,
                            ws: torch.Tensor | None = None):
    """bf16 x -> fwht128 + per-token int8 -> g256 GEMM on packed codes -> bf16 y."""
    _req(x, torch.bfloat16, "x")
    _req(qw_packed, torch.int8, "qw_packed")
    M, K = x.shape
    N = su8.shape[0]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device) if y is None else y
    ws, wsb = _workspace(lib().linear_w8a8_g256_workspace_bytes(M, N, K), x.device, ws)
    _check("linear_w8a8_g256_packed",
           lib().linear_w8a8_g256_packed(_ptr(x), M, K, x.stride(0), _ptr(qw_packed), _ptr(su8),
                                         _ptr(s2), N, _ptr(y), y.stride(0), _ptr(ws), wsb,
                                         _stream(x.device)))
    return y


def fwht128_weight_prep_g128(W):
    """Rotated int8 weights with a bf16 scale per row per 128 of K.

    Returns (qw int8 [N, K] row-major, s bf16 [N, K/128])."""
    _req(W, torch.float32, "W")
    W = W.contiguous()
    N, K = W.shape
    qw = torch.empty((N, K), dtype=torch.int8, device=W.device)
    s = torch.empty((N, K // 128), dtype=torch.bfloat16, device=W.device)
    _check("fwht128_weight_prep_g128",
           lib().fwht128_weight_prep_g128(_ptr(W), N, K, _ptr(qw), _ptr(s), _stream(W.device)))
    return qw, s


def router_gate_bf16(x, wg, logits: torch.Tensor | None = None):
    """fp32 router logits [T, E] = x [T, H] . wg [E, H]^T, bf16 operands."""
    _req(x, torch.bfloat16, "x")
    _req(wg, torch.bfloat16, "wg")
    T, H = x.shape
    E = wg.shape[0]
    if not wg.is_contiguous():
        raise ValueError("wg: expected a contiguous [E, H] tensor")
    if logits is None:
        logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    _check("router_gate_bf16",
           lib().router_gate_bf16(_ptr(x), T, H, x.stride(0), _ptr(wg), E, _ptr(logits),
                                  logits.stride(0), _stream(x.device)))
    return logits


def moe_w8a8_rot_forward(x, logits, w13_packed, s13, w2_packed, s2, topk: int, shared=None,
                         topk_ids=None, topk_w=None, out=None, ws=None, debug: bool = False):
    """Routed MoE layer in the Hadamard domain (experts with bf16 scales per 128 of K).

    ``w13_packed`` [E, 2I, H] and ``w2_packed`` [E, H, I] are prepared codes
    (``fwht128_weight_prep_g128``) packed with ``pack_moe_weights``; ``s13``
    bf16 [E, 2I, H/128], ``s2`` bf16 [E, H, I/128]; ``shared`` fp32 [T, H]
    (the shared expert's output) or None.  Returns out, topk_ids, topk_w
    (and the intermediates qx, sx, act, qa, sa2 with ``debug``)."""
    _req(x, torch.bfloat16, "x")
    _req(s13, torch.bfloat16, "s13")
    _req(s2, torch.bfloat16, "s2")
    if not x.is_contiguous():
        raise ValueError("x: expected a contiguous [T, H] tensor")
    T, H = x.shape
    E, I2, _ = w13_packed.shape
    I = I2 // 2
    dev = x.device
    if shared is not None:
        _req(shared, torch.float32, "shared")
        if not shared.is_contiguous() or tuple(shared.shape) != (T, H):
            raise ValueError("shared: expected a contiguous fp32 [T, H] tensor")
    if topk_ids is None:
        topk_ids = torch.empty((T, topk), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, topk), dtype=torch.float32, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev) if out is None else out
    ws, wsb = _workspace(moe_w8a8_workspace_bytes(T, H, E, I, topk), dev, ws)
    dbg_t = None
    dbg_p = None
    if debug:
        R = T * topk
        dbg_t = dict(qx=torch.empty((T, H), dtype=torch.int8, device=dev),
                     sx=torch.empty((T,), dtype=torch.float32, device=dev),
                     act=torch.empty((R, I), dtype=torch.float32, device=dev),
                     qa=torch.empty((R, I), dtype=torch.int8, device=dev),
                     sa2=torch.empty((R,), dtype=torch.float32, device=dev))
        dbg_p = ctypes.pointer(MoeDebug(**{k: v.data_ptr() for k, v in dbg_t.items()}))
    _check("moe_w8a8_rot_forward_packed",
           lib().moe_w8a8_rot_forward_packed(_ptr(x), _ptr(logits), T, H, E, I, topk,
                                             _ptr(w13_packed), _ptr(s13), _ptr(w2_packed),
                                             _ptr(s2), _ptr(shared), _ptr(topk_ids),
                                             _ptr(topk_w), _ptr(out), _ptr(ws), wsb, dbg_p,
                                             _stream(dev)))
    if debug:
        return out, topk_ids, topk_w, dbg_t
    return out, topk_ids, topk_w


def moe_w8a8_rot_shared_forward(x, logits, w13_packed, s13, w2_packed, s2, topk: int,
                                shared_w, topk_ids=None, topk_w=None, out=None, ws=None,
                                debug: bool = False):
    """The Hadamard-domain MoE layer with its shared expert in one call.

    ``shared_w`` = (wgu_packed, su8, sgu, wd_packed, sd) as for
    ``shared_expert_w8a8_rot``; the rest as ``moe_w8a8_rot_forward``.  The
    result equals ``moe_w8a8_rot_forward(..., shared=shared_expert_w8a8_rot(x,
    *shared_w))``; one token runs in two launches with the shared expert
    inside them."""
    _req(x, torch.bfloat16, "x")
    _req(s13, torch.bfloat16, "s13")
    _req(s2, torch.bfloat16, "s2")
    if not x.is_contiguous():
        raise ValueError("x: expected a contiguous [T, H] tensor")
    wgu_packed, su8, sgu, wd_packed, sd = shared_w
    _req(su8, torch.uint8, "su8")
    _req(sgu, torch.bfloat16, "sgu")
    _req(sd, torch.bfloat16, "sd")
    T, H = x.shape
    E, I2, _ = w13_packed.shape
    I = I2 // 2
    Is = su8.shape[0] // 2
    dev = x.device
    if topk_ids is None:
        topk_ids = torch.empty((T, topk), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, topk), dtype=torch.float32, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev) if out is None else out
    ws, wsb = _workspace(lib().moe_w8a8_rot_shared_workspace_bytes(T, H, E, I, topk, Is), dev,
                         ws)
    dbg_t = None
    dbg_p = None
    if debug:
        R = T * topk
        dbg_t = dict(qx=torch.empty((T, H), dtype=torch.int8, device=dev),
                     sx=torch.empty((T,), dtype=torch.float32, device=dev),
                     act=torch.empty((R, I), dtype=torch.float32, device=dev),
                     qa=torch.empty((R, I), dtype=torch.int8, device=dev),
                     sa2=torch.empty((R,), dtype=torch.float32, device=dev))
        dbg_p = ctypes.pointer(MoeDebug(**{k: v.data_ptr() for k, v in dbg_t.items()}))
    _check("moe_w8a8_rot_shared_forward_packed",
           lib().moe_w8a8_rot_shared_forward_packed(
               _ptr(x), _ptr(logits), T, H, E, I, topk, _ptr(w13_packed), _ptr(s13),
               _ptr(w2_packed), _ptr(s2), Is, _ptr(wgu_packed), _ptr(su8), _ptr(sgu),
               _ptr(wd_packed), _ptr(sd), _ptr(topk_ids), _ptr(topk_w), _ptr(out), _ptr(ws),
               wsb, dbg_p, _stream(dev)))
    if debug:
        return out, topk_ids, topk_w, dbg_t
    return out, topk_ids, topk_w


def shared_expert_w8a8_rot_workspace_bytes(T: int, H: int, Is: int) -> int:
    return int(lib().shared_expert_w8a8_rot_workspace_bytes(T, H, Is))


def shared_expert_w8a8_rot(x, wgu_packed, su8, s2, wd_packed, sd, y=None, ws=None,
                           debug: bool = False):
    """The shared expert in the Hadamard domain: fp32 y [T, H].

    ``wgu_packed`` [2Is, H] (g256 codes, ``fwht128_weight_prep_g256``, packed)
    with ``su8`` [2Is, H/256] and ``s2`` bf16 [2Is]; ``wd_packed`` [H, Is]
    (g128 codes, packed) with ``sd`` bf16 [H, Is/128]."""
    _req(x, torch.bfloat16, "x")
    _req(s2, torch.bfloat16, "s2")
    _req(sd, torch.bfloat16, "sd")
    if not x.is_contiguous():
        raise ValueError("x: expected a contiguous [T, H] tensor")
    T, H = x.shape
    Is = su8.shape[0] // 2
    dev = x.device
    y = torch.empty((T, H), dtype=torch.float32, device=dev) if y is None else y
    ws, wsb = _workspace(shared_expert_w8a8_rot_workspace_bytes(T, H, Is), dev, ws)
    dbg_t = None
    dbg_p = None
    if debug:
        dbg_t = dict(act=torch.empty((T, Is), dtype=torch.float32, device=dev),
                     qa=torch.empty((T, Is), dtype=torch.int8, device=dev),
                     sa=torch.empty((T,), dtype=torch.float32, device=dev))
        dbg_p = ctypes.pointer(SharedDebug(**{k: v.data_ptr() for k, v in dbg_t.items()}))
    _check("shared_expert_w8a8_rot_packed",
           lib().shared_expert_w8a8_rot_packed(_ptr(x), T, H, Is, _ptr(wgu_packed), _ptr(su8),
                                               _ptr(s2), _ptr(wd_packed), _ptr(sd), _ptr(y),
                                               _ptr(ws), wsb, dbg_p, _stream(dev)))
    return (y, dbg_t) if debug else y
