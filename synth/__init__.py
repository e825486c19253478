"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and lays them out; it holds none of the
quantisation, GEMM, routing or transform arithmetic.  Both the oracle side and
the GPU side of a test take their inputs from here, so they see identical data.

Every tensor comes from ``numpy.random.default_rng([workload, shape, tensor
(, expert)])`` (PCG64 seeded through SeedSequence).  Tensor ids: 0 = outlier
channel indices, 1 = activation normals, 2 = outlier values, 3 = dense weight
or w13, 4 = w2, 5 = router logits.  fp32 -> bf16 uses round-to-nearest-even
(torch's conversion).

Workloads (sizes and distributions):
  W1  small linear: M=16, K=512, N=256; activations N(0,1) with 4 channels x20.
  W2  decode linear: M in {1,2,4,8}; (K,N) = (5120,17408) gate_up, (8704,5120)
      down; activations N(0,1) with round(1% K) channels x10.
  W3  prefill linear: M=4096, K=5120, N in {5120,17408}; activations as W1.
  W4  routed MoE: T in {1,64,2048}, 256 experts, top-8, hidden 2048, expert
      intermediate 512; x N(0,1); logits N(0,1) fp32.
  W5  Hadamard-domain linear: M in {1,256}, K=2048, N=8192; activations N(0,1)
      with round(1% K) channels drawn from Student-t (nu=3) x10.
  Weights are fp32 N(0, 0.02) in every workload.
"""
from __future__ import annotations

import numpy as np

T_OUTLIER_IDX, T_X, T_OUTLIER_VAL, T_W, T_W2, T_LOGITS = range(6)


def rng(key, tensor_id, *extra) -> np.random.Generator:
    return np.random.default_rng([*key, tensor_id, *extra])


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even (torch)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def activations(key, M: int, K: int, n_outliers: int, outlier_scale: float,
                heavy_tail: bool = False) -> np.ndarray:
    """bf16 activations [M, K] (uint16 bit patterns).

    N(0,1) everywhere; ``n_outliers`` channels (drawn without replacement) are
    multiplied by ``outlier_scale``.  With ``heavy_tail`` those channels hold
    Student-t (nu=3) draws instead of normals before scaling.
    """
    x = rng(key, T_X).standard_normal((M, K), dtype=np.float32)
    if n_outliers > 0:
        ch = rng(key, T_OUTLIER_IDX).choice(K, size=n_outliers, replace=False)
        if heavy_tail:
            vals = rng(key, T_OUTLIER_VAL).standard_t(3.0, size=(M, n_outliers))
            x[:, ch] = vals.astype(np.float32)
        x[:, ch] *= np.float32(outlier_scale)
    return to_bf16_bits(x)


def weights(key, N: int, K: int, std: float = 0.02, tensor_id: int = T_W) -> np.ndarray:
    """fp32 weights [N, K] ~ N(0, std)."""
    w = rng(key, tensor_id).standard_normal((N, K), dtype=np.float32)
    w *= np.float32(std)
    return w


def expert_weights(key, expert: int, rows: int, cols: int, tensor_id: int,
                   std: float = 0.02) -> np.ndarray:
    """fp32 weights of one expert [rows, cols] ~ N(0, std)."""
    w = rng(key, tensor_id, expert).standard_normal((rows, cols), dtype=np.float32)
    w *= np.float32(std)
    return w


def router_logits(key, T: int, E: int) -> np.ndarray:
    """fp32 router logits [T, E] ~ N(0, 1)."""
    return rng(key, T_LOGITS).standard_normal((T, E), dtype=np.float32)


# Workload descriptions -----------------------------------------------------

def small_linear():
    return dict(xkey=(1, 0), wkey=(1, 0), M=16, K=512, N=256, n_outliers=4,
                outlier_scale=20.0)


DECODE_SHAPES = [(5120, 17408, "gate_up"), (8704, 5120, "down")]
DECODE_M = [1, 2, 4, 8]


def decode_linear(M: int, shape_idx: int):
    K, N, name = DECODE_SHAPES[shape_idx]
    return dict(xkey=(2, shape_idx * 16 + M), wkey=(2, shape_idx), M=M, K=K, N=N, name=name,
                n_outliers=int(round(0.01 * K)), outlier_scale=10.0)


def prefill_linear(N: int):
    return dict(xkey=(3, N), wkey=(3, N), M=4096, K=5120, N=N, n_outliers=4,
                outlier_scale=20.0)


def moe(T: int):
    return dict(xkey=(4, T), wkey=(4, 0), T=T, E=256, k=8, H=2048, I=512)


def hadamard_linear(M: int):
    return dict(xkey=(5, M), wkey=(5, 0), M=M, K=2048, N=8192,
                n_outliers=int(round(0.01 * 2048)), outlier_scale=10.0)
