"""Small helpers shared by the GPU parity tests (marshalling and comparison only)."""
import sys

import numpy as np
import torch

# bf16 output tolerance: |gpu - oracle| <= ATOL + RTOL * |oracle|, elementwise
ATOL = 1e-3
RTOL = 1e-2

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns (host) -> bf16 device tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def bf16_host(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> uint16 bit patterns (host)."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def assert_bf16_close(got_bits, ref_bits, what=""):
    """Tolerance check of bf16 outputs; returns the number of bit mismatches."""
    g = f32(got_bits).astype(np.float64)
    r = f32(ref_bits).astype(np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - r)
    bad = err > ATOL + RTOL * np.abs(r)
    assert not bad.any(), (f"{what}: {bad.sum()} elements out of tolerance, max abs err "
                           f"{err.max():.3e}")
    return int((np.asarray(got_bits) != np.asarray(ref_bits)).sum())


def ulp_diff_f32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in units in the last place between fp32 arrays of equal sign."""
    ai = np.ascontiguousarray(a, np.float32).view(np.int32).astype(np.int64)
    bi = np.ascontiguousarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(ai - bi)


def tie_logits(pattern, E):
    """One token's router logits with ties: at the top, everywhere, across
    the 8th slot, or in pairs."""
    lg = np.zeros((1, E), np.float32)
    if pattern == "top3":      # three-way tie at the top, the rest tied below
        lg[0, [E - 3, 9, 2]] = 1.0
    elif pattern == "all":     # every logit equal: experts 0..k-1
        lg[0, :] = 0.5
    elif pattern == "boundary":  # ten tied logits straddle the k-th slot
        lg[0, :] = np.linspace(-1.0, -2.0, E, dtype=np.float32)
        lg[0, np.arange(3, E, max(1, E // 10))[:10]] = 0.25
        lg[0, E - 1] = 3.0
    else:                      # descending values in pairs of equal logits
        lg[0, ::-1] = (np.arange(E) // 2).astype(np.float32)
    return lg
