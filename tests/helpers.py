"""Shared helpers of the GPU parity tests: moving identical input bytes to the
device, reading results back, and the error metric."""
from __future__ import annotations

import numpy as np
import torch

from oracle import formats as F


def to_dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bf16 bit patterns -> a bfloat16 GPU tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def to_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_f64(t: torch.Tensor) -> np.ndarray:
    return F.bf16_to_f64(bf16_bits(t))


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of ||got - ref||_inf / ||ref||_inf (rows = last axis)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(num / den)) if num.size else 0.0


def sorted_ids(rng: np.random.Generator, n_entries: int, k: int, n_valid: int | None = None) -> np.ndarray:
    """k ids in ascending order drawn without replacement from [0, n_entries),
    the first n_valid of them real and the rest -1 (the layout top-k returns)."""
    n_valid = k if n_valid is None else n_valid
    n_valid = min(n_valid, n_entries)
    out = np.full(k, -1, dtype=np.int32)
    out[:n_valid] = np.sort(rng.choice(n_entries, size=n_valid, replace=False))
    return out
