"""Seeded synthetic inputs for the compressed-KV decode path (host side).

This module draws the numbers both sides of every check consume; it holds no
step of the method itself. The generator is SplitMix64 (Steele, Lea and Flood,
"Fast splittable pseudorandom number generators", OOPSLA 2014): the i-th output
of a generator started at state ``key`` is ``mix64(key + (i + 1) * GOLDEN)``.
Because it is counter based, any slice of any tensor can be regenerated on the
host without producing the rest, and the device filler in ``synth/synth.hip``
implements the same definition bit for bit.

Value recipes (all exact integer arithmetic until the final cast):

* ``normal``: Irwin-Hall sum of twelve 16-bit uniforms, centred and scaled by
  2^-16 (mean 0, variance ~1). Element i consumes draws 3i, 3i+1, 3i+2; each
  draw supplies four 16-bit fields. The fp32 value is exact; the bf16 version
  rounds it to nearest even.
* ``int_uniform(a)``: an integer in [-a, a] by multiply-shift of the top 32 bits.
* ``bytes``: the low byte of each draw.
* ``pow2_e4m3(emin, emax)``: the E4M3 code of 2^e, e uniform in [emin, emax].
* ``fp8_codes``: an E4M3 code with random sign, exponent field in [4, 9] and
  random mantissa (finite, magnitudes 2^-3 .. 3.75).
* ``pos_scale``: a positive fp32 row scale (|normal| + 0.5) / 64.
"""
from __future__ import annotations

import numpy as np

from . import configs  # noqa: F401  (workload recipes live beside the generator)

MASK64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
M1 = 0xBF58476D1CE4E5B9
M2 = 0x94D049BB133111EB

# Tensor identifiers: each tensor of a workload draws from its own stream.
T_S, T_GATE, T_Q, T_QIDX, T_KIDX, T_KIDX_SCALE, T_CACHE, T_CACHE_SCALE, T_WIN, T_WIN_SCALE, T_MISC = range(11)

# Generator kinds shared with the device filler (synth.hip keeps the same numbers).
KIND_NORMAL_F32 = 0
KIND_NORMAL_BF16 = 1
KIND_INT_BF16 = 2
KIND_BYTES = 3
KIND_POW2_E4M3 = 4
KIND_FP8_CODES = 5
KIND_POS_SCALE = 6


def _mix64_np(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.uint64, copy=True)
    with np.errstate(over="ignore"):
        z ^= z >> np.uint64(30)
        z *= np.uint64(M1)
        z ^= z >> np.uint64(27)
        z *= np.uint64(M2)
        z ^= z >> np.uint64(31)
    return z


def mix64(z: int) -> int:
    """SplitMix64 output function on one Python integer."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * M1) & MASK64
    z = ((z ^ (z >> 27)) * M2) & MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, tensor: int, layer: int = 0) -> int:
    """Start state of the stream for one tensor of one layer of a workload."""
    k = mix64((seed + GOLDEN * (tensor + 1)) & MASK64)
    return mix64((k + GOLDEN * (layer + 1)) & MASK64)


def draws(key: int, idx: np.ndarray) -> np.ndarray:
    """Outputs number ``idx`` (uint64 array) of the generator started at ``key``."""
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(key) + (idx + np.uint64(1)) * np.uint64(GOLDEN)
    return _mix64_np(z)


def _index(offset: int, n: int) -> np.ndarray:
    return np.arange(offset, offset + n, dtype=np.uint64)


def normal_f32(key: int, offset: int, n: int) -> np.ndarray:
    i = _index(offset, n)
    acc = np.zeros(n, dtype=np.int64)
    for j in range(3):
        d = draws(key, i * np.uint64(3) + np.uint64(j))
        for f in range(4):
            acc += ((d >> np.uint64(16 * f)) & np.uint64(0xFFFF)).astype(np.int64)
    acc -= 6 * 65535
    return (acc.astype(np.float64) * 2.0 ** -16).astype(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the raw uint16 bits."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    r = np.where(nan, np.uint64(0x7FC0), r)
    return (r & np.uint64(0xFFFF)).astype(np.uint16)


def normal_bf16(key: int, offset: int, n: int) -> np.ndarray:
    return f32_to_bf16_bits(normal_f32(key, offset, n))


def int_uniform(key: int, offset: int, n: int, a: int) -> np.ndarray:
    d = draws(key, _index(offset, n))
    hi = d >> np.uint64(32)
    with np.errstate(over="ignore"):
        v = (hi * np.uint64(2 * a + 1)) >> np.uint64(32)
    return v.astype(np.int64) - a


def int_bf16(key: int, offset: int, n: int, a: int) -> np.ndarray:
    """Integers in [-a, a] (a <= 256) stored as bf16 bits; exact."""
    return f32_to_bf16_bits(int_uniform(key, offset, n, a).astype(np.float32))


def random_bytes(key: int, offset: int, n: int) -> np.ndarray:
    return (draws(key, _index(offset, n)) & np.uint64(0xFF)).astype(np.uint8)


def pow2_e4m3(key: int, offset: int, n: int, emin: int, emax: int) -> np.ndarray:
    """E4M3 codes of 2^e with e uniform in [emin, emax] (needs -6 <= emin, emax <= 8)."""
    d = draws(key, _index(offset, n))
    hi = d >> np.uint64(32)
    with np.errstate(over="ignore"):
        e = ((hi * np.uint64(emax - emin + 1)) >> np.uint64(32)).astype(np.int64) + emin
    return ((e + 7) << 3).astype(np.uint8)


def fp8_codes(key: int, offset: int, n: int) -> np.ndarray:
    d = draws(key, _index(offset, n))
    sign = (d >> np.uint64(63)) & np.uint64(1)
    hi = (d >> np.uint64(32)) & np.uint64(0xFFFFFFFF)
    with np.errstate(over="ignore"):
        e = ((hi * np.uint64(6)) >> np.uint64(32)) + np.uint64(4)
    m = d & np.uint64(7)
    return ((sign << np.uint64(7)) | (e << np.uint64(3)) | m).astype(np.uint8)


def pos_scale(key: int, offset: int, n: int) -> np.ndarray:
    x = normal_f32(key, offset, n)
    return ((np.abs(x) + np.float32(0.5)) / np.float32(64.0)).astype(np.float32)


def generate(kind: int, key: int, offset: int, n: int, a: int = 0, emin: int = 0, emax: int = 0) -> np.ndarray:
    """One entry point by kind number, mirroring the device filler's signature."""
    if kind == KIND_NORMAL_F32:
        return normal_f32(key, offset, n)
    if kind == KIND_NORMAL_BF16:
        return normal_bf16(key, offset, n)
    if kind == KIND_INT_BF16:
        return int_bf16(key, offset, n, a)
    if kind == KIND_BYTES:
        return random_bytes(key, offset, n)
    if kind == KIND_POW2_E4M3:
        return pow2_e4m3(key, offset, n, emin, emax)
    if kind == KIND_FP8_CODES:
        return fp8_codes(key, offset, n)
    if kind == KIND_POS_SCALE:
        return pos_scale(key, offset, n)
    raise ValueError(f"unknown generator kind {kind}")
