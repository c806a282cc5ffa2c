"""Number formats of the compressed caches, from their public definitions.

[P1] paragraph on quantisation: the attention cache is stored in fp8 ("partly
token-wise") and the indexer cache in fp4. [P3] "Three mechanisms instead of one
trick", third mechanism: FP4 values are E2M1 with one E4M3 scale per 16 channels.

Formats (OCP 8-bit floating point and OCP microscaling specifications):
* bf16: the upper half of an IEEE binary32.
* E4M3 ("E4M3FN"): sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent
  field 0 is subnormal; no infinities; S.1111.111 is NaN; largest finite 448.
* E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent field 0 is
  subnormal; magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.

Readings where the pages are silent (the encoders are not printed anywhere):
* fp8 rows: one fp32 scale per row, scale = amax / 448 (fp32 division);
  code = E4M3 nearest of x / scale, ties to even, saturating at 448.
  An all-zero row gets scale 1.
* fp4 groups: scale code = E4M3 nearest of amax / 6 (fp32 division), raised to
  the smallest subnormal if it rounds to zero while amax > 0; code = E2M1
  nearest of x / value(scale), ties to even, saturating at 6; a group whose
  scale is zero gets all-zero codes. Packing: byte j holds channel 2j in its
  low nibble and channel 2j+1 in its high nibble.
"""
from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------- bf16

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) to float64 (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 to bf16 bits, round to nearest even (NaN kept quiet)."""
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    r = np.where(np.isnan(x), np.uint64(0x7FC0), r)
    return (r & np.uint64(0xFFFF)).astype(np.uint16)


# --------------------------------------------------------------------- E4M3

def _e4m3_value(code: int) -> float:
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        mag = (m / 8.0) * 2.0 ** (1 - 7)
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
E4M3_MAX = 448.0
# finite non-negative codes in increasing order of value: 0x00 .. 0x7E
_E4M3_POS = E4M3_TABLE[:0x7F]


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def _nearest_code(mag: np.ndarray, values: np.ndarray) -> np.ndarray:
    """Index of the nearest entry of the increasing array ``values`` to each
    magnitude; ties go to the even index; beyond the last entry saturates."""
    hi = np.searchsorted(values, mag, side="left")
    hi = np.clip(hi, 1, len(values) - 1)
    lo = hi - 1
    d_lo = mag - values[lo]
    d_hi = values[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(mag >= values[-1], len(values) - 1, idx)
    idx = np.where(mag <= values[0], 0, idx)
    return idx


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float32 values to E4M3 codes: nearest, ties to even, saturating at 448.

    The distances are compared in float64, where the difference of two float32
    numbers of this range is exact, so the decision equals the exact one."""
    x = np.asarray(x, dtype=np.float32)
    xd = x.astype(np.float64)
    mag = np.abs(xd)
    idx = _nearest_code(np.where(np.isnan(mag), 0.0, mag), _E4M3_POS)
    sign = np.signbit(x).astype(np.uint8) << np.uint8(7)
    codes = (idx.astype(np.uint8) | sign).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), codes).astype(np.uint8)


def encode_fp8_rows(x: np.ndarray):
    """Rows of float32 values to (E4M3 codes uint8 [..., D], fp32 scale [...])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = (x / scale[..., None]).astype(np.float32)
    return e4m3_encode(q), scale


def decode_fp8_rows(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """E4M3 codes times the row scale, in float64 (exact)."""
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float32).astype(np.float64)[..., None]


# --------------------------------------------------------------------- E2M1

def encode_mixed_rows(x: np.ndarray, R: int):
    """[P1] mixed-precision bullet and quantisation paragraph: the rotary
    channels (the last R) stay bf16, the other channels are fp8 with one scale
    per row (token), as encode_fp8_rows over those channels alone.
    Returns (codes uint8 [..., D-R], rotary bf16 bits uint16 [..., R], scale fp32 [...])."""
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    codes, scale = encode_fp8_rows(x[..., : D - R])
    return codes, f32_to_bf16(x[..., D - R:]), scale


def decode_mixed_rows(codes: np.ndarray, rope_bits: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Rows back to float64: fp8 part value(code) * scale, then the bf16 rotary part."""
    return np.concatenate([decode_fp8_rows(codes, scale), bf16_to_f64(rope_bits)], axis=-1)


def mixed_row_bytes(codes: np.ndarray, rope_bits: np.ndarray) -> np.ndarray:
    """The stored row: the D-R codes, then the R bf16 channels little-endian."""
    rb = np.ascontiguousarray(rope_bits, dtype="<u2").view(np.uint8)
    return np.concatenate([np.asarray(codes, dtype=np.uint8), rb.reshape(rope_bits.shape[:-1] + (-1,))], axis=-1)


def fp4_row_bytes(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """An fp4 attention-cache row as stored ([P3] "Three mechanisms", third: E2M1
    values with one E4M3 scale per 16 channels, applied to the main KV): the D/2
    packed code bytes, then the D/16 scale bytes."""
    return np.concatenate([np.asarray(packed, dtype=np.uint8), np.asarray(scales, dtype=np.uint8)], axis=-1)


def decode_fp4_rows(rows: np.ndarray, D: int) -> np.ndarray:
    """Stored fp4 rows [..., D/2 + D/16] back to float64 [..., D]."""
    rows = np.asarray(rows, dtype=np.uint8)
    return decode_fp4_g16(rows[..., : D // 2], rows[..., D // 2: D // 2 + D // 16])


def _e2m1_value(code: int) -> float:
    s = (code >> 3) & 1
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        mag = (m / 2.0) * 2.0 ** (1 - 1)
    else:
        mag = (1.0 + m / 2.0) * 2.0 ** (e - 1)
    return -mag if s else mag


E2M1_TABLE = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)
E2M1_MAX = 6.0
_E2M1_POS = E2M1_TABLE[:8]


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    return E2M1_TABLE[np.asarray(codes, dtype=np.uint8) & np.uint8(0xF)]


def e2m1_encode(x: np.ndarray) -> np.ndarray:
    """float32 values to E2M1 codes (uint8 in 0..15): nearest, ties to even,
    saturating at 6; NaN is not representable and maps to code 0."""
    x = np.asarray(x, dtype=np.float32)
    mag = np.abs(x.astype(np.float64))
    idx = _nearest_code(np.where(np.isnan(mag), 0.0, mag), _E2M1_POS)
    sign = np.signbit(x).astype(np.uint8) << np.uint8(3)
    codes = (idx.astype(np.uint8) | sign).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0), codes).astype(np.uint8)


def pack_fp4(codes: np.ndarray) -> np.ndarray:
    """[..., 2n] codes -> [..., n] bytes; channel 2j low nibble, 2j+1 high."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << np.uint8(4))).astype(np.uint8)


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & np.uint8(0xF)
    out[..., 1::2] = p >> np.uint8(4)
    return out


def encode_fp4_g16(x: np.ndarray):
    """Rows of float32 values [..., Di] to (packed codes [..., Di/2],
    E4M3 scale codes [..., Di/16])."""
    x = np.asarray(x, dtype=np.float32)
    Di = x.shape[-1]
    assert Di % 16 == 0
    g = x.reshape(x.shape[:-1] + (Di // 16, 16))
    amax = np.max(np.abs(g), axis=-1)
    sc = e4m3_encode((amax / np.float32(E2M1_MAX)).astype(np.float32))
    sc = np.where((E4M3_TABLE[sc] == 0) & (amax > 0), np.uint8(0x01), sc).astype(np.uint8)
    sval = E4M3_TABLE[sc].astype(np.float32)
    safe = np.where(sval == 0, np.float32(1.0), sval).astype(np.float32)
    q = (g / safe[..., None]).astype(np.float32)
    codes = e2m1_encode(q)
    codes = np.where((sval == 0)[..., None], np.uint8(0), codes).astype(np.uint8)
    return pack_fp4(codes.reshape(x.shape)), sc


def decode_fp4_g16(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Dequantised keys in float64: E2M1(code) * E4M3(scale of its 16-group)."""
    v = e2m1_decode(unpack_fp4(packed))
    s = e4m3_decode(scales)
    Di = v.shape[-1]
    return (v.reshape(v.shape[:-1] + (Di // 16, 16)) * s[..., None]).reshape(v.shape)
