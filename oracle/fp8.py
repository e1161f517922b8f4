"""FP8 (e4m3fn) and FP16 page encodings (test oracle).

Follows "Minima-KV" (twodots.gr), section "Recent, Anchor and Stale": recent
pages stay in FP8, anchor pages (the initial attention sinks among them) keep
higher fidelity.  "Show HN: Vantage-V-AI", quick-start and benchmark table,
names a dynamic FP8 streaming mode and a lossless 16-bit mode.

Readings where the pages are silent:
  * FP8 flavour: OCP e4m3fn (exponent bias 7, no infinities, one NaN code
    per sign, largest finite 448).  Stored code = the nearest finite e4m3fn
    value to float32(x / s), ties to the even code, saturating at +-448, with
    s a static per-cache scale (1.0 by default).  Dequantised value = s * v.
  * Anchor (sink) pages are IEEE float16, rounded to nearest even from the
    input (float16 input is stored verbatim).
  * Dynamic FP8 (the "dynamic FP8 streaming mode" of Show HN: Vantage-V-AI,
    core architecture and benchmark table): the scale is not fixed per cache
    but taken from the data, one per (token, KV head) for keys and one for
    values: s = float32(amax / 448) with amax = max |x| over the head's D
    elements (float32 division); codes e4m3fn(float32(x / s)) as above; an
    all-zero vector has s = 0 and codes 0.  Dequantised value = s * v.

The e4m3fn table is built by enumerating the format's definition, not by
calling a conversion routine.
"""
from __future__ import annotations

import numpy as np


def e4m3fn_value(code: int) -> float:
    """Value of one e4m3fn byte (NaN for 0x7F / 0xFF)."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# finite non-negative values, indexed by code 0x00..0x7E (increasing)
E4M3_POS = np.array([e4m3fn_value(c) for c in range(0x7F)], dtype=np.float64)
E4M3_MAX = 448.0


def e4m3fn_encode(v: np.ndarray) -> np.ndarray:
    """Nearest e4m3fn code (ties to even code), saturating, for float values."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(E4M3_POS, a, side="left")          # first table value >= a
    hi = np.minimum(hi, len(E4M3_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - E4M3_POS[lo]
    dhi = E4M3_POS[hi] - a
    exact = E4M3_POS[hi] == a
    pick_hi = exact | (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(v), code | np.uint8(0x80), code).astype(np.uint8)


def e4m3fn_decode(codes: np.ndarray) -> np.ndarray:
    table = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def fp8_encode_input(x: np.ndarray, scale: float) -> np.ndarray:
    """Stored code of each input value: e4m3fn(float32(x / s))."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    with np.errstate(over="ignore"):
        return e4m3fn_encode(x32 / np.float32(scale))


def fp8_dequantize(codes: np.ndarray, scale: float) -> np.ndarray:
    return np.float64(np.float32(scale)) * e4m3fn_decode(codes)


def fp8_dynamic_encode(x: np.ndarray):
    """Dynamic FP8 of vectors along the last axis: (codes uint8 [..., D], scales float32 [...])."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    s = (amax / np.float32(448.0)).astype(np.float32)            # float32 division
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    with np.errstate(over="ignore"):
        codes = e4m3fn_encode(x32 / safe[..., None])
    codes = np.where((s > 0)[..., None], codes, np.uint8(0)).astype(np.uint8)
    return codes, s


def fp8_dynamic_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    return np.asarray(scales, dtype=np.float32).astype(np.float64)[..., None] * e4m3fn_decode(codes)


def f16_encode_input(bits: np.ndarray, dtype: int) -> np.ndarray:
    """float16 bit patterns of each input value (F16 = 0, BF16 = 1)."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == 0:
        return bits.copy()
    x32 = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    with np.errstate(over="ignore"):
        return x32.astype(np.float16).view(np.uint16)


def f16_value(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)
