"""Ternary absmean quantisation and 2-bit packing (test oracle).

Follows "Show HN: Vantage-V-AI", section "core architecture" (the 2-bit packed
ternary bullet): keys and values are mapped to {-1, 0, +1} with a per-tensor
dynamic scale gamma = mean(|X|), and packed four elements per uint8.

Readings where that page is silent:
  * RoundClip(X / (gamma + eps), -1, 1): round to nearest, ties to even
    (numpy.rint), then clip.  eps is additive, 1e-5 by default.
  * gamma is the float64 mean of |x| rounded to float32; d = float32(gamma) +
    float32(eps) in float32; the quotient x / d is the IEEE float32 quotient.
    If d == 0 (every x is +-0 and eps == 0) every code is 0.
  * Dequantised value = gamma * code (eps only guards the division).
  * 2-bit code map: u = code + 1, so -1 -> 0b00, 0 -> 0b01, +1 -> 0b10;
    0b11 is never written.
  * Flat tensors and key page rows pack along the last axis, element 4j+i in
    bits [2i, 2i+1] of byte j (least significant first).
  * Value page tiles are stored per 16-token unit (4*D bytes each, units in
    token order).  A unit is 64 chunks of D/16 bytes; chunk 4*c + g holds the
    codes of tokens 4g..4g+3 of the unit for the dimensions 16*j + c
    (j = 0..D/16-1), read as little-endian 32-bit words:
      D = 128: word h (h = 0, 1) holds token 4g+2h in its low 16 bits and
               token 4g+2h+1 in its high 16 bits, dimension 16j+c at bits 2j;
      D = 64:  one word; its low 16 bits hold token 4g (bits 0-7) and 4g+2
               (bits 8-15), its high 16 bits token 4g+1 and 4g+3; dimension
               16j+c at bits 2j of each byte;
      D = 256: four words, two D = 128 chunks one after the other: words 0
               and 1 hold the dimensions with j < 8 as D = 128 does, words 2
               and 3 those with j >= 8 at bits 2(j - 8).
    Still four codes per byte.

All inputs are the raw 16-bit patterns of float16 or bfloat16 tensors.
"""
from __future__ import annotations

import numpy as np

F16 = 0
BF16 = 1


def values16(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Exact float64 values of float16 / bfloat16 bit patterns."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == F16:
        return bits.view(np.float16).astype(np.float64)
    if dtype == BF16:
        with np.errstate(invalid="ignore"):
            return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError("dtype must be F16 or BF16")


def absmean_gamma(x: np.ndarray) -> np.float32:
    """gamma = mean(|X|): the float64 mean of |x| rounded to float32.

    numpy's float64 sum (pairwise) stands in for the exact sum; its error is
    far below the float32 rounding of the mean.
    """
    x = np.asarray(x, dtype=np.float64).ravel()
    if x.size == 0:
        raise ValueError("gamma of an empty tensor")
    return np.float32(np.sum(np.abs(x), dtype=np.float64) / np.float64(x.size))


def divisor(gamma: np.float32, eps: float) -> np.float32:
    """d = gamma + eps, added in float32."""
    return np.float32(np.float32(gamma) + np.float32(eps))


def ternary_codes(x: np.ndarray, gamma: np.float32, eps: float) -> np.ndarray:
    """RoundClip(x / (gamma + eps), -1, 1) as int8 codes in {-1, 0, +1}."""
    d = divisor(gamma, eps)
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)  # exact for 16-bit inputs
    if d == 0:
        return np.zeros(x32.shape, dtype=np.int8)
    with np.errstate(over="ignore"):
        t = x32 / d  # IEEE float32 quotient
    return np.clip(np.rint(t), -1, 1).astype(np.int8)


def dequantize(codes: np.ndarray, gamma: np.float32) -> np.ndarray:
    """gamma * code, in float64."""
    return np.float64(np.float32(gamma)) * np.asarray(codes, dtype=np.float64)


def pack_flat(codes: np.ndarray) -> np.ndarray:
    """Four codes per byte along the last axis, least significant first."""
    q = np.asarray(codes, dtype=np.int16)
    if q.shape[-1] % 4:
        raise ValueError("last axis must be a multiple of 4")
    u = (q + 1).astype(np.uint8).reshape(q.shape[:-1] + (q.shape[-1] // 4, 4))
    return (u[..., 0] | (u[..., 1] << 2) | (u[..., 2] << 4) | (u[..., 3] << 6)).astype(np.uint8)


def unpack_flat(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_flat.  Raises if a reserved 0b11 field is present."""
    b = np.asarray(packed, dtype=np.uint8)
    u = np.stack([(b >> (2 * i)) & 3 for i in range(4)], axis=-1)
    if np.any(u == 3):
        raise ValueError("reserved 2-bit code 0b11")
    return (u.astype(np.int8) - 1).reshape(b.shape[:-1] + (b.shape[-1] * 4,))


def quantize_pack(bits: np.ndarray, dtype: int, eps: float = 1e-5):
    """The flat write side: (packed bytes, gamma) of one 16-bit tensor."""
    x = values16(bits, dtype)
    g = absmean_gamma(x)
    return pack_flat(ternary_codes(x, g, eps).ravel()), g


def k_tile(codes: np.ndarray) -> np.ndarray:
    """Key page tile of one head: codes [Bs, D] -> bytes [Bs, D/4] (token-major)."""
    return pack_flat(codes)


def _v_bit(r: int, j: int, dim: int) -> int:
    """Bit position, inside its chunk, of token 4g+r and dimension 16j+c."""
    if dim == 128:
        return 32 * (r // 2) + 16 * (r % 2) + 2 * j
    if dim == 64:
        return 16 * (r % 2) + 8 * (r // 2) + 2 * j
    if dim == 256:
        return 64 * (j // 8) + 32 * (r // 2) + 16 * (r % 2) + 2 * (j % 8)
    raise ValueError("head_dim must be 64, 128 or 256")


def v_tile(codes: np.ndarray) -> np.ndarray:
    """Value page tile of one head: codes [Bs, D] -> bytes [Bs*D/4] (chunked, see module doc)."""
    q = np.asarray(codes, dtype=np.int16)
    bs, dim = q.shape
    if bs % 16:
        raise ValueError("block size must be a multiple of 16")
    u = q + 1
    nb = dim // 16                                  # dimensions per chunk; chunk = nb bytes
    out = np.zeros((bs // 16, 64, nb), dtype=np.uint8)
    for k in range(bs // 16):
        for c in range(16):
            for g in range(4):
                val = 0                             # the chunk as one little-endian integer
                for r in range(4):
                    for j in range(nb):
                        val |= int(u[16 * k + 4 * g + r, 16 * j + c]) << _v_bit(r, j, dim)
                out[k, 4 * c + g] = np.frombuffer(val.to_bytes(nb, "little"), dtype=np.uint8)
    return out.reshape(-1)


def v_tile_codes(tile: np.ndarray, bs: int, dim: int) -> np.ndarray:
    """Inverse of v_tile: bytes [Bs*D/4] -> codes [Bs, D]."""
    b = np.asarray(tile, dtype=np.uint8).reshape(bs // 16, 64, dim // 16)
    nb = dim // 16
    out = np.zeros((bs, dim), dtype=np.int8)
    for k in range(bs // 16):
        for c in range(16):
            for g in range(4):
                val = int.from_bytes(bytes(b[k, 4 * c + g]), "little")
                for r in range(4):
                    for j in range(nb):
                        u = (val >> _v_bit(r, j, dim)) & 3
                        if u == 3:
                            raise ValueError("reserved 2-bit code 0b11")
                        out[16 * k + 4 * g + r, 16 * j + c] = u - 1
    return out
