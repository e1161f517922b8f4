"""Lossless bfloat16 page tier: exponent / sign+mantissa split (test oracle).

Follows "ExANS komprimerer KV-cache og gør AI-svar hurtigere på H100 GPU"
(ainews.dk), sections "Kort" and "Begynder" and the paragraphs after them:
each BF16 value is split into two streams, one holding the exponent field and
one holding the sign and the mantissa; values are processed per group of a
physical KV block (K and V apart), with a centre of the exponents computed per
group; the exponent stream is then entropy coded ("a modified ANS", not
specified further).

Readings where the page is silent (this module is the definition the GPU path
is checked against):
  * Group = one 16-token unit of one KV head's K (or V) tile of a page: the
    centre is per (block, head) rather than per block, so that one wave holds
    every value it is computed from.
  * Centre c = floor(mean of the group's exponent fields that are not 0); c = 0
    when every field is 0 (zeros and subnormals).
  * Exponent stream: a fixed-width 4-bit code per value (the page's ANS variant
    is not specified; a fixed width keeps every value addressable by the decode
    lanes, which read only the attended pages): code = e - c + 11 for
    c - 11 <= e <= c + 3, else the escape code 15 and the exponent byte goes to
    an exception list.
  * Sign+mantissa stream: one byte per value, (sign << 7) | mantissa.
  * Layout of a group's slot (32 D + 16 bytes, D = head_dim):
        [16-byte header: centre, mode, 2 zero bytes, exception count (uint32
         little endian), 8 zero bytes]
        mode 0 (coded):   [sign+mantissa bytes: 16 D][codes: 8 D][exceptions][zero fill]
        mode 1 (raw):     [the 16 D bfloat16 values, little endian]
    Keys are stored token-major ([16][D]) and values dimension-major ([D][16]),
    as in the fp8 and fp16 tiles; codes pack two per byte in the same order
    (element 2i in the low nibble of byte i).  Exceptions are listed in the
    order of (decode lane, position in the lane) with, for head_dim D and
    W = D/4 dimensions per lane group:
        keys:   lane = (d // W) * 16 + t,            position = d % W
        values: lane = (t // 4) * 16 + (d % 16),     position = (d // 16) * 4 + t % 4
    The group is coded when its exceptions fit the slot (at most 8 D of them),
    else stored raw.
  * A page of this tier holds Bs / 16 such groups per (K or V, head), in unit
    order: tile = [group of unit 0][group of unit 1]...; page = [K tiles of
    heads 0..Hkv-1][V tiles of heads 0..Hkv-1].  The slot is as large as the raw
    values plus the header, so any input fits; the decode reads only the
    header, the two streams and the exceptions of a coded group.
"""
from __future__ import annotations

import numpy as np

HEADER = 16
ESCAPE = 15
LOW = 11          # code of e == c is LOW; codes 0..14 cover c - 11 .. c + 3
HIGH = 3


def slot_bytes(dim: int) -> int:
    """Bytes of one group's slot (16 tokens of one head, K or V)."""
    return 32 * dim + HEADER


def split(bits: np.ndarray):
    """(exponent field, sign+mantissa byte) of bfloat16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    exp = ((b >> 7) & 0xFF).astype(np.uint8)
    sm = (((b >> 8) & 0x80) | (b & 0x7F)).astype(np.uint8)
    return exp, sm


def join(exp: np.ndarray, sm: np.ndarray) -> np.ndarray:
    """Inverse of split."""
    e = np.asarray(exp, dtype=np.uint32)
    s = np.asarray(sm, dtype=np.uint32)
    return (((s & 0x80) << 8) | (e << 7) | (s & 0x7F)).astype(np.uint16)


def centre(exp: np.ndarray) -> int:
    """floor(mean of the nonzero exponent fields); 0 when there is none."""
    e = np.asarray(exp, dtype=np.int64).ravel()
    nz = e[e != 0]
    if nz.size == 0:
        return 0
    return int(nz.sum() // nz.size)


def codes(exp: np.ndarray, c: int) -> np.ndarray:
    """4-bit exponent codes: e - c + 11 inside [c - 11, c + 3], else 15 (escape)."""
    e = np.asarray(exp, dtype=np.int64)
    inside = (e >= c - LOW) & (e <= c + HIGH)
    return np.where(inside, e - c + LOW, ESCAPE).astype(np.uint8)


def lane_order(dim: int, which: str) -> np.ndarray:
    """For every element of a [16][D] group (token-major index t * D + d), its rank in the
    (decode lane, position in the lane) order of the exception list."""
    t, d = np.meshgrid(np.arange(16), np.arange(dim), indexing="ij")
    w = dim // 4
    if which == "k":
        lane, pos, per = (d // w) * 16 + t, d % w, w
    else:
        lane, pos, per = (t // 4) * 16 + (d % 16), (d // 16) * 4 + t % 4, dim // 4
    key = lane * per + pos
    return key.ravel()


def stored_order(x: np.ndarray, which: str) -> np.ndarray:
    """A [16][D] group in its stored order: keys token-major, values dimension-major."""
    return np.ascontiguousarray(x if which == "k" else x.T).ravel()


def encode_group(bits: np.ndarray, which: str) -> np.ndarray:
    """Slot bytes of one group: bits [16][D] bfloat16 patterns (token, dimension)."""
    bits = np.asarray(bits, dtype=np.uint16)
    t, dim = bits.shape
    if t != 16 or dim % 64:
        raise ValueError("a group is 16 tokens of a head dim that is a multiple of 64")
    exp, sm = split(bits)
    c = centre(exp)
    cd = codes(exp, c)
    esc = cd == ESCAPE
    n_exc = int(esc.sum())
    out = np.zeros(slot_bytes(dim), dtype=np.uint8)
    out[0] = c
    if n_exc > 8 * dim:
        out[1] = 1
        out[HEADER:HEADER + 32 * dim] = stored_order(bits, which).astype("<u2").view(np.uint8)
        return out
    out[4:8] = np.array([n_exc], dtype="<u4").view(np.uint8)
    o = HEADER
    out[o:o + 16 * dim] = stored_order(sm, which)
    o += 16 * dim
    cs = stored_order(cd, which)
    out[o:o + 8 * dim] = cs[0::2] | (cs[1::2] << 4)
    o += 8 * dim
    rank = lane_order(dim, which)                     # per token-major element
    sel = np.nonzero(esc.ravel())[0]
    exc = exp.ravel()[sel[np.argsort(rank[sel], kind="stable")]]
    out[o:o + n_exc] = exc
    return out


def decode_group(slot: np.ndarray, dim: int, which: str) -> np.ndarray:
    """Inverse of encode_group: slot bytes -> bits [16][D]."""
    s = np.asarray(slot, dtype=np.uint8)
    c, mode = int(s[0]), int(s[1])
    if mode == 1:
        raw = s[HEADER:HEADER + 32 * dim].view("<u2").astype(np.uint16)
        return raw.reshape(16, dim) if which == "k" else raw.reshape(dim, 16).T.copy()
    n_exc = int(s[4:8].view("<u4")[0])
    o = HEADER
    sm_s = s[o:o + 16 * dim]
    o += 16 * dim
    packed = s[o:o + 8 * dim]
    o += 8 * dim
    cs = np.empty(16 * dim, dtype=np.uint8)
    cs[0::2] = packed & 0xF
    cs[1::2] = packed >> 4
    exc = s[o:o + n_exc]

    def unstore(a):
        return a.reshape(16, dim) if which == "k" else a.reshape(dim, 16).T

    sm = unstore(sm_s)
    cd = unstore(cs).astype(np.int64)
    exp = (cd + c - LOW).astype(np.int64)
    esc = cd == ESCAPE
    if int(esc.sum()) != n_exc:
        raise ValueError("exception count does not match the escape codes")
    rank = lane_order(dim, which)
    sel = np.nonzero(esc.ravel())[0]
    flat = exp.ravel()
    flat[sel[np.argsort(rank[sel], kind="stable")]] = exc
    return join(flat.reshape(16, dim).astype(np.uint8), sm)


def tile(bits: np.ndarray, which: str) -> np.ndarray:
    """Tile bytes of one head: bits [Bs][D] -> Bs/16 group slots in unit order."""
    bits = np.asarray(bits, dtype=np.uint16)
    bs = bits.shape[0]
    if bs % 16:
        raise ValueError("block size must be a multiple of 16")
    return np.concatenate([encode_group(bits[16 * u:16 * u + 16], which) for u in range(bs // 16)])


def read_bytes(slot: np.ndarray, dim: int) -> int:
    """Bytes a decode reads from a group: the header and, coded, the two streams and the
    exceptions; raw, the values."""
    s = np.asarray(slot, dtype=np.uint8)
    if s[1] == 1:
        return HEADER + 32 * dim
    return HEADER + 24 * dim + int(s[4:8].view("<u4")[0])
