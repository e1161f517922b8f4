"""Vectorised reading of device pages back into per-token arrays (test code).

The GPU parity tests read every page of a (layer, sequence) back from the
device and compare what it holds with the oracle's encoding of the same
tokens.  The oracle's own tile functions (oracle.ternary.k_tile, v_tile,
v_tile_codes) spell the layouts out element by element and are far too slow
for hundreds of thousands of pages, so this module decodes whole arrays of
pages at once with numpy shifts and reshapes.  It is written from the layout
text of include/vk.h, not from the oracle, and tests/test_page_codec.py pins
it to the oracle's tile functions on random tiles before any GPU test relies
on it.

Layouts (one page: [K tile of head 0..Hkv-1][V tile of head 0..Hkv-1]):
  * ternary key tile: [Bs][D/4] bytes, element 4j+i of a token row at bits
    2i of byte j, stored as code + 1;
  * ternary value tile: per 16-token unit 64 chunks of D/16 bytes; chunk
    4c+g holds tokens 4g..4g+3 of the unit for the dimensions 16j+c.  The
    chunk read as one little-endian integer holds token 4g+r, dimension 16j+c
    at bit value_bit(r, j): head_dim 128 -> two 32-bit words, word r//2 with
    token r even in its low and odd in its high half, dimension at 2j inside
    the half; head_dim 64 -> one word, token r at byte (r%2)*2 + r//2,
    dimension at 2j inside the byte; head_dim 256 -> four 32-bit words, the
    dimensions with j < 8 in words 0 and 1 as head_dim 128 places them, those
    with j >= 8 in words 2 and 3 at 2(j - 8);
  * fp8 / fp16 tiles: keys [Bs][D], values [D][Bs]; dynamic FP8 tiles end
    with Bs float32 token scales.
  * lossless tiles: per 16-token unit a slot of 32 D + 16 bytes: a 16-byte
    header (byte 0 the exponent centre c, byte 1 the mode, bytes 4..7 the
    exception count), then either (mode 1) the raw bfloat16 values or
    (mode 0) one sign+mantissa byte per value, 4-bit exponent codes two per
    byte (value e - c + 11, 15 = look the exponent up in the exception list)
    and the exception list, values in the stored order (keys [16][D], values
    [D][16]); the exception list runs over decode lanes in order and, within
    a lane, over its positions: keys of dim d, token t sit in lane
    (d // (D/4)) * 16 + t at position d % (D/4); values in lane
    (t // 4) * 16 + d % 16 at position (d // 16) * 4 + t % 4.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

TERNARY2, FP8E4M3, F16, LOSSLESS = 0, 1, 2, 3


def value_bit(r: int, j: int, dim: int) -> int:
    """Bit of token 4g+r, dimension 16j+c inside its value chunk."""
    if dim == 128:
        word, half = r // 2, r % 2
        return 32 * word + 16 * half + 2 * j
    if dim == 64:
        byte = 2 * (r % 2) + r // 2
        return 8 * byte + 2 * j
    if dim == 256:
        word, half = 2 * (j // 8) + r // 2, r % 2
        return 32 * word + 16 * half + 2 * (j % 8)
    raise ValueError("head_dim must be 64, 128 or 256")


def _fields_to_codes(u: np.ndarray) -> np.ndarray:
    if np.any(u == 3):
        raise ValueError("reserved 2-bit field 0b11 in a page")
    return u.astype(np.int8) - 1


def key_codes(tiles: np.ndarray, dim: int) -> np.ndarray:
    """[..., Bs, D/4] bytes -> [..., Bs, D] int8 codes."""
    b = np.asarray(tiles, dtype=np.uint8)
    u = (b[..., None] >> np.array([0, 2, 4, 6], dtype=np.uint8)) & 3
    return _fields_to_codes(u.reshape(b.shape[:-1] + (dim,)))


def value_codes(tiles: np.ndarray, bs: int, dim: int) -> np.ndarray:
    """[..., Bs*D/4] bytes -> [..., Bs, D] int8 codes."""
    b = np.asarray(tiles, dtype=np.uint8)
    lead = b.shape[:-1]
    nb = dim // 16                       # bytes per chunk
    units = bs // 16
    chunks = b.reshape(lead + (units, 16, 4, nb))           # [..., unit, c, g, byte]
    bits = np.array([[value_bit(r, j, dim) for j in range(nb)] for r in range(4)])
    # field of (r, j): byte bits // 8 of the chunk, shifted down by bits % 8
    u = (chunks[..., bits // 8] >> (bits % 8).astype(np.uint8)) & np.uint8(3)   # [..., unit, c, g, r, j]
    nd = len(lead)
    perm = tuple(range(nd)) + (nd, nd + 2, nd + 3, nd + 4, nd + 1)   # -> [..., unit, g, r, j, c]
    u = np.transpose(u, perm).reshape(lead + (bs, dim))      # token 16*unit + 4g + r, dim 16j + c
    return _fields_to_codes(u)


def lossless_group_bits(slot: np.ndarray, dim: int, keys: bool) -> np.ndarray:
    """One lossless slot -> its bfloat16 bits [16][D] (token, dimension)."""
    slot = np.asarray(slot, dtype=np.uint8)
    c, mode = int(slot[0]), int(slot[1])
    body = slot[16:]
    if mode == 1:
        v = body[:32 * dim].view("<u2").astype(np.uint16)
        return v.reshape(16, dim) if keys else v.reshape(dim, 16).T
    if mode != 0:
        raise ValueError("unknown lossless mode")
    n_exc = int(slot[4:8].view("<u4")[0])
    sm = body[:16 * dim]
    nib = body[16 * dim:24 * dim]
    cd = np.empty(16 * dim, dtype=np.int64)
    cd[0::2] = nib & 0xF
    cd[1::2] = nib >> 4
    to_td = (lambda a: a.reshape(16, dim)) if keys else (lambda a: a.reshape(dim, 16).T)
    sm, cd = to_td(sm), to_td(cd)
    exp = cd + c - 11
    t, d = np.meshgrid(np.arange(16), np.arange(dim), indexing="ij")
    if keys:
        lane, pos = (d // (dim // 4)) * 16 + t, d % (dim // 4)
    else:
        lane, pos = (t // 4) * 16 + d % 16, (d // 16) * 4 + t % 4
    esc = cd == 15
    if int(esc.sum()) != n_exc:
        raise ValueError("exception count does not match the escape codes")
    order = np.lexsort((pos[esc], lane[esc]))
    e_idx = np.argwhere(esc)[order]
    exp[e_idx[:, 0], e_idx[:, 1]] = body[24 * dim:24 * dim + n_exc]
    if np.any((exp < 0) | (exp > 255)):
        raise ValueError("exponent out of range")
    return (((sm.astype(np.uint32) & 0x80) << 8) | (exp.astype(np.uint32) << 7) | (sm.astype(np.uint32) & 0x7F)).astype(np.uint16)


def decode_pages(buf: np.ndarray, fmts: np.ndarray, length: int, n_kv_heads: int, head_dim: int,
                 block_size: int, fp8_dynamic: bool = False, chunk: int = 512) -> Dict[str, np.ndarray]:
    """Per-token contents of every page of one (layer, sequence).

    buf: [n_pages, stride] bytes as read from the device (page j in row j);
    fmts: [n_pages] formats.  Returns arrays shaped like the oracle's encoding
    ([T, Hkv, D], zero where a token is not in that format, T = length) plus
    "k_pad" / "v_pad": the ternary codes of token slots past `length` in the
    last page (the pages hold code 0 there).
    """
    bs, hkv, dim = block_size, n_kv_heads, head_dim
    n_pages = len(fmts)
    T = n_pages * bs
    out = {
        "k_code": np.zeros((T, hkv, dim), np.int8), "v_code": np.zeros((T, hkv, dim), np.int8),
        "k_fp8": np.zeros((T, hkv, dim), np.uint8), "v_fp8": np.zeros((T, hkv, dim), np.uint8),
        "k_f16": np.zeros((T, hkv, dim), np.uint16), "v_f16": np.zeros((T, hkv, dim), np.uint16),
        "k_fp8_scale": np.zeros((T, hkv), np.float32), "v_fp8_scale": np.zeros((T, hkv), np.float32),
        "k_lossless": np.zeros((T, hkv, dim), np.uint16), "v_lossless": np.zeros((T, hkv, dim), np.uint16),
    }
    by_page = {k: a.reshape((n_pages, bs) + a.shape[1:]) for k, a in out.items()}
    fmts = np.asarray(fmts)
    slot = 32 * dim + 16
    for p in np.nonzero(fmts == LOSSLESS)[0]:
        tb = (bs // 16) * slot
        for w, which in ((0, "k"), (1, "v")):
            for h in range(hkv):
                base = (w * hkv + h) * tb
                for u in range(bs // 16):
                    g = lossless_group_bits(buf[p, base + u * slot:base + (u + 1) * slot], dim, which == "k")
                    by_page[which + "_lossless"][p, 16 * u:16 * u + 16, h] = g
    for f in (TERNARY2, FP8E4M3, F16):
        idx_all = np.nonzero(fmts == f)[0]
        for c0 in range(0, idx_all.size, chunk):
            idx = idx_all[c0:c0 + chunk]
            n = idx.size
            if f == TERNARY2:
                tb = bs * dim // 4
                raw = buf[idx, :2 * hkv * tb].reshape(n, 2, hkv, tb)
                kc = key_codes(raw[:, 0].reshape(n, hkv, bs, dim // 4), dim)      # [n, hkv, bs, dim]
                vc = value_codes(raw[:, 1], bs, dim)
                by_page["k_code"][idx] = kc.transpose(0, 2, 1, 3)
                by_page["v_code"][idx] = vc.transpose(0, 2, 1, 3)
            else:
                es = 1 if f == FP8E4M3 else 2
                tb = bs * dim * es
                stride = tb + (4 * bs if (f == FP8E4M3 and fp8_dynamic) else 0)
                raw = buf[idx, :2 * hkv * stride].reshape(n, 2, hkv, stride)
                dt = np.uint8 if es == 1 else np.dtype("<u2")
                name = "fp8" if f == FP8E4M3 else "f16"
                k = np.ascontiguousarray(raw[:, 0, :, :tb]).view(dt).reshape(n, hkv, bs, dim)
                v = np.ascontiguousarray(raw[:, 1, :, :tb]).view(dt).reshape(n, hkv, dim, bs)
                by_page["k_" + name][idx] = k.transpose(0, 2, 1, 3)
                by_page["v_" + name][idx] = v.transpose(0, 3, 1, 2)
                if stride != tb:
                    for w, which in ((0, "k"), (1, "v")):
                        sc = np.ascontiguousarray(raw[:, w, :, tb:]).view("<f4").reshape(n, hkv, bs)
                        by_page[which + "_fp8_scale"][idx] = sc.transpose(0, 2, 1)
    res = {k: a[:length] for k, a in out.items()}
    last_tern = n_pages > 0 and fmts[-1] == TERNARY2
    res["k_pad"] = out["k_code"][length:] if last_tern else np.zeros((0, hkv, dim), np.int8)
    res["v_pad"] = out["v_code"][length:] if last_tern else np.zeros((0, hkv, dim), np.int8)
    return res
