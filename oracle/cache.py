"""Paged, tiered cache contents for one (layer, sequence) (test oracle).

Follows "Minima-KV" (twodots.gr): pages are the unit of storage and of format
("Recent, Anchor and Stale" tiers); compressed pages stay addressable in the
request; no dense copy is kept.  "Show HN: Vantage-V-AI", core architecture:
per-tensor gamma, attention-sink retention in the block-chunked cache.

Readings where the pages are silent:
  * Page p covers tokens [p*Bs, (p+1)*Bs).  When an append brings the length
    to L', a NEW page p takes the sink format if p < ceil(S / Bs); else the
    recent format if R > 0 and its token range meets [L' - R, L'); else the
    ternary format.  A page keeps the format it was first written in.
  * A ternary page is written by one append only (its tokens share that
    append's gamma); appending into a partly filled ternary page is an error.
    So is appending into a partly filled lossless page (its groups' exponent
    centres cover all 16 tokens of a unit); lossless pages take bfloat16 input.
  * "Per tensor" gamma = one gamma per (layer, sequence, K or V, append call),
    over that call's ternary-routed tokens (all heads and dimensions).
  * Page bytes: [K tile of head 0..Hkv-1][V tile of head 0..Hkv-1]; ternary
    key tiles token-major, ternary value tiles chunked per 16-token unit (see
    ternary.v_tile); fp8 and fp16 value tiles are [D][Bs] arrays, key tiles
    [Bs][D].  With dynamic FP8 each FP8 tile is followed by its Bs float32
    scales in token order.

Retiering ("Minima-KV", tiers in "Recent, Anchor and Stale"; the evaluated
profile runs with dynamic retiering, "quality" section): recent pages leave
the FP8 tier for the packed tier once they are out of the recent window.
Readings where the page is silent:
  * At length L a page p is retiered when it is in FP8, is not a sink page
    (p >= ceil(S / Bs)) and lies wholly before the window: (p + 1) * Bs <= L - R.
    Such a page is full.  Sink pages and pages already packed are untouched.
  * Its source is what the page holds: x = s * v, the dequantised FP8 values
    (s the cache's static scale, or the token's dynamic scale; the original
    16-bit input is gone; no dense copy is kept).
  * gamma is per (page, K or V): mean(|x|) over the page's Bs * Hkv * D
    elements, as float64 rounded to float32 (the per-tensor absmean with the
    page as the tensor).  Codes are RoundClip(x / (gamma + eps), -1, 1) with x
    taken in float32 (exact when s is a power of two) and the float32 quotient.
  * The page's FP8 bytes are replaced, not kept beside the packed copy.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Sequence, Tuple

import numpy as np

from . import fp8 as _fp8
from . import lossless as _ll
from . import ternary as _t

TERNARY2 = 0
FP8E4M3 = 1
F16 = 2
LOSSLESS = 3      # bfloat16 kept exactly, exponent / sign+mantissa split (lossless.py)


class AlignError(ValueError):
    pass


@dataclasses.dataclass
class CacheSpec:
    n_kv_heads: int
    head_dim: int
    block_size: int
    sink_tokens: int = 4
    sink_format: int = TERNARY2
    recent_tokens: int = 0
    recent_format: int = FP8E4M3
    eps: float = 1e-5
    fp8_scale: float = 1.0
    fp8_dynamic: bool = False      # FP8 pages carry a scale per (token, KV head) (fp8.fp8_dynamic_encode)


def new_page_format(spec: CacheSpec, page: int, new_len: int) -> int:
    """Format of a page first written by an append that ends at length new_len."""
    bs = spec.block_size
    if page < -(-spec.sink_tokens // bs):
        return spec.sink_format
    lo, hi = page * bs, (page + 1) * bs
    if spec.recent_tokens > 0 and lo < new_len and hi > new_len - spec.recent_tokens:
        return spec.recent_format
    return TERNARY2


@dataclasses.dataclass
class EncodedSequence:
    """Everything the cache holds for one (layer, sequence)."""
    length: int
    page_format: List[int]                # per page
    token_format: np.ndarray              # [T] int8
    token_call: np.ndarray                # [T] index of the append call that wrote it
    gamma: List[Tuple[np.float32, np.float32]]  # per append call: (gamma_K, gamma_V); nan if none
    k_code: np.ndarray                    # [T, Hkv, D] int8 ternary codes (0 where not ternary)
    v_code: np.ndarray
    k_fp8: np.ndarray                     # [T, Hkv, D] uint8 (0 where not fp8)
    v_fp8: np.ndarray
    k_f16: np.ndarray                     # [T, Hkv, D] uint16 (0 where not fp16)
    v_f16: np.ndarray
    k_hat: np.ndarray                     # [T, Hkv, D] float64 dequantised
    v_hat: np.ndarray
    k_lossless: np.ndarray = None         # [T, Hkv, D] uint16 bfloat16 bits kept exactly (0 elsewhere)
    v_lossless: np.ndarray = None
    k_fp8_scale: np.ndarray = None        # [T, Hkv] float32 dynamic FP8 scales (0 where not fp8)
    v_fp8_scale: np.ndarray = None
    # pages converted from FP8 by retier(): page -> (gamma_K, gamma_V) of that page
    page_gamma: Dict[int, Tuple[np.float32, np.float32]] = dataclasses.field(default_factory=dict)


def encode_sequence(spec: CacheSpec, k_bits: np.ndarray, v_bits: np.ndarray, dtype: int,
                    calls: Sequence[Tuple[int, int]],
                    gamma_override: Sequence[Tuple[float, float]] = None) -> EncodedSequence:
    """Encode one (layer, sequence) appended by ``calls`` = [(t0, n), ...] in order.

    k_bits / v_bits: [T, Hkv, D] raw 16-bit patterns of the whole sequence.
    gamma_override: per call, a (gamma_K, gamma_V) to quantise with instead of
    the computed one (used to check codes bit-exactly against a gamma read back
    from the device, whose float32 rounding may differ by one ulp).
    """
    T = k_bits.shape[0]
    bs = spec.block_size
    n_pages = -(-T // bs)
    page_format = [-1] * n_pages
    length = 0
    tok_fmt = np.full(T, -1, dtype=np.int8)
    tok_call = np.full(T, -1, dtype=np.int32)
    gammas = []
    kx = _t.values16(k_bits, dtype)
    vx = _t.values16(v_bits, dtype)
    shape = k_bits.shape
    out = {name: np.zeros(shape, dt) for name, dt in
           (("k_code", np.int8), ("v_code", np.int8), ("k_fp8", np.uint8), ("v_fp8", np.uint8),
            ("k_f16", np.uint16), ("v_f16", np.uint16), ("k_hat", np.float64), ("v_hat", np.float64))}
    out["k_fp8_scale"] = np.zeros(shape[:2], np.float32)
    out["v_fp8_scale"] = np.zeros(shape[:2], np.float32)
    out["k_lossless"] = np.zeros(shape, np.uint16)
    out["v_lossless"] = np.zeros(shape, np.uint16)
    for ci, (t0, n) in enumerate(calls):
        if t0 != length:
            raise ValueError("appends must be contiguous")
        new_len = t0 + n
        if t0 % bs and page_format[t0 // bs] in (TERNARY2, LOSSLESS):
            raise AlignError("append into a partly filled ternary or lossless page")
        for p in range(-(-t0 // bs), -(-new_len // bs)):
            page_format[p] = new_page_format(spec, p, new_len)
        for t in range(t0, new_len):
            tok_fmt[t] = page_format[t // bs]
            tok_call[t] = ci
        tern = np.nonzero(tok_fmt[t0:new_len] == TERNARY2)[0] + t0
        gk = gv = np.float32(np.nan)
        if tern.size:
            if gamma_override is not None:
                gk, gv = np.float32(gamma_override[ci][0]), np.float32(gamma_override[ci][1])
            else:
                gk = _t.absmean_gamma(kx[tern])
                gv = _t.absmean_gamma(vx[tern])
            for src, g, code, hat in ((kx, gk, "k_code", "k_hat"), (vx, gv, "v_code", "v_hat")):
                c = _t.ternary_codes(src[tern], g, spec.eps)
                out[code][tern] = c
                out[hat][tern] = _t.dequantize(c, g)
        gammas.append((gk, gv))
        f8 = np.nonzero(tok_fmt[t0:new_len] == FP8E4M3)[0] + t0
        if f8.size:
            for src, code, hat in ((kx, "k_fp8", "k_hat"), (vx, "v_fp8", "v_hat")):
                if spec.fp8_dynamic:
                    c, sc = _fp8.fp8_dynamic_encode(src[f8])
                    out[code][f8] = c
                    out[code + "_scale"][f8] = sc
                    out[hat][f8] = _fp8.fp8_dynamic_dequantize(c, sc)
                else:
                    c = _fp8.fp8_encode_input(src[f8], spec.fp8_scale)
                    out[code][f8] = c
                    out[hat][f8] = _fp8.fp8_dequantize(c, spec.fp8_scale)
        ls = np.nonzero(tok_fmt[t0:new_len] == LOSSLESS)[0] + t0
        if ls.size:
            if dtype != _t.BF16:
                raise ValueError("the lossless tier holds bfloat16 input")
            for bits, code, hat, src in ((k_bits, "k_lossless", "k_hat", kx), (v_bits, "v_lossless", "v_hat", vx)):
                out[code][ls] = bits[ls]
                out[hat][ls] = src[ls]          # exact: the values themselves
        f16 = np.nonzero(tok_fmt[t0:new_len] == F16)[0] + t0
        if f16.size:
            for bits, code, hat in ((k_bits, "k_f16", "k_hat"), (v_bits, "v_f16", "v_hat")):
                c = _fp8.f16_encode_input(bits[f16], dtype)
                out[code][f16] = c
                out[hat][f16] = _fp8.f16_value(c)
        length = new_len
    return EncodedSequence(length, page_format, tok_fmt, tok_call, gammas, **out)


def retier_pages(spec: CacheSpec, enc: EncodedSequence, length: int = None) -> List[int]:
    """Pages that retiering at ``length`` (default: the sequence's length) converts."""
    L = enc.length if length is None else length
    if L > enc.length:
        raise ValueError("length beyond the sequence")
    bs = spec.block_size
    first = -(-spec.sink_tokens // bs)
    if spec.recent_tokens <= 0:
        return []
    return [p for p, f in enumerate(enc.page_format)
            if f == FP8E4M3 and p >= first and (p + 1) * bs <= L - spec.recent_tokens]


def retier(spec: CacheSpec, enc: EncodedSequence, length: int = None,
           gamma_override: Dict[int, Tuple[float, float]] = None) -> EncodedSequence:
    """A copy of ``enc`` with every page of retier_pages(spec, enc, length) re-encoded
    as a ternary page from its FP8 values.

    gamma_override: page -> (gamma_K, gamma_V) to quantise with instead of the
    computed one (to check codes bit-exactly against a gamma read from the device).
    """
    out = dataclasses.replace(
        enc, page_format=list(enc.page_format), token_format=enc.token_format.copy(),
        k_code=enc.k_code.copy(), v_code=enc.v_code.copy(), k_fp8=enc.k_fp8.copy(),
        v_fp8=enc.v_fp8.copy(), k_hat=enc.k_hat.copy(), v_hat=enc.v_hat.copy(),
        k_fp8_scale=enc.k_fp8_scale.copy(), v_fp8_scale=enc.v_fp8_scale.copy(),
        page_gamma=dict(enc.page_gamma))
    bs = spec.block_size
    for p in retier_pages(spec, enc, length):
        t = slice(p * bs, (p + 1) * bs)
        gammas = []
        for which in ("k", "v"):
            if spec.fp8_dynamic:
                x = _fp8.fp8_dynamic_dequantize(getattr(out, which + "_fp8")[t], getattr(out, which + "_fp8_scale")[t])
            else:
                x = _fp8.fp8_dequantize(getattr(out, which + "_fp8")[t], spec.fp8_scale)
            if gamma_override is not None:
                g = np.float32(gamma_override[p][which == "v"])
            else:
                g = _t.absmean_gamma(x)
            c = _t.ternary_codes(x, g, spec.eps)
            getattr(out, which + "_code")[t] = c
            getattr(out, which + "_hat")[t] = _t.dequantize(c, g)
            getattr(out, which + "_fp8")[t] = 0
            getattr(out, which + "_fp8_scale")[t] = 0
            gammas.append(g)
        out.page_format[p] = TERNARY2
        out.token_format[t] = TERNARY2
        out.page_gamma[p] = (gammas[0], gammas[1])
    return out


def evict_pages(spec: CacheSpec, length: int, window: int) -> List[int]:
    """Pages bounded-memory eviction frees at length L for window W (sorted).

    "Show HN: Vantage-V-AI", quick start (max_active_tokens bounds the active
    window, sink_tokens are kept) and core architecture (bounded-memory
    streaming cache with attention-sink retention).  Reading: a page is freed
    when it is not a sink page (p >= ceil(S / Bs)) and holds no token of the
    window, i.e. it ends at or before L - W: (p + 1) * Bs <= L - W.  Its tokens
    are gone for good; a later decode may only attend windows W' <= W (measured
    from a length >= L).  W = -1 (the whole context) frees nothing.
    """
    if window < 0:
        return []
    bs = spec.block_size
    first = -(-spec.sink_tokens // bs)
    last = (length - window) // bs if length > window else 0   # pages [first, last) end by L - W
    return list(range(first, max(first, last)))


def page_tiles(spec: CacheSpec, enc: EncodedSequence, page: int) -> np.ndarray:
    """Expected bytes of one page ([K tiles][V tiles]) for a page filled to the end.

    Token slots of a ternary page past the sequence length hold code 0.
    """
    bs, hkv, dim = spec.block_size, spec.n_kv_heads, spec.head_dim
    fmt = enc.page_format[page]
    lo = page * bs
    hi = min(lo + bs, enc.length)
    parts = []
    for which in ("k", "v"):
        for h in range(hkv):
            if fmt == TERNARY2:
                c = np.zeros((bs, dim), dtype=np.int8)
                c[: hi - lo] = getattr(enc, which + "_code")[lo:hi, h]
                parts.append((_t.k_tile(c) if which == "k" else _t.v_tile(c)).ravel())
            elif fmt == FP8E4M3:
                c = np.zeros((bs, dim), dtype=np.uint8)
                c[: hi - lo] = getattr(enc, which + "_fp8")[lo:hi, h]
                parts.append((c if which == "k" else c.T.copy()).ravel())
                if spec.fp8_dynamic:   # then the tile's Bs float32 scales, token order
                    sc = np.zeros(bs, dtype="<f4")
                    sc[: hi - lo] = getattr(enc, which + "_fp8_scale")[lo:hi, h]
                    parts.append(sc.view(np.uint8))
            elif fmt == LOSSLESS:   # token slots past the length hold the bits 0
                c = np.zeros((bs, dim), dtype=np.uint16)
                c[: hi - lo] = getattr(enc, which + "_lossless")[lo:hi, h]
                parts.append(_ll.tile(c, which))
            else:
                c = np.zeros((bs, dim), dtype=np.uint16)
                c[: hi - lo] = getattr(enc, which + "_f16")[lo:hi, h]
                parts.append((c if which == "k" else c.T.copy()).ravel().view(np.uint8))
    return np.concatenate(parts)


def page_bytes(spec: CacheSpec, fmt: int) -> int:
    """Bytes of one page of a format (K and V, every head)."""
    if fmt == LOSSLESS:
        return 2 * spec.n_kv_heads * (spec.block_size // 16) * _ll.slot_bytes(spec.head_dim)
    per_elem = {TERNARY2: 0.25, FP8E4M3: 1, F16: 2}[fmt]
    extra = 4 * spec.block_size if fmt == FP8E4M3 and spec.fp8_dynamic else 0   # scales per tile
    return int(2 * spec.n_kv_heads * (spec.block_size * spec.head_dim * per_elem + extra))


def stored_bytes(spec: CacheSpec, page_formats: Sequence[int]) -> int:
    """Bytes held by a set of pages, counting one float32 gamma per ternary page for K and V."""
    total = 0
    for f in page_formats:
        total += page_bytes(spec, f) + (8 if f == TERNARY2 else 0)
    return total


def storage_ratio_vs_f16(spec: CacheSpec, page_formats: Sequence[int]) -> float:
    """FP16 bytes of the same tokens divided by the stored bytes (full pages)."""
    f16 = len(page_formats) * page_bytes(spec, F16)
    return f16 / stored_bytes(spec, page_formats)
