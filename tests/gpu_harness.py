"""Shared pieces of the GPU parity tests: run a seeded workload through the
library (C ABI via the binding) and compare it with the CPU oracle.

Bars: page bytes and codes bit-exact given the device's gamma; gamma within
2^-22 relative of the oracle's; decode outputs within max-abs 2e-3 of the
oracle's float64 attention.
"""
from __future__ import annotations

import math
import sys
from typing import Dict, List, Sequence

import numpy as np
import torch

from bit_ternary_attention_amd import vk
from bit_ternary_attention_amd import workloads as wl
from oracle import attention as oa
from oracle import cache as oc
from oracle import ternary as ot

GAMMA_RTOL = 2.0 ** -22
ATTN_ATOL = 2e-3


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def spec_of(w: wl.Workload, eps=1e-5, fp8_scale=1.0, fp8_dynamic=False) -> oc.CacheSpec:
    return oc.CacheSpec(n_kv_heads=w.n_kv_heads, head_dim=w.head_dim, block_size=w.block_size,
                        sink_tokens=w.sink_tokens, sink_format=w.sink_format, recent_tokens=w.recent_tokens,
                        recent_format=w.recent_format, eps=eps, fp8_scale=fp8_scale, fp8_dynamic=bool(fp8_dynamic))


def seq_calls(w: wl.Workload, seq: int):
    return [(t0, n) for ids, t0, n in w.appends() if seq in ids]


def pages_needed(w: wl.Workload) -> List[int]:
    """Pages per format per layer that the append schedule takes (plus slack)."""
    spec = spec_of(w)
    need = [0, 0, 0]
    for s in range(w.n_seqs):
        length = 0
        for t0, n in seq_calls(w, s):
            for p in range(-(-t0 // w.block_size), -(-(t0 + n) // w.block_size)):
                need[oc.new_page_format(spec, p, t0 + n)] += 1
            length = t0 + n
    return [x + 2 for x in need]


def make_cache(w: wl.Workload, shuffle=None, eps=1e-5, fp8_scale=1.0, slack_pages=(0, 0, 0),
               max_tokens=None, decode_kernel=0, fp8_dynamic=0) -> vk.Cache:
    need = pages_needed(w)
    cfg = vk.make_config(n_layers=w.n_layers, n_kv_heads=w.n_kv_heads, n_q_heads=w.n_q_heads,
                         head_dim=w.head_dim, block_size=w.block_size, max_seqs=w.n_seqs,
                         max_tokens_per_seq=max_tokens or w.max_len, sink_tokens=w.sink_tokens, sink_format=w.sink_format,
                         recent_tokens=w.recent_tokens, recent_format=w.recent_format,
                         pages_ternary=need[0] + slack_pages[0], pages_fp8=need[1] + slack_pages[1],
                         pages_f16=need[2] + slack_pages[2], eps=eps, fp8_scale=fp8_scale,
                         page_shuffle_seed=w.page_shuffle_seed if shuffle is None else shuffle,
                         decode_kernel=decode_kernel, fp8_dynamic=int(fp8_dynamic))
    return vk.Cache(cfg)


def fill(cache: vk.Cache, w: wl.Workload) -> None:
    for ids, t0, n in w.appends():
        k, v = wl.append_inputs(w, ids, t0, n, device="cuda")
        cache.append(k, v, ids)
        del k, v
    torch.cuda.synchronize()


def host_kv(w: wl.Workload, layer: int, seq: int):
    L = w.lengths[seq]
    k = wl.to_bits(wl.kv_block(w, "k", layer, seq, 0, L, device="cuda"))
    v = wl.to_bits(wl.kv_block(w, "v", layer, seq, 0, L, device="cuda"))
    return k, v


def page_sample(n_pages: int, k: int = 6) -> List[int]:
    if n_pages <= 3 * k:
        return list(range(n_pages))
    rng = np.random.default_rng(n_pages)
    mid = rng.choice(np.arange(k, n_pages - k), size=k, replace=False)
    return sorted(set(range(k)) | set(int(x) for x in mid) | set(range(n_pages - k, n_pages)))


def read_page(cache: vk.Cache, layer: int, seq: int, p: int):
    buf, fmt, gam = cache.read_pages(layer, seq, p, 1)
    return buf[0], int(fmt[0]), gam[0]


def check_pages(cache: vk.Cache, w: wl.Workload, layer: int, seq: int, kbits, vbits, pages=None,
                eps=1e-5, fp8_scale=1.0, fp8_dynamic=False) -> oc.EncodedSequence:
    """Formats, gamma (2^-22 rel) and bytes (exact, re-encoded with the device gamma) of sampled pages."""
    spec = spec_of(w, eps, fp8_scale, fp8_dynamic)
    calls = seq_calls(w, seq)
    enc = oc.encode_sequence(spec, kbits, vbits, w.dtype, calls)
    bs = w.block_size
    n_pages = len(enc.page_format)
    # device gamma of every call that wrote ternary pages
    dev_gamma = [(np.nan, np.nan)] * len(calls)
    for ci in range(len(calls)):
        toks = np.nonzero((enc.token_call == ci) & (enc.token_format == oc.TERNARY2))[0]
        if toks.size:
            _, fmt, gam = read_page(cache, layer, seq, int(toks[0]) // bs)
            assert fmt == oc.TERNARY2
            dev_gamma[ci] = (float(gam[0]), float(gam[1]))
            for j in range(2):
                want = float(enc.gamma[ci][j])
                assert abs(dev_gamma[ci][j] - want) <= GAMMA_RTOL * want, (layer, seq, ci, j, dev_gamma[ci][j], want)
    enc_dev = oc.encode_sequence(spec, kbits, vbits, w.dtype, calls, gamma_override=dev_gamma)
    pages = page_sample(n_pages) if pages is None else pages
    for p in pages:
        buf, fmt, gam = read_page(cache, layer, seq, p)
        assert fmt == enc.page_format[p], (layer, seq, p, fmt, enc.page_format[p])
        nb = oc.page_bytes(spec, fmt)
        got = buf[:nb]
        lo, hi = p * bs, min((p + 1) * bs, enc.length)
        if fmt == oc.TERNARY2 and (hi - lo == bs or bs == 16):
            want = oc.page_tiles(spec, enc_dev, p)
            if not np.array_equal(got, want):
                bad = np.nonzero(got != want)[0]
                raise AssertionError(f"page bytes differ: layer {layer} seq {seq} page {p} fmt {fmt} "
                                     f"first bad byte {bad[0]} of {nb} ({bad.size} bad)")
        else:
            check_partial_page(spec, enc_dev, p, got, fmt, hi - lo)
    return enc


def check_partial_page(spec, enc, p, got, fmt, n_tok):
    """Per-token comparison for a page whose tail was never written."""
    bs, hkv, dim = spec.block_size, spec.n_kv_heads, spec.head_dim
    tb = {oc.TERNARY2: bs * dim // 4, oc.FP8E4M3: bs * dim, oc.F16: bs * dim * 2}[fmt]
    stride = tb + (4 * bs if fmt == oc.FP8E4M3 and spec.fp8_dynamic else 0)   # + token scales
    lo = p * bs
    for which, off in (("k", 0), ("v", hkv * stride)):
        for h in range(hkv):
            tile = got[off + h * stride: off + h * stride + tb]
            if stride != tb:
                sc = got[off + h * stride + tb: off + (h + 1) * stride].view("<f4")
                assert np.array_equal(sc[:n_tok], getattr(enc, which + "_fp8_scale")[lo:lo + n_tok, h]), (p, which, h)
            if fmt == oc.TERNARY2:
                codes = ot.unpack_flat(tile.reshape(bs, dim // 4)) if which == "k" else \
                    ot.v_tile_codes(tile, bs, dim)
                want = getattr(enc, which + "_code")[lo:lo + n_tok, h]
            elif fmt == oc.FP8E4M3:
                codes = tile.reshape(bs, dim) if which == "k" else tile.reshape(dim, bs).T
                want = getattr(enc, which + "_fp8")[lo:lo + n_tok, h]
            else:
                t16 = tile.view(np.uint16)
                codes = t16.reshape(bs, dim) if which == "k" else t16.reshape(dim, bs).T
                want = getattr(enc, which + "_f16")[lo:lo + n_tok, h]
            assert np.array_equal(codes[:n_tok], want), (p, which, h, fmt)


def q_values(q: torch.Tensor, dtype: int) -> np.ndarray:
    return ot.values16(wl.to_bits(q), dtype)


def check_decode(out: torch.Tensor, q: torch.Tensor, w: wl.Workload, encs: Dict[int, oc.EncodedSequence],
                 window: int, ids: Sequence[int] = None, scale=None) -> float:
    """Max-abs error over the sequences with an oracle encoding."""
    ids = list(range(w.n_seqs)) if ids is None else list(ids)
    o = out.float().cpu().numpy()
    assert np.all(np.isfinite(o))
    qv = q_values(q, w.dtype)
    worst = 0.0
    for row, s in enumerate(ids):
        if s not in encs:
            continue
        enc = encs[s]
        ref = oa.decode_attention(qv[row], enc.k_hat, enc.v_hat, enc.length, w.sink_tokens, window, scale)
        err = float(np.max(np.abs(o[row] - ref)))
        worst = max(worst, err)
        assert err <= ATTN_ATOL, (s, err)
    return worst


def run_workload(w: wl.Workload, sample_seqs: Sequence[int], page_layers: Sequence[int],
                 decode_layers: Sequence[int], shuffle=None, decode_kernel=0, fp8_dynamic=0) -> dict:
    say(f"[{w.name}] create+fill (decode kernel {decode_kernel}, dynamic fp8 {fp8_dynamic})")
    cache = make_cache(w, shuffle=shuffle, decode_kernel=decode_kernel, fp8_dynamic=fp8_dynamic)
    fill(cache, w)
    report = {"gamma_checked": 0, "max_err": 0.0}
    encs_by_layer = {}
    for layer in sorted(set(page_layers) | set(decode_layers)):
        encs = {}
        for s in sample_seqs:
            kb, vb = host_kv(w, layer, s)
            if layer in page_layers:
                say(f"[{w.name}] pages layer {layer} seq {s}")
                encs[s] = check_pages(cache, w, layer, s, kb, vb, fp8_dynamic=fp8_dynamic)
            else:
                encs[s] = oc.encode_sequence(spec_of(w, fp8_dynamic=fp8_dynamic), kb, vb, w.dtype, seq_calls(w, s))
        encs_by_layer[layer] = encs
        if layer in decode_layers:
            q = wl.queries(w, layer, device="cuda")
            out = cache.decode(q, list(range(w.n_seqs)), layer, window=w.window)
            torch.cuda.synchronize()
            err = check_decode(out, q, w, encs, w.window)
            report["max_err"] = max(report["max_err"], err)
            say(f"[{w.name}] decode kernel {decode_kernel} layer {layer}: max abs err {err:.3e}")
        encs_by_layer.pop(layer, None)
    report["stats"] = cache.stats()
    cache.close()
    return report
