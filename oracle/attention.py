"""Decode attention over the cache's dequantised keys and values (test oracle).

Follows "Minima-KV" (twodots.gr), section on mixed-format attention: every
page format is read directly, and the per-branch partial states are merged by
one online-softmax normalisation in logical page order; the result equals
softmax attention over the dequantised values.  "Show HN: Vantage-V-AI",
quick start and core architecture: the attended tokens are the first
sink_tokens plus a bounded recent window (max_active_tokens); the window may
be the whole context (retention-preserving, Minima-KV).

Readings where the pages are silent:
  * Attended set A = [0, min(S, L)) union [max(0, L - W), L); W = -1 means
    the whole context.  The decode query's own token is not in the cache.
  * Softmax scale 1/sqrt(D) unless given; GQA groups are contiguous: query
    head h reads KV head h // (Hq / Hkv).
  * The output is float32-sized but computed here in float64.
"""
from __future__ import annotations

import numpy as np


def attended_tokens(length: int, sink_tokens: int, window: int) -> np.ndarray:
    """Sorted token indices of A for a sequence of ``length`` tokens."""
    if length <= 0:
        raise ValueError("empty sequence")
    if window < 0:
        return np.arange(length)
    sinks = set(range(min(sink_tokens, length)))
    recent = set(range(max(0, length - window), length))
    return np.array(sorted(sinks | recent), dtype=np.int64)


def decode_attention(q: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray, length: int,
                     sink_tokens: int, window: int, scale: float = None) -> np.ndarray:
    """One decode step: q [Hq, D], k_hat / v_hat [T >= length, Hkv, D] -> [Hq, D] float64."""
    q = np.asarray(q, dtype=np.float64)
    hq, dim = q.shape
    hkv = k_hat.shape[1]
    g = hq // hkv
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(dim)
    idx = attended_tokens(length, sink_tokens, window)
    out = np.zeros((hq, dim), dtype=np.float64)
    for h in range(hq):
        kv = h // g
        kk = np.asarray(k_hat[idx, kv, :], dtype=np.float64)
        vv = np.asarray(v_hat[idx, kv, :], dtype=np.float64)
        s = scale * (kk @ q[h])
        p = np.exp(s - s.max())
        out[h] = (p @ vv) / p.sum()
    return out
