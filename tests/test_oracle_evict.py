"""Pins of the oracle's bounded-memory eviction rule.

Eviction follows "Show HN: Vantage-V-AI" (quick start: max_active_tokens and
sink_tokens; core architecture: bounded-memory streaming cache that keeps the
attention sinks).  The pins check the page rule against the attended set
(itself pinned against masked SDPA), a hand-worked case, the memory bound,
monotonicity, and that attention never reads a freed token (freed tokens are
poisoned with NaN and the outputs stay identical).
"""
import numpy as np

from oracle import attention as oa
from oracle import cache as oc
from oracle import ternary as ot


def spec(bs=16, S=4, sink_fmt=oc.F16, R=0):
    return oc.CacheSpec(n_kv_heads=2, head_dim=64, block_size=bs, sink_tokens=S, sink_format=sink_fmt,
                        recent_tokens=R, recent_format=oc.FP8E4M3)


def test_hand_example():
    # L = 1000, S = 4, W = 256, Bs = 16: the window starts at 744; pages 1..45 end by 736 <= 744,
    # page 46 = [736, 752) holds window tokens; page 0 holds the sinks
    sp = spec()
    ev = oc.evict_pages(sp, 1000, 256)
    assert ev == list(range(1, 46))
    kept = [p for p in range(63) if p not in ev]
    assert kept == [0] + list(range(46, 63)) and len(kept) == 18
    assert oc.evict_pages(sp, 1000, -1) == []
    assert oc.evict_pages(sp, 200, 256) == []          # the window covers everything
    assert oc.evict_pages(spec(S=40), 1000, 0) == list(range(3, 62))  # sinks 0..2; page 62 partial


def test_freed_pages_hold_no_attended_token_and_memory_is_bounded():
    rng = np.random.default_rng(0)
    for _ in range(300):
        bs = int(rng.choice([16, 32, 64]))
        S = int(rng.integers(0, 70))
        W = int(rng.integers(0, 400))
        L = int(rng.integers(1, 3000))
        sp = spec(bs=bs, S=S)
        ev = set(oc.evict_pages(sp, L, W))
        n_pages = -(-L // bs)
        assert ev <= set(range(n_pages))
        # no token of any later window W' <= W (from any length L' >= L) is in a freed page
        for L2 in (L, L + int(rng.integers(0, 100))):
            for W2 in (W, int(rng.integers(0, W + 1))):
                if S == 0 and W2 == 0:
                    continue
                att = oa.attended_tokens(L2, S, W2)
                assert not ({int(t) // bs for t in att} & ev), (bs, S, W, L, L2, W2)
        # every page that holds no such token and is past the sinks is freed (nothing kept needlessly)
        att_pages = {int(t) // bs for t in oa.attended_tokens(L, S, W)} if (S or W) else set()
        first = -(-S // bs)
        for p in range(first, n_pages):
            if p not in att_pages and (p + 1) * bs <= L - W:
                assert p in ev
        kept = n_pages - len(ev)
        assert kept <= -(-S // bs) + -(-W // bs) + 1


def test_monotone_in_length():
    sp = spec()
    prev = set()
    for L in range(1, 2000, 7):
        ev = set(oc.evict_pages(sp, L, 100))
        assert prev <= ev
        prev = ev


def test_attention_never_reads_freed_tokens():
    rng = np.random.default_rng(1)
    sp = spec(S=4, R=48)
    T = 700
    bits_k = np.asarray(rng.standard_normal((T, 2, 64)), dtype=np.float16).view(np.uint16)
    bits_v = np.asarray(rng.standard_normal((T, 2, 64)), dtype=np.float16).view(np.uint16)
    enc = oc.encode_sequence(sp, bits_k, bits_v, ot.F16, [(0, 300), (300, 1), (301, 399)])
    W = 100
    ev = oc.evict_pages(sp, T, W)
    k, v = enc.k_hat.copy(), enc.v_hat.copy()
    for p in ev:
        k[p * 16:(p + 1) * 16] = np.nan
        v[p * 16:(p + 1) * 16] = np.nan
    q = rng.standard_normal((8, 64))
    for w in (W, 60, 1, 0):
        a = oa.decode_attention(q, enc.k_hat, enc.v_hat, T, 4, w)
        b = oa.decode_attention(q, k, v, T, 4, w)
        assert np.array_equal(a, b) and np.all(np.isfinite(b))
    assert np.isnan(oa.decode_attention(q, k, v, T, 4, -1)).any()   # the whole context would read them
