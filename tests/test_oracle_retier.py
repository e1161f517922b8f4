"""Pins of the oracle's retiering (FP8 recent pages re-encoded as ternary pages).

Retiering follows "Minima-KV" (twodots.gr): the Recent tier is FP8, older
pages are packed, and the evaluated profile retiers pages dynamically.  The
pins use a hand-worked page, exact rational arithmetic, the already pinned
append path (a page appended as 16-bit values equal to the FP8 values must
quantise identically), and invariants (idempotence, independence of when the
retiering runs, pages outside the eligible set untouched, attention over the
untouched window unchanged).
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import attention as oa
from oracle import cache as oc
from oracle import fp8 as of
from oracle import ternary as ot


def f16_bits(vals):
    return np.asarray(vals, dtype=np.float16).view(np.uint16)


def bf16_bits_exact(vals):
    """bfloat16 patterns of values that bfloat16 holds exactly (checked)."""
    x = np.asarray(vals, dtype=np.float32)
    b = (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    assert np.array_equal(ot.values16(b, ot.BF16), x.astype(np.float64))
    return b


def _f32_nearest(fr: Fraction) -> np.float32:
    """Round an exact rational to the nearest float32, ties to even, without float division."""
    f = np.float32(float(fr))
    cands = {f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))}
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - fr), int(np.float32(c).view(np.uint32)) & 1))
    return np.float32(best)


def _exact_code(x: Fraction, d: Fraction) -> int:
    if d == 0:
        return 0
    if abs(x) / d > Fraction(1, 2) + Fraction(1, 2 ** 25):
        return 1 if x > 0 else -1
    return 0


SPEC = oc.CacheSpec(n_kv_heads=1, head_dim=4, block_size=16, sink_tokens=4, sink_format=oc.F16,
                    recent_tokens=32, recent_format=oc.FP8E4M3)


def test_eligible_pages_hand_example():
    rng = np.random.default_rng(0)
    k = f16_bits(rng.standard_normal((112, 1, 4)))
    enc = oc.encode_sequence(SPEC, k, k, ot.F16, [(0, 64), (64, 48)])
    # first call (L' = 64): page 0 sink, page 1 ternary, pages 2, 3 meet [32, 64) -> fp8;
    # second call (L' = 112): page 4 = [64, 80) ends at 80 = L' - R -> ternary; 5, 6 fp8
    assert enc.page_format == [oc.F16, oc.TERNARY2, oc.FP8E4M3, oc.FP8E4M3, oc.TERNARY2,
                               oc.FP8E4M3, oc.FP8E4M3]
    assert oc.retier_pages(SPEC, enc) == [2, 3]          # (p+1)*16 <= 112 - 32 = 80
    assert oc.retier_pages(SPEC, enc, 64) == []          # at L = 64 the window starts at 32
    assert oc.retier_pages(SPEC, enc, 95) == [2]         # page 3 ends at 64 > 63
    assert oc.retier_pages(SPEC, enc, 96) == [2, 3]
    assert oc.retier_pages(SPEC, enc, 111) == [2, 3]     # page 5 ends at 96 > 79
    spec_fp8_sink = oc.CacheSpec(n_kv_heads=1, head_dim=4, block_size=16, sink_tokens=4,
                                 sink_format=oc.FP8E4M3, recent_tokens=32)
    enc2 = oc.encode_sequence(spec_fp8_sink, k, k, ot.F16, [(0, 64), (64, 48)])
    assert enc2.page_format[0] == oc.FP8E4M3 and 0 not in oc.retier_pages(spec_fp8_sink, enc2)
    spec_no_recent = oc.CacheSpec(n_kv_heads=1, head_dim=4, block_size=16)
    enc3 = oc.encode_sequence(spec_no_recent, k, k, ot.F16, [(0, 112)])
    assert oc.retier_pages(spec_no_recent, enc3) == []


def test_hand_worked_page():
    """One page (16 tokens x 1 head x 4 dims = 64 elements), eps = 0:
    30 x (+-2), 2 x (+-1), 4 x (+-1/2), the rest 0 -> sum |x| = 64, gamma = 1, d = 1;
    +-2 and +-1 -> +-1; +-1/2 is an exact tie of x/d = 1/2 -> 0 (ties to even)."""
    spec = oc.CacheSpec(n_kv_heads=1, head_dim=4, block_size=16, sink_tokens=0, eps=0.0,
                        recent_tokens=16, recent_format=oc.FP8E4M3)
    vals = np.zeros(64)
    vals[:30] = [2.0, -2.0] * 15
    vals[30:32] = [1.0, -1.0]
    vals[32:36] = [0.5, -0.5, 0.5, -0.5]
    x = np.zeros((32, 1, 4))
    x[:16] = vals.reshape(16, 1, 4)
    x[16:] = 1.0
    bits = f16_bits(x)
    enc = oc.encode_sequence(spec, bits, bits, ot.F16, [(0, 16), (16, 16)])
    assert enc.page_format == [oc.FP8E4M3, oc.FP8E4M3]
    r = oc.retier(spec, enc)
    assert r.page_format == [oc.TERNARY2, oc.FP8E4M3]
    assert r.page_gamma == {0: (np.float32(1.0), np.float32(1.0))}
    want = np.zeros(64, dtype=np.int8)
    want[:30] = [1, -1] * 15
    want[30:32] = [1, -1]
    assert r.k_code[:16].ravel().tolist() == want.tolist()
    assert r.v_hat[:16].ravel().tolist() == want.astype(float).tolist()
    assert not r.k_fp8[:16].any() and np.array_equal(r.k_fp8[16:], enc.k_fp8[16:])
    assert np.all(r.token_format[:16] == oc.TERNARY2)


def test_all_zero_page():
    for eps in (1e-5, 0.0):
        spec = oc.CacheSpec(n_kv_heads=2, head_dim=4, block_size=16, sink_tokens=0, eps=eps,
                            recent_tokens=16, recent_format=oc.FP8E4M3)
        x = np.zeros((32, 2, 4))
        x[16:] = 1.0
        bits = f16_bits(x)
        r = oc.retier(spec, oc.encode_sequence(spec, bits, bits, ot.F16, [(0, 16), (16, 16)]))
        assert r.page_gamma[0] == (np.float32(0.0), np.float32(0.0))
        assert not r.k_code[:16].any() and not r.v_hat[:16].any()


@pytest.mark.parametrize("scale", [1.0, 0.25, 0.3])
def test_gamma_and_codes_against_exact_rationals(scale):
    rng = np.random.default_rng(12)
    spec = oc.CacheSpec(n_kv_heads=2, head_dim=8, block_size=16, sink_tokens=0, recent_tokens=16,
                        recent_format=oc.FP8E4M3, fp8_scale=scale)
    x = rng.standard_normal((48, 2, 8)) * 3.0
    x[5, 1, :] = 0.0
    bits = f16_bits(x)
    enc = oc.encode_sequence(spec, bits, bits[::-1].copy(), ot.F16, [(0, 20), (20, 12), (32, 16)])
    r = oc.retier(spec, enc)
    assert oc.retier_pages(spec, enc) == [0, 1]
    s = Fraction(float(np.float32(scale)))
    for p in (0, 1):
        for which, gi in (("k", 0), ("v", 1)):
            codes8 = getattr(enc, which + "_fp8")[16 * p:16 * (p + 1)].ravel()
            exact = [s * Fraction(of.e4m3fn_value(int(c))) for c in codes8]
            g = _f32_nearest(sum(abs(e) for e in exact) / len(exact))
            assert r.page_gamma[p][gi] == g
            d = Fraction(float(np.float32(g + np.float32(spec.eps))))
            want = [_exact_code(Fraction(float(_f32_nearest(e))), d) for e in exact]
            assert getattr(r, which + "_code")[16 * p:16 * (p + 1)].ravel().tolist() == want


def test_retiered_page_equals_a_ternary_append_of_the_same_values():
    """A page appended once as ternary from 16-bit values equal to an FP8 page's values
    (bfloat16 holds every e4m3fn value) gets the same gamma and codes as the retiered page."""
    rng = np.random.default_rng(21)
    for hkv, dim in ((1, 4), (8, 128)):
        spec = oc.CacheSpec(n_kv_heads=hkv, head_dim=dim, block_size=16, sink_tokens=0,
                            recent_tokens=16, recent_format=oc.FP8E4M3)
        k = f16_bits(rng.standard_normal((32, hkv, dim)))
        v = f16_bits(rng.standard_normal((32, hkv, dim)) * 0.1)
        enc = oc.encode_sequence(spec, k, v, ot.F16, [(0, 16), (16, 16)])
        r = oc.retier(spec, enc)
        spec_t = oc.CacheSpec(n_kv_heads=hkv, head_dim=dim, block_size=16, sink_tokens=0)
        kb = bf16_bits_exact(of.fp8_dequantize(enc.k_fp8[:16], 1.0))
        vb = bf16_bits_exact(of.fp8_dequantize(enc.v_fp8[:16], 1.0))
        t = oc.encode_sequence(spec_t, kb, vb, ot.BF16, [(0, 16)])
        assert r.page_gamma[0] == t.gamma[0]
        assert np.array_equal(r.k_code[:16], t.k_code) and np.array_equal(r.v_code[:16], t.v_code)
        assert np.array_equal(oc.page_tiles(spec, r, 0), oc.page_tiles(spec_t, t, 0))


def test_idempotent_and_independent_of_when_it_runs():
    rng = np.random.default_rng(31)
    spec = oc.CacheSpec(n_kv_heads=2, head_dim=8, block_size=16, sink_tokens=4, sink_format=oc.F16,
                        recent_tokens=40, recent_format=oc.FP8E4M3)
    T = 300
    k = f16_bits(rng.standard_normal((T, 2, 8)))
    v = f16_bits(rng.standard_normal((T, 2, 8)))
    calls, t = [], 0
    while t < T:
        n = int(min(T - t, rng.integers(1, 40)))
        calls.append((t, n))
        t += n
    enc = oc.encode_sequence(spec, k, v, ot.F16, calls)
    once = oc.retier(spec, enc)
    assert once.page_format.count(oc.FP8E4M3) >= 3   # pages meeting the last 40 tokens stay
    twice = oc.retier(spec, once)
    staged = oc.retier(spec, oc.retier(spec, enc, 150), T)
    for a in (twice, staged):
        assert a.page_format == once.page_format and a.page_gamma == once.page_gamma
        for f in ("k_code", "v_code", "k_fp8", "v_fp8", "k_hat", "v_hat"):
            assert np.array_equal(getattr(a, f), getattr(once, f)), f
    # pages outside the retiered set are untouched, byte for byte
    done = set(oc.retier_pages(spec, enc))
    for p in range(len(enc.page_format)):
        if p not in done and (p + 1) * 16 <= T:
            assert np.array_equal(oc.page_tiles(spec, once, p), oc.page_tiles(spec, enc, p))
    # every retiered value is gamma_page * {-1, 0, +1}
    for p in done:
        gk, gv = once.page_gamma[p]
        assert set(np.unique(once.k_hat[16 * p:16 * p + 16] / float(gk))) <= {-1.0, 0.0, 1.0}
        assert set(np.unique(once.v_hat[16 * p:16 * p + 16] / float(gv))) <= {-1.0, 0.0, 1.0}


def test_attention_over_the_window_is_unchanged():
    """Decoding with sinks + a window no wider than the recent tier reads no retiered page."""
    rng = np.random.default_rng(41)
    spec = oc.CacheSpec(n_kv_heads=2, head_dim=64, block_size=16, sink_tokens=4, sink_format=oc.F16,
                        recent_tokens=64, recent_format=oc.FP8E4M3)
    k = f16_bits(rng.standard_normal((400, 2, 64)))
    v = f16_bits(rng.standard_normal((400, 2, 64)))
    enc = oc.encode_sequence(spec, k, v, ot.F16, [(0, 100), (100, 150), (250, 150)])
    r = oc.retier(spec, enc)
    assert oc.retier_pages(spec, enc)
    q = rng.standard_normal((8, 64))
    for w in (1, 33, 64):
        a = oa.decode_attention(q, enc.k_hat, enc.v_hat, 400, 4, w)
        b = oa.decode_attention(q, r.k_hat, r.v_hat, 400, 4, w)
        assert np.array_equal(a, b)
    full_a = oa.decode_attention(q, enc.k_hat, enc.v_hat, 400, 4, -1)
    full_b = oa.decode_attention(q, r.k_hat, r.v_hat, 400, 4, -1)
    assert not np.array_equal(full_a, full_b)          # the whole context does see them
    assert np.max(np.abs(full_a - full_b)) < 0.5
