"""Pins of the lossless bfloat16 tier's oracle (oracle/lossless.py) to facts fixed outside it:
IEEE field definitions, a hand-worked group, every bfloat16 pattern through a round trip,
and the closed-form storage ratio on N(0,1) data."""
import math

import numpy as np
import pytest

from oracle import lossless as ll
from oracle import ternary as ot


def all_patterns():
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)


def test_split_matches_the_float_fields():
    """The exponent field is floor(log2 |x|) + 127 for normal values; the sign+mantissa byte
    is the sign and (|x| / 2^floor(log2 |x|) - 1) * 128, from the values, not the bits."""
    bits = all_patterns()
    vals = ot.values16(bits, ot.BF16)
    exp, sm = ll.split(bits)
    normal = np.isfinite(vals) & (np.abs(vals) >= 2.0 ** -126)
    m, e = np.frexp(np.abs(vals[normal]))          # |x| = m 2^e, m in [0.5, 1)
    assert np.array_equal(exp[normal].astype(np.int64), (e - 1 + 127).astype(np.int64))
    assert np.array_equal((sm[normal] & 0x7F).astype(np.int64), np.rint((2 * m - 1) * 128).astype(np.int64))
    assert np.array_equal(sm[normal] >> 7, np.signbit(vals[normal]).astype(np.uint8))
    assert np.array_equal(exp[(vals == 0) | (np.abs(vals) < 2.0 ** -126)], np.zeros(int(np.sum(~normal & np.isfinite(vals))), np.uint8))
    assert np.array_equal(ll.join(exp, sm), bits)


def test_hand_worked_group():
    """16 x 64 keys of 1.0 (field 127) except: t=0,d=0 is 0.0 (field 0); t=5,d=40 is 2^-30
    (field 97); t=2,d=17 is 3.0 (field 128); t=9,d=63 is -2^20 (field 147).
    Nonzero fields: 1019 of 127 plus 97, 128, 147 -> mean (1019*127 + 372) / 1022 = 126.98...
    -> centre 126.  Codes: 127 -> 12, 128 -> 13, 97 -> escape, 147 -> escape, 0 -> escape.
    Exception order by (lane, position), lane = (d // 16) * 16 + t, position = d % 16:
    (0,0) lane 0; (5,40) lane 37; (9,63) lane 57 -> bytes 0, 97, 147."""
    x = np.full((16, 64), 1.0, dtype=np.float32)
    x[0, 0] = 0.0
    x[5, 40] = 2.0 ** -30
    x[2, 17] = 3.0
    x[9, 63] = -(2.0 ** 20)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)   # exact in bfloat16
    slot = ll.encode_group(bits, "k")
    assert slot.size == 32 * 64 + 16
    assert slot[0] == 126 and slot[1] == 0 and int(slot[4:8].view("<u4")[0]) == 3
    assert not slot[2:4].any() and not slot[8:16].any()
    sm = slot[16:16 + 1024].reshape(16, 64)
    assert sm[9, 63] == 0x80 and sm[2, 17] == 0x40 and sm[0, 0] == 0 and sm[3, 3] == 0
    codes = slot[16 + 1024:16 + 1536]
    nib = lambda t, d: (codes[(t * 64 + d) // 2] >> (4 * ((t * 64 + d) % 2))) & 0xF  # noqa: E731
    assert nib(1, 1) == 12 and nib(2, 17) == 13 and nib(0, 0) == 15 and nib(5, 40) == 15 and nib(9, 63) == 15
    assert list(slot[16 + 1536:16 + 1536 + 3]) == [0, 97, 147]
    assert not slot[16 + 1536 + 3:].any()
    assert np.array_equal(ll.decode_group(slot, 64, "k"), bits)


def test_value_exception_order():
    """Values list exceptions by lane = (t // 4) * 16 + d % 16, position (d // 16) * 4 + t % 4."""
    x = np.full((16, 128), 0.5, dtype=np.float32)
    picks = [(15, 127), (0, 33), (4, 1), (3, 1)]      # lanes 63, 1, 17, 1; positions 31, 8, 0, 3
    for i, (t, d) in enumerate(picks):
        x[t, d] = 2.0 ** (40 + i)                       # fields 167 .. 170, all escapes
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    slot = ll.encode_group(bits, "v")
    n = int(slot[4:8].view("<u4")[0])
    exc = list(slot[16 + 24 * 128:16 + 24 * 128 + n])
    # (lane, position): (1, 3) field 170, (1, 8) field 168, (17, 0) field 169, (63, 31) field 167
    assert exc == [170, 168, 169, 167]
    assert np.array_equal(ll.decode_group(slot, 128, "v"), bits)


@pytest.mark.parametrize("dim", [64, 128])
@pytest.mark.parametrize("which", ["k", "v"])
def test_every_bf16_pattern_round_trips(dim, which):
    bits = all_patterns()
    n_groups = 65536 // (16 * dim)
    arrangements = [bits,                                                  # narrow exponent ranges: coded
                    bits.reshape(16 * dim, n_groups).T.ravel(),            # every exponent in a group: raw
                    np.random.default_rng(3).permutation(bits)]
    modes = set()
    for b in arrangements:
        for g in b.reshape(-1, 16, dim):
            slot = ll.encode_group(g, which)
            modes.add(int(slot[1]))
            assert np.array_equal(ll.decode_group(slot, dim, which), g)
    assert modes == {0, 1}


def test_raw_fallback_when_exceptions_overflow():
    x = np.where(np.arange(16 * 64).reshape(16, 64) % 2 == 0, 1e-30, 1e30).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    slot = ll.encode_group(bits, "v")
    assert slot[1] == 1
    assert ll.read_bytes(slot, 64) == 16 + 32 * 64
    assert np.array_equal(ll.decode_group(slot, 64, "v"), bits)


def test_lane_order_is_a_permutation_matching_the_lane_layout():
    for dim in (64, 128):
        for which in ("k", "v"):
            r = ll.lane_order(dim, which)
            assert np.array_equal(np.sort(r), np.arange(16 * dim))
    r = ll.lane_order(128, "k")
    assert r[3 * 128 + 70] == (2 * 16 + 3) * 32 + 6        # lane 35, position 6
    r = ll.lane_order(128, "v")
    assert r[6 * 128 + 37] == (1 * 16 + 5) * 32 + 2 * 4 + 2  # lane 21, position 10


def test_storage_ratio_on_normal_data_matches_closed_form():
    """N(0,1) values: exponent field k + 127 with P = 2 (Phi(2^(k+1)) - Phi(2^k)); the centre is
    floor(127 + E[k]) = 125; escapes are the fields outside [114, 128]; expected bytes read per
    group = 16 + 16 D (1 + 1/2 + P(escape))."""
    from scipy.stats import norm
    ks = np.arange(-150, 10)
    p = np.array([2 * (norm.cdf(2.0 ** (k + 1)) - norm.cdf(2.0 ** k)) for k in ks])
    c = int(math.floor(127 + float((ks * p).sum())))
    assert c == 125
    e = ks + 127
    p_esc = float(p[(e < c - 11) | (e > c + 3)].sum())
    dim = 128
    want = (16 + 16 * dim * (1.5 + p_esc)) / (32 * dim)
    rng = np.random.default_rng(2024)
    x = rng.standard_normal((256, 16, dim)).astype(np.float32)
    bits = ((x.view(np.uint32) + 0x7FFF + ((x.view(np.uint32) >> 16) & 1)) >> 16).astype(np.uint16)  # RNE
    got = 0
    for g in bits:
        slot = ll.encode_group(g, "k")
        assert slot[0] == c
        got += ll.read_bytes(slot, dim)
    frac = got / (256 * 32 * dim)
    assert abs(frac - want) < 2e-4, (frac, want)
    assert 1.32 < 1 / frac < 1.34          # about 1.33x fewer bytes than bfloat16


def test_cache_pages_of_the_lossless_tier():
    """A sequence whose sink pages (and recent pages) are lossless: the page bytes are the group
    slots of each head's 16-token units; decoding them gives back the input bits; the attention
    inputs are the input values exactly; an append into a partly filled lossless page is refused,
    and so is float16 input."""
    from oracle import cache as oc
    spec = oc.CacheSpec(n_kv_heads=2, head_dim=64, block_size=32, sink_tokens=40, sink_format=oc.LOSSLESS,
                        recent_tokens=20, recent_format=oc.LOSSLESS)
    rng = np.random.default_rng(8)
    T = 32 * 4 + 9
    x = rng.standard_normal((2, T, 2, 64)).astype(np.float32)
    bits = ((x.view(np.uint32) + 0x7FFF + ((x.view(np.uint32) >> 16) & 1)) >> 16).astype(np.uint16)
    kb, vb = bits[0], bits[1]
    enc = oc.encode_sequence(spec, kb, vb, ot.BF16, [(0, 64), (64, T - 64)])
    assert enc.page_format == [oc.LOSSLESS, oc.LOSSLESS, oc.TERNARY2, oc.LOSSLESS, oc.LOSSLESS]
    assert oc.page_bytes(spec, oc.LOSSLESS) == 2 * 2 * 2 * (32 * 64 + 16)
    for p in (0, 4):
        page = oc.page_tiles(spec, enc, p)
        assert page.size == oc.page_bytes(spec, oc.LOSSLESS)
        slots = page.reshape(2, 2, 2, 32 * 64 + 16)        # [K|V][head][unit][slot]
        for w, which, src in ((0, "k", kb), (1, "v", vb)):
            for h in range(2):
                for u in range(2):
                    t0 = p * 32 + u * 16
                    want = np.zeros((16, 64), np.uint16)
                    n = max(0, min(16, T - t0))
                    want[:n] = src[t0:t0 + n, h]
                    assert np.array_equal(slots[w, h, u], ll.encode_group(want, which))
                    assert np.array_equal(ll.decode_group(slots[w, h, u], 64, which), want)
    ls = enc.token_format == oc.LOSSLESS
    assert np.array_equal(enc.k_hat[ls], ot.values16(kb, ot.BF16)[ls])
    assert np.array_equal(enc.v_lossless[ls], vb[ls])
    with pytest.raises(oc.AlignError):
        oc.encode_sequence(spec, kb, vb, ot.BF16, [(0, 20), (20, T - 20)])
    with pytest.raises(ValueError):
        oc.encode_sequence(spec, kb, vb, ot.F16, [(0, T)])
