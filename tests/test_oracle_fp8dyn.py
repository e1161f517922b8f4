"""Pins of the oracle's dynamic FP8 (one scale per token and KV head).

Dynamic FP8 follows "Show HN: Vantage-V-AI" (its dynamic FP8 streaming mode;
quant_mode "fp8" in the quick start).  The pins compute the scale and the codes
from exact rationals with a brute-force nearest e4m3fn search (no float32
division), check the closed forms (the largest element maps to +-448; the
relative error bound of a 3-bit mantissa), the page layout, and that
retiering a dynamic page equals a ternary append of the same values when the
scales are powers of two.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import cache as oc
from oracle import fp8 as of
from oracle import ternary as ot

E4M3 = [Fraction(of.e4m3fn_value(c)) for c in range(0x7F)]   # 0 .. 448, exact


def f32_nearest(fr: Fraction) -> Fraction:
    f = np.float32(float(fr))
    cands = [f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - fr), int(np.float32(c).view(np.uint32)) & 1))
    return Fraction(float(best))


def e4m3_nearest(fr: Fraction) -> int:
    """Nearest e4m3fn code by brute force over every magnitude, ties to the even code, saturating."""
    a = min(abs(fr), Fraction(448))
    best = min(range(0x7F), key=lambda c: (abs(E4M3[c] - a), c & 1))
    return best | (0x80 if fr < 0 else 0)


def exact_dynamic(x_row):
    xs = [Fraction(float(np.float32(v))) for v in x_row]
    amax = max(abs(v) for v in xs)
    if amax == 0:
        return [0] * len(xs), Fraction(0)
    s = f32_nearest(amax / 448)
    return [e4m3_nearest(f32_nearest(v / s)) for v in xs], s


def test_against_exact_rationals():
    rng = np.random.default_rng(0)
    rows = [rng.standard_normal(32) * 10.0 ** rng.integers(-6, 4) for _ in range(40)]
    rows += [np.array([2.0, 1.0, -0.5, 0.0] * 8), np.array([1e-30, -3e-31] * 16), np.zeros(32),
             np.array([448.0] + [448.0 * 2 ** -k for k in range(1, 32)])]
    x = np.stack(rows)
    codes, scales = of.fp8_dynamic_encode(x)
    for i, row in enumerate(rows):
        want_c, want_s = exact_dynamic(row)
        assert Fraction(float(scales[i])) == want_s, i
        assert codes[i].tolist() == want_c, i


def test_hand_example():
    # amax 2: s = float32(2/448); 2 -> 448 (0x7E), 1 -> 224 (0x76), -0.5 -> -112 (0xEE), 0 -> 0
    codes, s = of.fp8_dynamic_encode(np.array([[2.0, 1.0, -0.5, 0.0]]))
    assert float(s[0]) == float(np.float32(2.0 / 448.0))
    assert codes[0].tolist() == [0x7E, 0x76, 0xEE, 0x00]
    hat = of.fp8_dynamic_dequantize(codes, s)
    assert hat[0].tolist() == [float(s[0]) * 448, float(s[0]) * 224, -float(s[0]) * 112, 0.0]


def test_closed_forms():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((500, 128)) * np.exp(rng.uniform(-8, 8, (500, 1)))
    x = x.astype(np.float32).astype(np.float64)
    codes, s = of.fp8_dynamic_encode(x)
    hat = of.fp8_dynamic_dequantize(codes, s)
    i = np.argmax(np.abs(x), axis=1)
    assert np.all((codes[np.arange(500), i] & 0x7F) == 0x7E)                  # the max maps to 448
    assert np.allclose(hat[np.arange(500), i], x[np.arange(500), i], rtol=2 ** -20)
    err = np.abs(hat - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, s[:, None].astype(np.float64) * 2.0 ** -10) * (1 + 2 ** -20)
    assert np.all(err <= bound)
    z, zs = of.fp8_dynamic_encode(np.zeros((2, 8)))
    assert not z.any() and not zs.any()


def test_page_layout_with_scales():
    spec = oc.CacheSpec(n_kv_heads=2, head_dim=64, block_size=16, sink_tokens=0, recent_tokens=64,
                        recent_format=oc.FP8E4M3, fp8_dynamic=True)
    assert oc.page_bytes(spec, oc.FP8E4M3) == 2 * 2 * (16 * 64 + 64)
    rng = np.random.default_rng(2)
    k = np.asarray(rng.standard_normal((20, 2, 64)), dtype=np.float16).view(np.uint16)
    v = np.asarray(rng.standard_normal((20, 2, 64)) * 3, dtype=np.float16).view(np.uint16)
    enc = oc.encode_sequence(spec, k, v, ot.F16, [(0, 20)])
    tile = 16 * 64 + 64
    b = oc.page_tiles(spec, enc, 1)                       # 4 tokens written, 12 empty slots
    ksc = b[tile - 64:tile].view("<f4")                  # head 0 key scales
    assert ksc[:4].tolist() == enc.k_fp8_scale[16:20, 0].tolist() and not ksc[4:].any()
    vt = b[3 * tile:4 * tile]                            # value tile of head 1
    assert np.array_equal(vt[:16 * 64].reshape(64, 16).T[:4], enc.v_fp8[16:20, 1])
    assert vt[16 * 64:].view("<f4")[:4].tolist() == enc.v_fp8_scale[16:20, 1].tolist()


def test_retier_of_dynamic_pages_equals_ternary_append():
    """Rows whose largest element is 448 * 2^k get the scale 2^k exactly, so their dequantised
    values are bfloat16 numbers; a ternary append of those values quantises identically."""
    rng = np.random.default_rng(3)
    spec = oc.CacheSpec(n_kv_heads=2, head_dim=64, block_size=16, sink_tokens=0, recent_tokens=16,
                        recent_format=oc.FP8E4M3, fp8_dynamic=True)
    x = rng.standard_normal((32, 2, 64)) * 0.2
    ks = rng.integers(-8, 3, size=(32, 2))
    x[:, :, 5] = 448.0 * 2.0 ** ks
    xb = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)    # truncate to bfloat16
    xv = ot.values16(xb, ot.BF16)
    assert np.all(np.max(np.abs(xv), axis=2) == 448.0 * 2.0 ** ks)
    enc = oc.encode_sequence(spec, xb, xb[:, ::-1].copy(), ot.BF16, [(0, 16), (16, 16)])
    assert np.array_equal(enc.k_fp8_scale[:16], (2.0 ** ks[:16]).astype(np.float32))
    r = oc.retier(spec, enc)
    assert r.page_format[0] == oc.TERNARY2 and not r.k_fp8_scale[:16].any()
    hk, hv = enc.k_hat[:16], enc.v_hat[:16]
    to_bf = lambda a: (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(ot.values16(to_bf(hk), ot.BF16), hk)            # exact in bfloat16
    t = oc.encode_sequence(oc.CacheSpec(n_kv_heads=2, head_dim=64, block_size=16, sink_tokens=0),
                           to_bf(hk), to_bf(hv), ot.BF16, [(0, 16)])
    assert r.page_gamma[0] == t.gamma[0]
    assert np.array_equal(oc.page_tiles(spec, r, 0), oc.page_tiles(spec, t, 0))
