"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these re-types the oracle's formula: they use hand-worked fixtures
(tests/golden, each citing its page), closed forms, exact rational
arithmetic, and library routines (torch conversions and SDPA) for the cases
that reduce to them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import cache as oc
from oracle import fp8 as of
from oracle import ternary as ot

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def f16_bits(vals):
    return np.asarray(vals, dtype=np.float16).view(np.uint16)


# ---------------------------------------------------------------- ternary ---

@pytest.mark.parametrize("name", ["ternary_hand_example.json", "ternary_tie_example.json"])
def test_hand_examples(name):
    g = golden(name)
    bits = f16_bits(g["x"])
    x = ot.values16(bits, ot.F16)
    gamma = ot.absmean_gamma(x)
    assert float(gamma) == g["gamma"]
    codes = ot.ternary_codes(x, gamma, g["eps"])
    assert codes.tolist() == g["codes"]
    assert ot.pack_flat(codes).tolist() == g["bytes"]
    packed, gamma2 = ot.quantize_pack(bits, ot.F16, g["eps"])
    assert packed.tolist() == g["bytes"] and float(gamma2) == g["gamma"]


def test_dequantize_hand_example():
    g = golden("ternary_hand_example.json")
    hat = ot.dequantize(np.array(g["codes"]), np.float32(g["gamma"]))
    assert hat.tolist() == [0.828125 * c for c in g["codes"]]


def test_gamma_rounds_the_float64_mean_to_float32():
    # 1/3 is not a float32: the mean of [1, 0, 0] must be float32(1/3)
    x = ot.values16(f16_bits([1.0, 0.0, -0.0]), ot.F16)
    assert ot.absmean_gamma(x) == np.float32(1.0 / 3.0)
    # sign does not matter, only |x|
    assert ot.absmean_gamma(np.array([-2.0, 2.0])) == np.float32(2.0)


def test_bf16_values_are_exact():
    # 0x3F80 = 1.0, 0xC020 = -2.5, 0x0001 = smallest subnormal 2^-133
    v = ot.values16(np.array([0x3F80, 0xC020, 0x0001], dtype=np.uint16), ot.BF16)
    assert v.tolist() == [1.0, -2.5, 2.0 ** -133]


def _exact_code(x: Fraction, d: Fraction) -> int:
    """RoundClip(float32(x/d)) from exact rationals, without dividing in floating point.

    float32(x/d) > 1/2 exactly when x/d lies above the midpoint 1/2 + 2^-25 between
    1/2 and the next float32 (a tie rounds to 1/2, whose significand is even);
    rint of anything in (1/2, inf] is >= 1, of [0, 1/2] is 0.  Symmetric for x < 0.
    """
    if d == 0:
        return 0
    t = abs(x) / d
    mid = Fraction(1, 2) + Fraction(1, 2 ** 25)
    if t > mid:
        return 1 if x > 0 else -1
    return 0


@pytest.mark.parametrize("dtype", [ot.F16, ot.BF16])
def test_codes_against_exact_rationals_exhaustive(dtype):
    """Every finite 16-bit input, several divisors (including exact-tie ones)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = ot.values16(bits, dtype)
    finite = np.isfinite(x)
    bits, x = bits[finite], x[finite]
    rng = np.random.default_rng(7)
    gammas = [np.float32(1.0), np.float32(0.828125), np.float32(2.0 ** -20),
              np.float32(0.7978846), np.float32(3.0), np.float32(rng.uniform(0.1, 5))]
    if dtype == ot.BF16:
        gammas.append(np.float32(1e30))
    sub = rng.choice(x.size, size=6000, replace=False)
    # always include the values sitting right at the thresholds
    for g in gammas:
        d = ot.divisor(g, 0.0)
        codes = ot.ternary_codes(x, g, 0.0)
        dd = Fraction(float(d))
        near = np.nonzero(np.abs(np.abs(x) - 0.5 * float(d)) <= 2e-3 * float(d) + 1e-300)[0]
        for i in np.unique(np.concatenate([sub, near])):
            assert codes[i] == _exact_code(Fraction(float(x[i])), dd), (hex(bits[i]), float(d))


def test_ties_go_to_even_and_zero_divisor():
    x = np.array([0.5, -0.5, 1.5, -1.5, 2.5])
    assert ot.ternary_codes(x, np.float32(1.0), 0.0).tolist() == [0, 0, 1, -1, 1]
    assert ot.ternary_codes(np.zeros(4), np.float32(0.0), 0.0).tolist() == [0, 0, 0, 0]


def test_closed_forms_for_standard_normal():
    rng = np.random.default_rng(11)
    x = rng.standard_normal(1_000_000).astype(np.float16).astype(np.float64)
    gamma = ot.absmean_gamma(x)
    assert abs(float(gamma) - math.sqrt(2 / math.pi)) < 4e-3        # E|X| = sqrt(2/pi)
    codes = ot.ternary_codes(x, gamma, 1e-5)
    p0 = np.mean(codes == 0)
    expect = math.erf(0.5 * math.sqrt(2 / math.pi) / math.sqrt(2))   # P(|X| < gamma/2) = 0.3101
    assert abs(expect - 0.3101) < 1e-4
    assert abs(p0 - expect) < 3e-3
    assert abs(np.mean(codes == 1) - np.mean(codes == -1)) < 3e-3    # symmetry


def test_pack_invariants_and_round_trip():
    rng = np.random.default_rng(3)
    q = rng.integers(-1, 2, size=(37, 128)).astype(np.int8)
    b = ot.pack_flat(q)
    assert b.shape == (37, 32)                      # N/4 bytes: 2.0 bits per element
    fields = np.stack([(b >> (2 * i)) & 3 for i in range(4)])
    assert not np.any(fields == 3)                  # 0b11 is never written
    assert np.array_equal(ot.unpack_flat(b), q)
    # first element sits in the two least significant bits
    one = np.zeros((1, 4), dtype=np.int8)
    one[0, 0] = 1
    assert ot.pack_flat(one).tolist() == [[0b01010110]]


def test_v_tile_hand_example_and_inverse():
    g = golden("v_tile_example.json")
    for case in g["cases"]:
        dim = case["dim"]
        codes = np.zeros((16, dim), dtype=np.int8)
        for t, d, c in case["codes"]:
            codes[t, d] = c
        tile = ot.v_tile(codes)
        assert tile.size == case["tile_bytes"]
        want = np.full(case["tile_bytes"], 0x55, dtype=np.uint8)
        for k, v in case["bytes_not_0x55"].items():
            want[int(k)] = v
        assert tile.tolist() == want.tolist(), dim
    rng = np.random.default_rng(5)
    for dim in (64, 128, 256):
        q = rng.integers(-1, 2, size=(64, dim)).astype(np.int8)
        assert np.array_equal(ot.v_tile_codes(ot.v_tile(q), 64, dim), q)
        # each unit's chunk bytes depend only on that unit's tokens
        q2 = q.copy()
        q2[20] = 0
        a, b = ot.v_tile(q).reshape(4, -1), ot.v_tile(q2).reshape(4, -1)
        assert np.array_equal(np.delete(a, 1, axis=0), np.delete(b, 1, axis=0))


# ------------------------------------------------------------ fp8 / fp16 ---

def test_e4m3fn_hand_points():
    pts = golden("e4m3fn_points.json")["points"]
    v = np.array([p[0] for p in pts], dtype=np.float64)
    assert of.e4m3fn_encode(v).tolist() == [p[1] for p in pts]


def test_e4m3fn_table_definition():
    assert of.e4m3fn_value(0x38) == 1.0
    assert of.e4m3fn_value(0x7E) == 448.0
    assert of.e4m3fn_value(0x01) == 2.0 ** -9
    assert math.isnan(of.e4m3fn_value(0x7F))
    assert np.all(np.diff(of.E4M3_POS) > 0)
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]
    assert np.array_equal(of.e4m3fn_encode(of.e4m3fn_decode(codes)), codes)


def test_e4m3fn_matches_torch_in_range():
    """torch's float8_e4m3fn cast (RNE) agrees wherever it does not overflow."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = ot.values16(bits, ot.BF16)
    x = x[np.isfinite(x) & (np.abs(x) <= 448.0)]
    rng = np.random.default_rng(1)
    extra = rng.uniform(-448, 448, 200000)
    x = np.concatenate([x, extra, extra / 300.0]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(of.fp8_encode_input(x, 1.0), ref)


def test_fp8_scale_divides_in_float32():
    x = np.array([3.0, -7.0], dtype=np.float64)
    # 3/2 = 1.5 (code 0x3C), -7/2 = -3.5 (code 0xC6)
    assert of.fp8_encode_input(x, 2.0).tolist() == [0x3C, 0xC6]
    assert of.fp8_dequantize(np.array([0x3C]), 2.0).tolist() == [3.0]


def test_f16_route_hand_points_and_torch():
    pts = golden("f16_route_points.json")["points"]
    got = of.f16_encode_input(np.array([p[0] for p in pts], dtype=np.uint16), 1)
    assert got.tolist() == [p[1] for p in pts]
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float16)
    ref = ref.view(torch.int16).numpy().view(np.uint16)
    fin = np.isfinite(ot.values16(bits, ot.BF16))
    assert np.array_equal(of.f16_encode_input(bits, 1)[fin], ref[fin])
    assert np.array_equal(of.f16_encode_input(bits[:100], 0), bits[:100])


# ----------------------------------------------------------- page layout ---

def test_page_format_rule_hand_example():
    spec = oc.CacheSpec(n_kv_heads=1, head_dim=4, block_size=16, sink_tokens=4, sink_format=oc.F16,
                        recent_tokens=256, recent_format=oc.FP8E4M3)
    # one append of 1000 tokens: page 0 sink; pages meeting [744, 1000) -> 46..62 fp8
    fmts = [oc.new_page_format(spec, p, 1000) for p in range(63)]
    assert fmts[0] == oc.F16
    assert fmts[1:46] == [oc.TERNARY2] * 45
    assert fmts[46:] == [oc.FP8E4M3] * 17
    rng = np.random.default_rng(0)
    k = rng.integers(0, 1 << 14, size=(1020, 1, 4)).astype(np.uint16)
    enc = oc.encode_sequence(spec, k, k, ot.F16, [(0, 1000), (1000, 20)])
    assert enc.page_format[62] == oc.FP8E4M3 and enc.page_format[63] == oc.FP8E4M3
    assert enc.token_format[1005] == oc.FP8E4M3 and enc.token_format[15] == oc.F16
    # with no recent tier the partly filled last page is ternary and cannot grow
    spec0 = oc.CacheSpec(n_kv_heads=1, head_dim=4, block_size=16)
    with pytest.raises(oc.AlignError):
        oc.encode_sequence(spec0, k, k, ot.F16, [(0, 1000), (1000, 20)])


def test_gamma_is_per_append_over_ternary_tokens_only():
    spec = oc.CacheSpec(n_kv_heads=1, head_dim=4, block_size=16, sink_tokens=4, sink_format=oc.F16)
    x = np.zeros((48, 1, 4))
    x[:16] = 100.0      # sink page (fp16): must not enter gamma
    x[16:32] = 1.0
    x[32:48] = 3.0
    bits = f16_bits(x)
    enc = oc.encode_sequence(spec, bits, bits, ot.F16, [(0, 32), (32, 16)])
    assert float(enc.gamma[0][0]) == 1.0       # tokens 16..31 only
    assert float(enc.gamma[1][0]) == 3.0       # second call has its own gamma
    assert np.all(enc.k_hat[:16] == 100.0)


def test_page_tiles_layout():
    spec = oc.CacheSpec(n_kv_heads=2, head_dim=64, block_size=16)
    rng = np.random.default_rng(2)
    k = f16_bits(rng.standard_normal((16, 2, 64)))
    enc = oc.encode_sequence(spec, k, k, ot.F16, [(0, 16)])
    b = oc.page_tiles(spec, enc, 0)
    assert b.size == oc.page_bytes(spec, oc.TERNARY2) == 2 * 2 * 16 * 64 // 4
    kt = 16 * 64 // 4
    assert np.array_equal(b[kt:2 * kt].reshape(16, 16), ot.pack_flat(enc.k_code[:, 1]))
    assert np.array_equal(ot.v_tile_codes(b[2 * kt:3 * kt], 16, 64), enc.v_code[:, 0])


def test_storage_ratio_matches_page():
    g = golden("storage_ratio.json")
    spec = oc.CacheSpec(**g["page_shape"])
    r = oc.storage_ratio_vs_f16(spec, [oc.TERNARY2] * 256)
    assert round(r, 2) == g["ratio_printed"]
    assert 7.9 <= r <= 8.0
    per_elem_bits = 8 * oc.page_bytes(spec, oc.TERNARY2) / (2 * 2 * 16 * 128)
    assert per_elem_bits == g["bits_per_element"]


# ------------------------------------------------------------- attention ---

def test_attended_set_hand_cases():
    assert oa.attended_tokens(10, 4, 3).tolist() == [0, 1, 2, 3, 7, 8, 9]
    assert oa.attended_tokens(5, 4, 3).tolist() == [0, 1, 2, 3, 4]
    assert oa.attended_tokens(3, 4, 0).tolist() == [0, 1, 2]
    assert oa.attended_tokens(10, 0, 0).tolist() == []
    assert oa.attended_tokens(10, 4, -1).tolist() == list(range(10))
    assert len(oa.attended_tokens(4096, 4, 256)) == 260


def _sdpa(q, k, v, mask=None, scale=None):
    """torch SDPA in float64 with KV heads repeated for GQA; q [Hq,D], k/v [T,Hkv,D]."""
    hq, hkv = q.shape[0], k.shape[1]
    kk = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2))).repeat_interleave(hq // hkv, 0)
    vv = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2))).repeat_interleave(hq // hkv, 0)
    qq = torch.from_numpy(q)[:, None, :]
    m = None if mask is None else torch.from_numpy(mask)[None, None, :].expand(hq, 1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=m, scale=scale)
    return o[:, 0, :].numpy()


def test_attention_full_context_is_sdpa():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((8, 64))
    k = rng.standard_normal((100, 2, 64))
    v = rng.standard_normal((100, 2, 64))
    ours = oa.decode_attention(q, k, v, 100, 4, -1)
    assert np.allclose(ours, _sdpa(q, k, v), atol=1e-12)
    ours = oa.decode_attention(q, k, v, 100, 0, -1, scale=0.3)
    assert np.allclose(ours, _sdpa(q, k, v, scale=0.3), atol=1e-12)


def test_attention_sinks_and_window_is_masked_sdpa():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((16, 128))
    k = rng.standard_normal((300, 4, 128))
    v = rng.standard_normal((300, 4, 128))
    for length, s, w in [(300, 4, 256), (300, 0, 17), (250, 4, 1), (300, 20, 0)]:
        mask = np.zeros(300, dtype=bool)
        mask[: min(s, length)] = True
        mask[max(0, length - w): length] = True
        ours = oa.decode_attention(q, k, v, length, s, w)
        assert np.allclose(ours, _sdpa(q, k, v, mask), atol=1e-12)


def test_attention_closed_forms():
    rng = np.random.default_rng(8)
    k = rng.standard_normal((50, 2, 64))
    v = rng.standard_normal((50, 2, 64))
    zero = np.zeros((4, 64))
    o = oa.decode_attention(zero, k, v, 50, 4, 10)       # q = 0: mean of V over A
    idx = [0, 1, 2, 3] + list(range(40, 50))
    assert np.allclose(o[0], v[idx, 0].mean(0)) and np.allclose(o[3], v[idx, 1].mean(0))
    q = rng.standard_normal((4, 64))
    o = oa.decode_attention(q, k, v, 1, 4, 10)            # a single attended token
    assert np.allclose(o[:2], v[0, 0]) and np.allclose(o[2:], v[0, 1])
    o = oa.decode_attention(q, k, v, 50, 0, 1)
    assert np.allclose(o[:2], v[49, 0])


def test_attention_over_dequantised_cache_equals_sdpa():
    """End to end on a tiny cache: encode, dequantise, attend == SDPA on the dequantised values."""
    spec = oc.CacheSpec(n_kv_heads=2, head_dim=64, block_size=16, sink_tokens=4, sink_format=oc.F16,
                        recent_tokens=32, recent_format=oc.FP8E4M3)
    rng = np.random.default_rng(9)
    k = f16_bits(rng.standard_normal((200, 2, 64)))
    v = f16_bits(rng.standard_normal((200, 2, 64)))
    enc = oc.encode_sequence(spec, k, v, ot.F16, [(0, 150), (150, 50)])
    q = rng.standard_normal((8, 64))
    mask = np.zeros(200, dtype=bool)
    mask[:4] = True
    mask[100:] = True
    ours = oa.decode_attention(q, enc.k_hat, enc.v_hat, 200, 4, 100)
    assert np.allclose(ours, _sdpa(q, enc.k_hat, enc.v_hat, mask), atol=1e-12)
    # dequantised ternary values are gamma * code, a bounded perturbation of the input
    tern = enc.token_format == oc.TERNARY2
    assert set(np.unique(enc.k_hat[tern] / float(enc.gamma[0][0]))) <= {-1.0, 0.0, 1.0}
