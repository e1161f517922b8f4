"""Pins the tests' vectorised page reader (tests/page_codec.py) to the oracle's
element-by-element tile functions, on the CPU, before the GPU parity tests use
it to read every page back from the device."""
import numpy as np
import pytest

from oracle import cache as oc
from oracle import ternary as ot

import page_codec as pc


@pytest.mark.parametrize("dim", [64, 128, 256])
@pytest.mark.parametrize("bs", [16, 32])
def test_value_codes_invert_oracle_v_tile(dim, bs):
    rng = np.random.default_rng(dim * 100 + bs)
    for _ in range(3):
        codes = rng.integers(-1, 2, size=(bs, dim)).astype(np.int8)
        tile = ot.v_tile(codes)
        assert np.array_equal(pc.value_codes(tile, bs, dim), codes)
        assert np.array_equal(pc.value_codes(tile, bs, dim), ot.v_tile_codes(tile, bs, dim))


@pytest.mark.parametrize("dim", [64, 128, 256])
def test_value_codes_single_field_positions(dim):
    """One nonzero code at a time lands where the oracle puts it (catches a swapped token or dimension)."""
    bs = 16
    for t in range(bs):
        for d in range(0, dim, 7):
            codes = np.zeros((bs, dim), np.int8)
            codes[t, d] = 1
            assert np.array_equal(pc.value_codes(ot.v_tile(codes), bs, dim), codes), (t, d)


def test_key_codes_invert_oracle_k_tile():
    rng = np.random.default_rng(5)
    codes = rng.integers(-1, 2, size=(3, 32, 128)).astype(np.int8)
    tiles = np.stack([ot.k_tile(c) for c in codes])
    assert np.array_equal(pc.key_codes(tiles, 128), codes)


def test_reserved_field_is_rejected():
    with pytest.raises(ValueError):
        pc.key_codes(np.full((1, 16, 16), 0xFF, np.uint8), 64)
    with pytest.raises(ValueError):
        pc.value_codes(np.full(16 * 16, 0xC0, np.uint8), 16, 64)


@pytest.mark.parametrize("dim,bs", [(64, 32), (128, 16)])
def test_lossless_pages_decode_to_the_oracle_bits(dim, bs):
    """Lossless sink and recent pages (coded groups, a raw group, zero padding past the end)
    read back to the input bits, as the oracle encoded them."""
    spec = oc.CacheSpec(n_kv_heads=2, head_dim=dim, block_size=bs, sink_tokens=20, sink_format=oc.LOSSLESS,
                        recent_tokens=24, recent_format=oc.LOSSLESS)
    rng = np.random.default_rng(dim + bs)
    T = 16 * 7 + 3
    x = rng.standard_normal((2, T, 2, dim)).astype(np.float32)
    x[0, 0:16, 1] *= np.where(rng.random((16, dim)) < 0.6, 1e30, 1e-30)   # a group of escapes: raw
    x[1, 3, 0, 5] = 0.0
    bits = ((x.view(np.uint32) + 0x7FFF + ((x.view(np.uint32) >> 16) & 1)) >> 16).astype(np.uint16)
    kb, vb = bits[0], bits[1]
    enc = oc.encode_sequence(spec, kb, vb, ot.BF16, [(0, T)])
    assert oc.LOSSLESS in enc.page_format and oc.TERNARY2 in enc.page_format
    n_pages = len(enc.page_format)
    stride = oc.page_bytes(spec, oc.LOSSLESS)
    buf = np.zeros((n_pages, stride), np.uint8)
    for p in range(n_pages):
        t = oc.page_tiles(spec, enc, p)
        buf[p, :t.size] = t
    got = pc.decode_pages(buf, np.array(enc.page_format), T, 2, dim, bs)
    for name in ("k_lossless", "v_lossless", "k_code", "v_code"):
        assert np.array_equal(got[name], getattr(enc, name)), name
    ls = enc.token_format == oc.LOSSLESS
    assert np.array_equal(got["k_lossless"][ls], kb[ls]) and np.array_equal(got["v_lossless"][ls], vb[ls])
    # the group of head 1's keys in unit 0 holds escapes beyond its exception room: raw
    assert buf[0, (32 * dim + 16) * (bs // 16) + 1] == 1


@pytest.mark.parametrize("dynamic", [False, True])
def test_decode_pages_matches_oracle_encoding(dynamic):
    """A mixed-format sequence encoded by the oracle, laid out as the device reads it back,
    decodes to the oracle's per-token arrays, with code-0 padding in the last ternary page."""
    spec = oc.CacheSpec(n_kv_heads=2, head_dim=64, block_size=16, sink_tokens=4, sink_format=oc.F16,
                        recent_tokens=40, recent_format=oc.FP8E4M3, fp8_dynamic=dynamic)
    rng = np.random.default_rng(11)
    T = 16 * 9 + 5
    x = rng.standard_normal((2, T, 2, 64)).astype(np.float16)
    kb, vb = x[0].view(np.uint16), x[1].view(np.uint16)
    calls = [(0, 16 * 5), (16 * 5, T - 16 * 5)]
    enc = oc.encode_sequence(spec, kb, vb, ot.F16, calls)
    n_pages = len(enc.page_format)
    stride = oc.page_bytes(oc.CacheSpec(2, 64, 16), oc.F16)
    buf = np.zeros((n_pages, stride), np.uint8)
    for p in range(n_pages):
        t = oc.page_tiles(spec, enc, p)
        buf[p, :t.size] = t
    got = pc.decode_pages(buf, np.array(enc.page_format), T, 2, 64, 16, fp8_dynamic=dynamic)
    assert set(enc.page_format) == {0, 1, 2}
    for name in ("k_code", "v_code", "k_fp8", "v_fp8", "k_f16", "v_f16"):
        assert np.array_equal(got[name], getattr(enc, name)), name
    if dynamic:
        assert np.array_equal(got["k_fp8_scale"], enc.k_fp8_scale)
        assert np.array_equal(got["v_fp8_scale"], enc.v_fp8_scale)
    # the last page is fp8 here (recent tier): no ternary padding to report
    assert got["k_pad"].size == 0
    # an all-ternary sequence ending inside a page reports the code-0 padding
    spec_t = oc.CacheSpec(n_kv_heads=2, head_dim=64, block_size=16)
    enc_t = oc.encode_sequence(spec_t, kb, vb, ot.F16, [(0, T)])
    buf_t = np.zeros((n_pages, stride), np.uint8)
    for p in range(n_pages):
        t = oc.page_tiles(spec_t, enc_t, p)
        buf_t[p, :t.size] = t
    got_t = pc.decode_pages(buf_t, np.array(enc_t.page_format), T, 2, 64, 16)
    assert np.array_equal(got_t["k_code"], enc_t.k_code) and np.array_equal(got_t["v_code"], enc_t.v_code)
    assert got_t["k_pad"].shape == (16 * n_pages - T, 2, 64) and not got_t["k_pad"].any()
    assert not got_t["v_pad"].any()
    # one changed code field in a value tile is seen
    pos = 2 * 16 * 16 + 7                      # page 3: a byte of the first value tile
    field = buf_t[3, pos] & 3
    buf_t[3, pos] = (buf_t[3, pos] & 0xFC) | (0 if field else 2)
    bad = pc.decode_pages(buf_t, np.array(enc_t.page_format), T, 2, 64, 16)
    assert np.sum(bad["v_code"] != enc_t.v_code) == 1
