"""CPU checks of the library boundary and the HIP-free host logic.

* libvk.so loads and exports every entry point include/vk.h declares;
* configuration checks and size arithmetic (no device call);
* the page allocator, tier router and planners (host_state.cpp, through a
  g++-built test shim) against the oracle's format rule and attended set.
"""
import ctypes
import json
import os
import re
import subprocess
import sys
import tempfile

import numpy as np
import pytest

from bit_ternary_attention_amd import vk
from oracle import attention as oa
from oracle import cache as oc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vk.h")
CSRC = os.path.join(ROOT, "bit_ternary_attention_amd", "csrc")


def declared_entry_points():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"VK_API\s+[\w\s\*]+?\b(vk_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_entry_points()
    assert len(names) >= 14
    L = vk.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(vk.EXPORTS), "binding and header disagree"
    out = subprocess.run(["nm", "-D", "--defined-only", vk.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported
    assert all(e.startswith("vk_") for e in exported), "only vk_* symbols are exported"


def base_cfg(**kw):
    d = dict(n_layers=2, n_kv_heads=2, n_q_heads=8, head_dim=128, block_size=16, max_seqs=4,
             max_tokens_per_seq=1024, pages_ternary=100, pages_fp8=10, pages_f16=5)
    d.update(kw)
    return vk.make_config(**d)


def test_config_defaults():
    c = vk.make_config()
    assert c.sink_tokens == 4 and c.sink_format == vk.FMT_TERNARY2 and c.recent_tokens == 0
    assert c.recent_format == vk.FMT_FP8E4M3 and abs(c.eps - 1e-5) < 1e-12 and c.fp8_scale == 1.0


@pytest.mark.parametrize("bad", [dict(n_layers=0), dict(n_q_heads=12), dict(n_q_heads=2, n_kv_heads=4),
                                 dict(n_q_heads=48, n_kv_heads=2), dict(head_dim=96), dict(head_dim=512), dict(block_size=24),
                                 dict(block_size=8), dict(max_seqs=0), dict(sink_tokens=-1),
                                 dict(sink_format=4), dict(pages_fp8=-1), dict(pages_lossless=-1),
                                 dict(decode_kernel=1, sink_format=3), dict(eps=-1.0),
                                 dict(head_dim=256, sink_format=3),
                                 dict(head_dim=256, recent_tokens=16, recent_format=3),
                                 dict(fp8_scale=0.0), dict(decode_kernel=3), dict(eps=float("nan"))])
def test_config_rejected(bad):
    with pytest.raises(vk.VkError) as e:
        vk.device_bytes(base_cfg(**bad))
    assert e.value.status == vk.ERR_ARG


def test_head_dim_256_config():
    """Head dim 256 is taken with every decode kernel; its pages scale with D."""
    for kern in (0, 1, 2):
        c = base_cfg(head_dim=256, decode_kernel=kern, recent_tokens=16)
        assert vk.device_bytes(c) > vk.device_bytes(base_cfg(decode_kernel=kern, recent_tokens=16))
        assert vk.page_bytes(c, vk.FMT_TERNARY2) == 2 * 2 * 16 * 256 // 4
        assert vk.page_bytes(c, vk.FMT_FP8E4M3) == 2 * 2 * 16 * 256
        assert vk.page_bytes(c, vk.FMT_F16) == 2 * 2 * 16 * 256 * 2


def test_sizes():
    c = base_cfg()
    assert vk.page_bytes(c, vk.FMT_TERNARY2) == 2 * 2 * 16 * 128 // 4
    assert vk.page_bytes(c, vk.FMT_FP8E4M3) == 2 * 2 * 16 * 128
    assert vk.page_bytes(c, vk.FMT_F16) == 2 * 2 * 16 * 128 * 2
    assert vk.page_bytes(c, vk.FMT_LOSSLESS) == 2 * 2 * (32 * 128 + 16)      # one 16-token group per tile
    assert vk.page_bytes(base_cfg(block_size=64, head_dim=64), vk.FMT_LOSSLESS) == 2 * 2 * 4 * (32 * 64 + 16)
    assert vk.page_bytes(c, 4) == 0
    total = vk.device_bytes(c)
    pools = 2 * (100 * 2048 + 10 * 8192 + 5 * 16384)
    assert total >= pools + 2 * 100 * 8 + 4 * 64 * 4
    # pools dominate a large cache: no hidden dense copy of the KV
    big = base_cfg(pages_ternary=1 << 20, pages_fp8=0, pages_f16=0)
    assert vk.device_bytes(big) - 2 * (1 << 20) * (2048 + 8) < 64 << 20
    assert vk.quantize_pack_workspace_bytes(1 << 20) >= 8 * 64


# ------------------------------------------------------------ host shim ---

# With VK_HS_SANITIZE=1 the shim is built with AddressSanitizer and UndefinedBehaviorSanitizer
# (the process must then have libasan preloaded; test_host_logic_under_sanitizers below runs
# the shim tests that way in a child process).
SANITIZE = os.environ.get("VK_HS_SANITIZE") == "1"
SANITIZER_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
SHIM_TESTS = ("tier_router or capacity_align or allocator or attended_units or route_counters or mixed_ranges "
              "or split_plan or retier_plan or retier_capacity or eviction")


@pytest.fixture(scope="module")
def hs():
    d = tempfile.mkdtemp(prefix="vk_hs_")
    so = os.path.join(d, "libhs.so")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-shared", "-fPIC", *(SANITIZER_FLAGS if SANITIZE else []),
                    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
                    os.path.join(ROOT, "tests", "native", "host_shim.cpp"),
                    os.path.join(CSRC, "host_state.cpp"), "-o", so], check=True)
    L = ctypes.CDLL(so)
    P = ctypes.POINTER
    L.hs_create.restype = ctypes.c_void_p
    L.hs_create.argtypes = [P(vk.CacheConfig), ctypes.c_char_p, ctypes.c_int]
    L.hs_destroy.argtypes = [ctypes.c_void_p]
    L.hs_append.argtypes = [ctypes.c_void_p, ctypes.c_int, P(ctypes.c_int), ctypes.c_int, P(ctypes.c_int),
                            P(ctypes.c_longlong), ctypes.c_char_p, ctypes.c_int]
    for n in ("hs_length", "hs_n_pages"):
        getattr(L, n).argtypes = [ctypes.c_void_p, ctypes.c_int]
    L.hs_page_entry.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int]
    L.hs_free_pages.restype = ctypes.c_longlong
    L.hs_free_pages.argtypes = [ctypes.c_void_p, ctypes.c_int]
    L.hs_tokens_stored.restype = ctypes.c_longlong
    L.hs_tokens_stored.argtypes = [ctypes.c_void_p, ctypes.c_int]
    L.hs_count_units.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, P(ctypes.c_longlong)]
    L.hs_mixed_ranges.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, P(ctypes.c_int)]
    L.hs_reset.argtypes = [ctypes.c_void_p, ctypes.c_int, P(ctypes.c_int)]
    L.hs_attended_units.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P(ctypes.c_int)]
    L.hs_retier.argtypes = [ctypes.c_void_p, ctypes.c_int, P(ctypes.c_int), P(ctypes.c_int), ctypes.c_int,
                            P(ctypes.c_int), ctypes.c_char_p, ctypes.c_int]
    L.hs_evict.argtypes = [ctypes.c_void_p, ctypes.c_int, P(ctypes.c_int), ctypes.c_int, P(ctypes.c_longlong)]
    L.hs_check_decode.argtypes = [ctypes.c_void_p, ctypes.c_int, P(ctypes.c_int), ctypes.c_int]
    L.hs_plan_splits.argtypes = [ctypes.c_longlong, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    L.hs_balance_splits.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_longlong] + [ctypes.c_int] * 6 + \
        [ctypes.POINTER(ctypes.c_int)]
    L.hs_plan_decode_order.argtypes = [P(ctypes.c_int), P(ctypes.c_longlong), ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int, P(ctypes.c_ushort)]
    return L


class Host:
    def __init__(self, L, cfg):
        self.L, self.cfg = L, cfg
        err = ctypes.create_string_buffer(256)
        self.h = L.hs_create(ctypes.byref(cfg), err, 256)
        assert self.h, err.value

    def append(self, ids, n):
        arr = (ctypes.c_int * len(ids))(*ids)
        rng = (ctypes.c_int * (2 * len(ids)))()
        newp = (ctypes.c_longlong * 3)()
        err = ctypes.create_string_buffer(256)
        st = self.L.hs_append(self.h, len(ids), arr, n, rng, newp, err, 256)
        return st, [(rng[2 * i], rng[2 * i + 1]) for i in range(len(ids))], list(newp), err.value.decode()

    def retier(self, ids):
        arr = (ctypes.c_int * len(ids))(*ids)
        buf = (ctypes.c_int * 4 * 4096)()
        n = ctypes.c_int(0)
        err = ctypes.create_string_buffer(256)
        st = self.L.hs_retier(self.h, len(ids), arr, ctypes.cast(buf, ctypes.POINTER(ctypes.c_int)), 4096,
                              ctypes.byref(n), err, 256)
        flat = list(ctypes.cast(buf, ctypes.POINTER(ctypes.c_int))[:4 * n.value])
        return st, [tuple(flat[4 * i:4 * i + 4]) for i in range(n.value)], err.value.decode()

    def evict(self, ids, window):
        arr = (ctypes.c_int * len(ids))(*ids)
        n = ctypes.c_longlong(0)
        st = self.L.hs_evict(self.h, len(ids), arr, window, ctypes.byref(n))
        return st, n.value

    def check_decode(self, ids, window):
        arr = (ctypes.c_int * len(ids))(*ids)
        return self.L.hs_check_decode(self.h, len(ids), arr, window)

    def pages(self, s):
        return [self.L.hs_page_entry(self.h, s, p) for p in range(self.L.hs_n_pages(self.h, s))]

    def free(self):
        return [self.L.hs_free_pages(self.h, f) for f in range(3)]

    def __del__(self):
        self.L.hs_destroy(self.h)


def spec_of(cfg):
    return oc.CacheSpec(n_kv_heads=cfg.n_kv_heads, head_dim=cfg.head_dim, block_size=cfg.block_size,
                        sink_tokens=cfg.sink_tokens, sink_format=cfg.sink_format,
                        recent_tokens=cfg.recent_tokens, recent_format=cfg.recent_format)


@pytest.mark.parametrize("bs,S,sinkf,R,recf", [(16, 4, 2, 256, 1), (16, 4, 0, 0, 1), (32, 40, 2, 33, 1),
                                               (64, 0, 0, 100, 2), (16, 20, 1, 16, 0)])
def test_tier_router_matches_oracle(hs, bs, S, sinkf, R, recf):
    cfg = base_cfg(block_size=bs, sink_tokens=S, sink_format=sinkf, recent_tokens=R, recent_format=recf,
                   max_tokens_per_seq=4096, pages_ternary=4000, pages_fp8=4000, pages_f16=4000, max_seqs=2)
    h = Host(hs, cfg)
    spec = spec_of(cfg)
    rng = np.random.default_rng(bs + S + R)
    calls, length = [], 0
    while length < 3000:
        n = int(rng.integers(1, 400))
        if length % bs and oc.new_page_format(spec, length // bs, length) == oc.TERNARY2:
            n = bs - length % bs + int(rng.integers(0, 3)) * bs   # never extend a ternary page
        bits = np.zeros((length + n, 1, 4), dtype=np.uint16)
        try:
            enc = oc.encode_sequence(spec, bits, bits, 0, calls + [(length, n)])
        except oc.AlignError:
            st, _, _, _ = h.append([1], n)
            assert st == vk.ERR_ALIGN
            break
        st, rngs, newp, err = h.append([1], n)
        assert st == 0, err
        fmts = [p >> 30 & 3 for p in h.pages(1)]
        assert fmts == enc.page_format
        tern = np.nonzero(enc.token_format[length:length + n] == oc.TERNARY2)[0]
        if tern.size:
            assert rngs[0] == (tern[0], tern[-1] + 1) and tern.size == tern[-1] + 1 - tern[0]
        else:
            assert rngs[0][0] == rngs[0][1]
        calls.append((length, n))
        length += n
        assert hs.hs_length(h.h, 1) == length
        for f in range(3):
            assert hs.hs_tokens_stored(h.h, f) == int(np.sum(enc.token_format == f))


def test_capacity_align_and_argument_errors_leave_state_unchanged(hs):
    cfg = base_cfg(pages_ternary=10, pages_fp8=2, pages_f16=1, sink_format=2, recent_tokens=16)
    h = Host(hs, cfg)
    st, _, newp, _ = h.append([0, 1], 64)     # per seq: page 0 f16, pages 1-2 ternary, page 3 fp8
    assert st == vk.ERR_CAPACITY               # two f16 pages needed, one in the pool
    assert h.free() == [10, 2, 1] and hs.hs_length(h.h, 0) == 0
    st, _, newp, err = h.append([0], 64)
    assert st == 0 and newp == [2, 1, 1], err
    assert h.free() == [8, 1, 0]
    st, *_ = h.append([0, 0], 1)
    assert st == vk.ERR_ARG                    # repeated id
    st, *_ = h.append([7], 1)
    assert st == vk.ERR_ARG                    # id out of range
    st, *_ = h.append([0], 2000)
    assert st == vk.ERR_ARG                    # beyond max_tokens_per_seq
    cfg0 = base_cfg(recent_tokens=0)
    h0 = Host(hs, cfg0)
    assert h0.append([2], 20)[0] == 0          # page 1 ternary, 4 of 16 tokens filled
    st, _, _, err = h0.append([2], 5)
    assert st == vk.ERR_ALIGN and "ternary" in err
    assert hs.hs_length(h0.h, 2) == 20


def test_allocator_shuffle_and_reset(hs):
    seq = Host(hs, base_cfg(page_shuffle_seed=0, recent_tokens=0, sink_tokens=0))
    assert seq.append([0], 160)[0] == 0
    assert [p & 0x3FFFFFFF for p in seq.pages(0)] == list(range(10))
    a = Host(hs, base_cfg(page_shuffle_seed=1004, sink_tokens=0, max_tokens_per_seq=1600))
    b = Host(hs, base_cfg(page_shuffle_seed=1004, sink_tokens=0, max_tokens_per_seq=1600))
    c = Host(hs, base_cfg(page_shuffle_seed=7, sink_tokens=0, max_tokens_per_seq=1600))
    for x in (a, b, c):
        assert x.append([0], 1600)[0] == 0
    pa, pb, pc = ([p & 0x3FFFFFFF for p in x.pages(0)] for x in (a, b, c))
    assert pa == pb and pa != pc and pa != list(range(100))
    assert sorted(pa) == list(range(100))      # a permutation of the whole pool
    assert a.free()[0] == 0
    arr = (ctypes.c_int * 1)(0)
    assert hs.hs_reset(a.h, 1, arr) == 0
    assert a.free()[0] == 100 and hs.hs_length(a.h, 0) == 0
    assert a.append([0], 1600)[0] == 0         # freed pages are reusable


def test_attended_units_match_oracle(hs):
    out = (ctypes.c_int * 3)()
    rng = np.random.default_rng(0)
    cases = [(1, 4, 256), (4, 4, 0), (17, 4, 0), (260, 4, 256), (261, 4, 256), (4096, 4, 256), (40, 0, 1),
             (100, 30, 10), (100, 4, -1), (33, 40, 5), (512, 4, 256)]
    cases += [(int(rng.integers(1, 3000)), int(rng.integers(0, 40)), int(rng.integers(-1, 600))) for _ in range(400)]
    for L, S, W in cases:
        if S == 0 and W == 0:
            continue
        hs.hs_attended_units(L, S, W, out)
        a_end, b0, b1 = out[0], out[1], out[2]
        units = set(range(a_end)) | set(range(b0, b1))
        assert a_end <= b0 <= b1 or (b0 == b1)
        want = {int(t) // 16 for t in oa.attended_tokens(L, S, W)}
        assert units == want, (L, S, W)


def test_route_counters_match_page_formats(hs):
    cfg = base_cfg(sink_format=2, recent_tokens=256, recent_format=1, max_tokens_per_seq=4096,
                   pages_ternary=400, pages_fp8=100, pages_f16=10, max_seqs=2)
    h = Host(hs, cfg)
    assert h.append([1], 1000)[0] == 0
    assert h.append([1], 37)[0] == 0
    spec = spec_of(cfg)
    bits = np.zeros((1037, 1, 4), dtype=np.uint16)
    enc = oc.encode_sequence(spec, bits, bits, 0, [(0, 1000), (1000, 37)])
    out = (ctypes.c_longlong * 3)()
    for W in (-1, 256, 100, 0, 1):
        hs.hs_count_units(h.h, 1, W, out)
        units = sorted({int(t) // 16 for t in oa.attended_tokens(1037, 4, W)})
        want = [0, 0, 0]
        for u in units:
            want[enc.page_format[u]] += 1
        assert list(out) == want, W


def _check_mixed_ranges(hs, h, seq, W):
    """The two ranges cover every attended non-ternary unit (logical numbering) and are as short
    as two intervals can be: the span minus the widest gap between runs of such units."""
    L = hs.hs_length(h.h, seq)
    out = (ctypes.c_int * 4)()
    hs.hs_mixed_ranges(h.h, seq, W, out)
    lo0, hi0, lo1, hi1 = list(out)
    bs = h.cfg.block_size
    fmts = [(e >> 30) & 3 for e in h.pages(seq)]
    units = sorted({int(t) // 16 for t in oa.attended_tokens(L, h.cfg.sink_tokens, W)})
    mixed = [i for i, u in enumerate(units) if fmts[u * 16 // bs] != 0]
    assert 0 <= lo0 <= hi0 <= lo1 <= hi1 <= len(units) or (lo1 == hi1 == 0 and hi0 <= len(units)), list(out)
    for i in mixed:
        assert lo0 <= i < hi0 or lo1 <= i < hi1, (seq, W, i, list(out))
    if not mixed:
        assert (hi0 - lo0) + (hi1 - lo1) == 0
        return
    gaps = [b - a - 1 for a, b in zip(mixed, mixed[1:])]
    assert (hi0 - lo0) + (hi1 - lo1) == (mixed[-1] - mixed[0] + 1) - max(gaps + [0]), (seq, W, list(out))


def test_mixed_ranges_cover_every_non_ternary_unit(hs):
    for bs, S, sinkf, R, recf in [(16, 4, 2, 256, 1), (16, 40, 1, 0, 1), (32, 4, 0, 100, 1), (64, 20, 2, 48, 2),
                                  (16, 4, 0, 0, 1)]:
        cfg = base_cfg(block_size=bs, sink_tokens=S, sink_format=sinkf, recent_tokens=R, recent_format=recf,
                       max_tokens_per_seq=4096, pages_ternary=800, pages_fp8=200, pages_f16=50, max_seqs=3)
        h = Host(hs, cfg)
        for n in (1008, 48, 16, 304, 37):  # whole units, then a ragged tail
            assert h.append([0, 2], n)[0] == 0
            for W in (-1, 256, 100, 17, 0, 1):
                if S == 0 and W == 0:
                    continue
                _check_mixed_ranges(hs, h, 0, W)
        if R > 0 and recf == 1:
            assert h.retier([0])[0] == 0    # fp8 pages past the window become ternary
            for W in (-1, 256, 5):
                _check_mixed_ranges(hs, h, 0, W)
        if h.check_decode([2], 300) == 0:
            assert h.evict([2], 300)[0] == 0
            _check_mixed_ranges(hs, h, 2, 300)


def _plan(hs, total, max_units, target, max_splits, min_units, granule=1):
    ups = ctypes.c_int(0)
    n = hs.hs_plan_splits(total, max_units, target, max_splits, min_units, granule, ctypes.byref(ups))
    return n, ups.value


def _balance(hs, n_seqs, max_units, n_cu=256, heads=8, cap=64, mn=32, gr=16):
    """The launch's plan as the library makes it: two blocks per CU wanted, then balanced."""
    items = n_seqs * heads
    base = _plan(hs, items * max_units, max_units, 2 * n_cu, cap, mn, gr)
    ups = ctypes.c_int(0)
    n = hs.hs_balance_splits(base[0], base[1], items, max_units, n_cu, 3, cap, mn, gr, ctypes.byref(ups))
    return base, (n, ups.value)


def test_split_balance(hs):
    # 32 x 32K tokens (2048 units) x 8 KV heads: two blocks on every CU already, kept
    assert _balance(hs, 32, 2048) == ((2, 1024), (2, 1024))
    # 24 sequences: 3 splits put 3 blocks on some CUs and 2 on others; 4 splits, 3 on every CU
    assert _balance(hs, 24, 2048) == ((3, 688), (4, 512))
    # 12 sequences: 6 splits (576 blocks) -> 8 splits (768 blocks, 3 per CU)
    assert _balance(hs, 12, 2048) == ((6, 352), (8, 256))
    # 20 sequences: 4 splits (640 blocks, up to 3 per CU) -> 3 splits (480, at most 2 per CU)
    assert _balance(hs, 20, 2048) == ((4, 512), (3, 688))
    # 4 x 128K tokens and 16 / 8 / 4 sequences of 32K: already even, kept
    for n_seqs, mx in ((4, 8192), (16, 2048), (8, 2048), (4, 2048)):
        base, bal = _balance(hs, n_seqs, mx)
        assert bal == base, (n_seqs, mx, base, bal)
    # launches that do not fill every CU are left alone (small batches, latency-bound)
    for n_seqs, mx in ((1, 17), (1, 300), (2, 64)):
        base, bal = _balance(hs, n_seqs, mx)
        assert bal == base
    # invariants over many shapes: whole granules, the minimum size, the cap, every unit covered,
    # and the busiest CU never holds more units than with the plain plan
    for n_seqs in range(1, 65):
        for mx in (33, 517, 2048, 3001, 8192):
            base, (n, ups) = _balance(hs, n_seqs, mx)
            assert ups % 16 == 0 and (ups >= 32 or (n, ups) == base) and 1 <= n <= 64
            assert n * ups >= mx and (n - 1) * ups < mx
            blocks = lambda s: n_seqs * 8 * s
            if (n, ups) != base:
                k_b, k_n = -(-blocks(base[0]) // 256), -(-blocks(n) // 256)
                assert blocks(n) >= 256 and k_n <= 3 and k_n * ups < k_b * base[1] or k_b == 1


def test_split_plan(hs):
    # 32 sequences x 8 heads x 2048 units, 2048 blocks wanted: 256-unit splits
    assert _plan(hs, 32 * 8 * 2048, 2048, 2048, 64, 32) == (8, 256)
    # few items: the minimum split size rules
    assert _plan(hs, 2 * 17, 17, 2048, 64, 32) == (1, 17)
    # the split cap rules: splits grow to cover the longest sequence
    assert _plan(hs, 4 * 8 * 8192, 8192, 2048, 32, 32) == (32, 256)
    # mixed lengths: the split size follows the total, the count the longest sequence
    n, ups = _plan(hs, 8 * (1024 + 64), 1024, 64, 64, 8)
    assert (n, ups) == (8, 128)  # 136 wanted; 8 splits then cover 1024 units with 128 each
    for total, mx, tgt, cap, mn in [(1, 1, 2048, 64, 32), (10**7, 12345, 2048, 64, 32), (500, 7, 4096, 3, 4)]:
        for gr in (1, 16):
            n, ups = _plan(hs, total, mx, tgt, cap, mn, gr)
            assert 1 <= n <= cap and n * ups >= mx and (n - 1) * ups < mx and ups % gr == 0
    # granule: 32 x 8 x 2048 units in 768 blocks wants 683-unit splits; rounded to 688 (3 splits)
    assert _plan(hs, 32 * 8 * 2048, 2048, 768, 64, 32) == (3, 683)
    assert _plan(hs, 32 * 8 * 2048, 2048, 768, 64, 32, 16) == (3, 688)
    assert _plan(hs, 2 * 17, 17, 2048, 64, 32, 16) == (1, 32)  # 17 units round up to one 32-unit split


@pytest.mark.parametrize("bs,S,sinkf,R", [(16, 4, 2, 256), (16, 4, 1, 16), (32, 40, 2, 33), (64, 0, 0, 100)])
def test_retier_plan_matches_oracle(hs, bs, S, sinkf, R):
    """Pages the host converts (and the free lists afterwards) against the oracle's rule,
    with retiering after random appends; pages already examined are not planned again."""
    cfg = base_cfg(block_size=bs, sink_tokens=S, sink_format=sinkf, recent_tokens=R, recent_format=1,
                   max_tokens_per_seq=4096, pages_ternary=4000, pages_fp8=4000, pages_f16=4000, max_seqs=2)
    h = Host(hs, cfg)
    spec = spec_of(cfg)
    rng = np.random.default_rng(bs + S + R)
    calls, length = [], 0
    bits = np.zeros((4096, 1, 4), dtype=np.uint16)
    converted = set()
    while length < 3500:
        n = int(rng.integers(1, 300))
        if length % bs and oc.new_page_format(spec, length // bs, length) == oc.TERNARY2:
            n = bs - length % bs
        assert h.append([1], n)[0] == 0
        calls.append((length, n))
        length += n
        free_before = h.free()
        enc = oc.encode_sequence(spec, bits[:length], bits[:length], 0, calls)
        want = [p for p in oc.retier_pages(spec, enc) if p not in converted]
        st, tasks, err = h.retier([1])
        assert st == 0, err
        assert [t[1] for t in tasks] == want and all(t[0] == 1 for t in tasks)
        converted |= set(want)
        pages = h.pages(1)
        for slot, page, src, dst in tasks:
            assert pages[page] == dst                    # format 0, pool index dst
        assert h.free() == [free_before[0] - len(tasks), free_before[1] + len(tasks), free_before[2]]
        fmts = [e >> 30 & 3 for e in pages]
        want_fmts = [oc.TERNARY2 if p in converted else f for p, f in enumerate(enc.page_format)]
        assert fmts == want_fmts
        assert h.retier([1])[1] == []                    # nothing left to do
    assert converted


def test_retier_capacity_and_argument_errors(hs):
    cfg = base_cfg(pages_ternary=3, pages_fp8=40, pages_f16=5, sink_format=2, recent_tokens=16,
                   max_tokens_per_seq=1024)
    h = Host(hs, cfg)
    for _ in range(40):                                   # 16 tokens at a time: all fp8 but page 0
        assert h.append([0], 16)[0] == 0
    before = (h.pages(0), h.free())
    st, tasks, err = h.retier([0])
    assert st == vk.ERR_CAPACITY and "ternary" in err     # 38 pages to convert, 3 free
    assert (h.pages(0), h.free()) == before
    assert h.retier([0, 0])[0] == vk.ERR_ARG
    assert h.retier([9])[0] == vk.ERR_ARG
    assert h.retier([1]) == (0, [], "")                   # empty sequence: nothing to do


@pytest.mark.parametrize("bs,S,sinkf,R,W", [(16, 4, 2, 64, 256), (16, 4, 0, 0, 100), (32, 40, 2, 33, 50),
                                            (64, 0, 0, 100, 0), (16, 20, 1, 16, 16)])
def test_eviction_matches_oracle_and_bounds_memory(hs, bs, S, sinkf, R, W):
    """Streaming appends with eviction (and retiering) after each: freed pages match the oracle's
    rule, memory stays bounded, pools recycle, decode windows are checked against freed tokens."""
    cfg = base_cfg(block_size=bs, sink_tokens=S, sink_format=sinkf, recent_tokens=R, recent_format=1,
                   max_tokens_per_seq=60000, pages_ternary=400, pages_fp8=400, pages_f16=40, max_seqs=2)
    h = Host(hs, cfg)
    spec = spec_of(cfg)
    rng = np.random.default_rng(bs + S + R + W)
    length, freed_total = 0, 0
    bound = -(-S // bs) + -(-W // bs) + 1
    while length < 20000:                         # far more tokens than the pools could hold
        n = int(rng.integers(1, 2 * bs + 40))
        if R == 0:
            n = bs * (1 + n % 3)                   # ternary pages are written whole
        elif length < -(-S // bs) * bs and sinkf == oc.TERNARY2:
            n = max(n, -(-S // bs) * bs - length)  # fill the ternary sink pages in one call
        st, _, _, err = h.append([1], n)
        assert st == 0, err
        length += n
        if R:
            assert h.retier([1])[0] == 0
        st, freed = h.evict([1], W)
        assert st == 0
        freed_total += freed
        pages = h.pages(1)
        gone = [p for p, e in enumerate(pages) if e == -1]
        assert gone == oc.evict_pages(spec, length, W)
        assert len(pages) - len(gone) <= bound
        # decode: windows inside the kept tokens pass, wider ones are refused
        if S or W:
            assert h.check_decode([1], W) == 0
        if gone:
            gone_end = (gone[-1] + 1) * bs
            assert h.check_decode([1], -1) == vk.ERR_ARG
            for w2 in (W + 1, W + bs, W + 3 * bs):
                want = vk.ERR_ARG if length - w2 < gone_end else 0
                assert h.check_decode([1], w2) == want, (length, w2, gone_end)
    assert freed_total > 0 and length > 4000
    used = [cfg.pages_ternary - h.free()[0], cfg.pages_fp8 - h.free()[1], cfg.pages_f16 - h.free()[2]]
    assert sum(used) == len([e for e in h.pages(1) if e != -1])
    arr = (ctypes.c_int * 1)(1)
    assert hs.hs_reset(h.h, 1, arr) == 0
    assert h.free() == [cfg.pages_ternary, cfg.pages_fp8, cfg.pages_f16]


def test_eviction_arguments(hs):
    h = Host(hs, base_cfg(recent_tokens=0))
    assert h.append([0], 300)[0] == 0
    assert h.evict([0], -2)[0] == vk.ERR_ARG
    assert h.evict([0, 0], 10)[0] == vk.ERR_ARG
    assert h.evict([5], 10)[0] == vk.ERR_ARG
    assert h.evict([0], -1) == (0, 0)            # the whole context: nothing to free
    assert h.evict([0], 400) == (0, 0)           # the window covers the sequence
    assert h.evict([0], 100) == (0, 11)          # pages 1..11 end by 200 (freed tokens 16..191)
    assert h.evict([0], 100) == (0, 0)           # already freed
    assert h.check_decode([0], 108) == 0         # the window starts at 192
    assert h.check_decode([0], 109) == vk.ERR_ARG and h.check_decode([0], -1) == vk.ERR_ARG


def test_bench_refuses_more_than_one_gpu():
    """bench.py runs on one GPU: --gpus above 1 prints why (one JSON line) and exits with 2."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


@pytest.mark.skipif(SANITIZE, reason="this is the parent of the sanitized run")
def test_host_logic_under_sanitizers():
    """The allocator, router, planner, retier and eviction tests again, in a child process,
    with the host logic built under AddressSanitizer and UndefinedBehaviorSanitizer."""
    libasan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(libasan) or not os.path.exists(libasan):
        pytest.skip("libasan is not available")
    env = dict(os.environ)
    env["LD_PRELOAD"] = libasan + ((":" + env["LD_PRELOAD"]) if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["VK_HS_SANITIZE"] = "1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", os.path.abspath(__file__),
                        "-k", SHIM_TESTS], env=env, capture_output=True, text=True, cwd=ROOT, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail


def test_two_e4m3_terms_hold_scaled_bfloat16_queries():
    """The decode's fp4 x fp8 score product takes a bfloat16 query, scaled so its largest
    magnitude lies in [2^6, 2^7), as t1 + t2 / 16 with t1 = e4m3(x) and t2 = e4m3(16 (x - t1))
    (round to nearest even).  Every bfloat16 value of magnitude 2^-6 .. 2^7 is then held exactly
    (so every element within 2^-12 of the largest), and smaller ones to within 2^-14."""
    from oracle.fp8 import e4m3fn_decode, e4m3fn_encode
    bits = np.arange(0x10000, dtype=np.uint32)
    x32 = (bits << 16).view(np.float32)
    x32 = x32[np.isfinite(x32)]
    x = x32.astype(np.float64)
    x = x[np.abs(x) < 2.0 ** 7]
    t1 = e4m3fn_decode(e4m3fn_encode(x))
    t2 = e4m3fn_decode(e4m3fn_encode(16.0 * (x - t1))) / 16.0
    err = np.abs(x - t1 - t2)
    big = np.abs(x) >= 2.0 ** -6
    assert big.sum() > 3000
    assert np.all(err[big] == 0.0)
    assert np.all(err[~big] <= 2.0 ** -14)


def _order(hs, units, mix_w, n_splits, ups, n_mix, max_entries=768):
    n = len(units)
    out = (ctypes.c_ushort * max(1, n * (n_splits + n_mix)))()
    k = hs.hs_plan_decode_order((ctypes.c_int * n)(*units), (ctypes.c_longlong * n)(*mix_w), n, n_splits, ups,
                                n_mix, max_entries, out)
    return [(out[j] >> 8, out[j] & 0xFF) for j in range(k)]


def test_decode_dispatch_order(hs):
    # equal lengths, no fp8 / fp16 parts: the plain grid order already is heaviest first
    assert _order(hs, [512] * 4, [0] * 4, 2, 256, 0) == []
    # brute force over small launches: every (part, sequence) once, weights never increase along
    # the order, equal weights in the plain order (part-major, then sequence)
    rng = __import__("random").Random(5)
    for _ in range(300):
        n = rng.randint(1, 9)
        ups = rng.choice([16, 32, 48])
        units = sorted((rng.randint(0, 200) for _ in range(n)), reverse=True)
        n_splits = max(1, -(-max(units) // ups))
        n_mix = rng.choice([0, 1, 2])
        mix_w = [rng.choice([0, 5, 40, 300]) for _ in range(n)]
        got = _order(hs, units, mix_w, n_splits, ups, n_mix)
        plain = [(z, i) for z in range(n_splits + n_mix) for i in range(n)]
        w = {(z, i): (min(max(units[i] - z * ups, 0), ups) if z < n_splits else mix_w[i]) for z, i in plain}
        want = sorted(plain, key=lambda zi: -w[zi])  # (sorted is stable)
        assert got == ([] if want == plain else want)
        if got:
            assert sorted(got) == plain
    # a hand-worked launch: lengths 100 and 30 units in 64-unit splits, one fp8 part of weight 50
    # on the second sequence: (0,0)=64, (0,1)=30, (1,0)=36, (1,1)=0, mix (2,0)=0, (2,1)=50
    assert _order(hs, [100, 30], [0, 50], 2, 64, 1) == [(0, 0), (2, 1), (1, 0), (0, 1), (1, 1), (2, 0)]
    # too many entries for the kernel-argument table: the plain grid
    assert _order(hs, [100, 30], [0, 50], 2, 64, 1, max_entries=5) == []
