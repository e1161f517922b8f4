"""GPU edge cases, exhaustive encoding sweeps and properties, against the oracle.

* every finite 16-bit input through the flat ternary pack (forced gamma, with
  exact ties), the fp8 page route and the fp16 page route, bit-exact;
* ragged appends, partial pages, window/sink corner cases, GQA 1..8,
  head_dim 64/128, block sizes 16..64, both input dtypes;
* bit-identical outputs under a different page placement and on repeats;
* error paths leave the cache usable and unchanged.
"""
import numpy as np
import pytest
import torch

from bit_ternary_attention_amd import vk
from bit_ternary_attention_amd import workloads as wl
from oracle import cache as oc
from oracle import fp8 as of
from oracle import ternary as ot

from gpu_harness import (ATTN_ATOL, GAMMA_RTOL, check_decode, check_pages, fill, host_kv, make_cache,
                         say, seq_calls, spec_of)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def all_finite_patterns(dtype):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = ot.values16(bits, dtype)
    bits = bits.copy()
    bits[~np.isfinite(vals)] = 0
    return bits


def to_dev(bits, dtype):
    t = torch.from_numpy(bits.view(np.int16).copy()).cuda()
    return t.view(torch.float16 if dtype == 0 else torch.bfloat16)


# ------------------------------------------------------------- sweeps ---

@pytest.mark.parametrize("dtype", [0, 1])
def test_flat_pack_exhaustive_forced_gamma(dtype):
    bits = all_finite_patterns(dtype)
    x = to_dev(bits, dtype)
    vals = ot.values16(bits, dtype)
    gammas = [1.0, 0.828125, 2.0 ** -20, 0.7978846, 3.0, 0.5, 1.0 / 3.0, 1e-3]
    if dtype == 1:
        # 1e38 and 3e38 put the bf16 threshold above pattern 32256, the last step of the
        # first search round
        gammas += [1e30, 7.5e-30, 1e38, 3e38]
    for g in gammas:
        for eps in (0.0, 1e-5):
            gt = torch.tensor([g], dtype=torch.float32, device="cuda")
            packed, gout = vk.quantize_pack(x, eps=eps, gamma=gt)
            torch.cuda.synchronize()
            want = ot.pack_flat(ot.ternary_codes(vals, np.float32(g), eps))
            got = packed.cpu().numpy()
            assert float(gout.item()) == float(np.float32(g))
            if not np.array_equal(got, want):
                bad = np.nonzero(got != want)[0]
                raise AssertionError(f"dtype {dtype} gamma {g} eps {eps}: {bad.size} bytes differ, first {bad[0]}")


@pytest.mark.parametrize("n,dtype", [(8, 0), (24, 1), (16384 + 8, 1), (3 * 1024 * 1024 + 40, 1), (1 << 20, 0)])
def test_flat_pack_gamma_and_codes(n, dtype):
    g = torch.Generator(device="cuda")
    g.manual_seed(n)
    x = (torch.randn(n, generator=g, device="cuda") * 1.7).to(torch.float16 if dtype == 0 else torch.bfloat16)
    packed, gout = vk.quantize_pack(x)
    torch.cuda.synchronize()
    bits = wl.to_bits(x)
    vals = ot.values16(bits, dtype)
    want_g = ot.absmean_gamma(vals)
    got_g = np.float32(gout.item())
    assert abs(float(got_g) - float(want_g)) <= GAMMA_RTOL * float(want_g)
    want = ot.pack_flat(ot.ternary_codes(vals, got_g, 1e-5))
    assert np.array_equal(packed.cpu().numpy(), want)


def _route_workload(fmt, dtype, scale=1.0):
    # 512 tokens x 1 head x 128 dims = every 16-bit pattern once
    if fmt == oc.FP8E4M3:
        return wl.small_workload(n_kv_heads=1, n_q_heads=1, head_dim=128, dtype=dtype, block_size=16,
                                 sink_tokens=0, recent_tokens=1 << 20, recent_format=oc.FP8E4M3, lengths=(512,))
    return wl.small_workload(n_kv_heads=1, n_q_heads=1, head_dim=128, dtype=dtype, block_size=16,
                             sink_tokens=512, sink_format=oc.F16, lengths=(512,))


@pytest.mark.parametrize("fmt,dtype,scale,dyn", [(oc.FP8E4M3, 1, 1.0, 0), (oc.FP8E4M3, 0, 1.0, 0),
                                                 (oc.FP8E4M3, 1, 3.0, 0), (oc.FP8E4M3, 1, 0.0078125, 0),
                                                 (oc.FP8E4M3, 1, 1.0, 1), (oc.FP8E4M3, 0, 1.0, 1),
                                                 (oc.F16, 1, 1.0, 0), (oc.F16, 0, 1.0, 0)])
def test_page_routes_exhaustive(fmt, dtype, scale, dyn):
    w = _route_workload(fmt, dtype)
    bits = all_finite_patterns(dtype)
    kb = bits.reshape(512, 1, 128)
    vb = np.ascontiguousarray(bits[::-1]).reshape(512, 1, 128)
    if dyn:  # a zero row (scale 0) among the rows of every pattern
        kb = kb.copy()
        kb[3] = 0
    cache = make_cache(w, fp8_scale=scale, fp8_dynamic=dyn)
    k = to_dev(kb.ravel(), dtype).view(1, 1, 512, 1, 128)
    v = to_dev(vb.ravel(), dtype).view(1, 1, 512, 1, 128)
    cache.append(k, v, [0])
    enc = check_pages(cache, w, 0, 0, kb, vb, pages=list(range(32)), fp8_scale=scale, fp8_dynamic=dyn)
    assert set(enc.page_format) == {fmt}
    cache.close()


# ---------------------------------------------------- ragged and edges ---

EDGE_CASES = [
    # (name, workload kwargs, windows)
    ("single-token", dict(lengths=(1,)), [-1, 0, 5]),
    ("short-partial-unit", dict(lengths=(5,), sink_tokens=4), [-1, 1, 2]),
    ("one-unit", dict(lengths=(16,)), [-1, 3]),
    ("unit-plus-one", dict(lengths=(17,)), [-1, 1, 13]),
    ("no-sinks", dict(lengths=(300,), sink_tokens=0), [-1, 1, 17, 256]),
    ("many-sinks", dict(lengths=(300,), sink_tokens=40), [-1, 0, 7, 256]),
    ("mha-d64", dict(n_q_heads=3, n_kv_heads=3, head_dim=64, lengths=(200, 77)), [-1, 50]),
    ("gqa2-bs32", dict(n_q_heads=4, n_kv_heads=2, block_size=32, lengths=(333, 64, 1)), [-1, 100]),
    ("gqa8-d128-bf16", dict(n_q_heads=16, n_kv_heads=2, head_dim=128, dtype=1, lengths=(1000, 513)), [-1, 256]),
    # the other group sizes at both head dims, long enough for whole 4-unit steps per wave
    ("gqa8-d64", dict(n_q_heads=16, n_kv_heads=2, head_dim=64, lengths=(1100, 405)), [-1, 300]),
    ("gqa2-d128", dict(n_q_heads=4, n_kv_heads=2, head_dim=128, dtype=1, lengths=(1300, 260)), [-1, 500]),
    ("gqa1-d128", dict(n_q_heads=2, n_kv_heads=2, head_dim=128, lengths=(1030,)), [-1, 700]),
    ("bs64-chunks", dict(block_size=64, lengths=(640,), chunk_tokens=128), [-1, 200]),
    ("mixed-tiers-f16-fp8", dict(n_q_heads=8, n_kv_heads=2, head_dim=128, dtype=1, sink_format=oc.F16,
                                 recent_tokens=48, recent_format=oc.FP8E4M3, lengths=(700, 31, 250),
                                 page_shuffle_seed=99, batch_appends=False), [-1, 60, 0]),
    ("recent-ternary-sink-fp8", dict(sink_tokens=20, sink_format=oc.FP8E4M3, recent_tokens=32,
                                     recent_format=oc.F16, lengths=(400,)), [-1, 33]),
]


@pytest.mark.parametrize("kernel", [2, 1], ids=["mfma", "valu"])
@pytest.mark.parametrize("name,kw,windows", EDGE_CASES, ids=[c[0] for c in EDGE_CASES])
def test_edge_workloads(name, kw, windows, kernel):
    w = wl.small_workload(**kw)
    say(f"edge {name} kernel {kernel}: {w}")
    cache = make_cache(w, decode_kernel=kernel)
    fill(cache, w)
    encs = {}
    for s in range(w.n_seqs):
        kb, vb = host_kv(w, 0, s)
        encs[s] = check_pages(cache, w, 0, s, kb, vb, pages=list(range(-(-w.lengths[s] // w.block_size))))
    q = wl.queries(w, 0, device="cuda")
    for W in windows:
        if w.sink_tokens == 0 and W == 0:
            continue
        out = cache.decode(q, list(range(w.n_seqs)), 0, window=W)
        torch.cuda.synchronize()
        err = check_decode(out, q, w, encs, W)
        say(f"edge {name} window {W}: max err {err:.2e}")
    cache.close()


UPI4_CASES = ["unit-plus-one", "many-sinks", "gqa8-d128-bf16", "gqa8-d64", "gqa1-d128", "mixed-tiers-f16-fp8"]


@pytest.mark.parametrize("name", UPI4_CASES)
def test_edge_workloads_ring_depth_4(name, monkeypatch):
    """The matrix-core kernel with a 4-slot ring (VK_DECODE_UPI=4): waves with at most four
    units take the short-range path at that depth, longer ones the ring."""
    monkeypatch.setenv("VK_DECODE_UPI", "4")
    _, kw, windows = next(c for c in EDGE_CASES if c[0] == name)
    w = wl.small_workload(**kw)
    say(f"edge {name} ring depth 4: {w}")
    cache = make_cache(w, decode_kernel=2)
    fill(cache, w)
    encs = {}
    for s in range(w.n_seqs):
        kb, vb = host_kv(w, 0, s)
        encs[s] = oc.encode_sequence(spec_of(w), kb, vb, w.dtype, seq_calls(w, s))
    q = wl.queries(w, 0, device="cuda")
    for W in windows:
        if w.sink_tokens == 0 and W == 0:
            continue
        out = cache.decode(q, list(range(w.n_seqs)), 0, window=W)
        torch.cuda.synchronize()
        err = check_decode(out, q, w, encs, W)
        say(f"edge {name} ring depth 4 window {W}: max err {err:.2e}")
    cache.close()


STEAL_CASES = [
    # (name, workload kwargs, windows, sequences checked against the oracle (None: all))
    # 128 (sequence, KV head) pairs: two splits of 16 pieces per pair, 12 waves sharing them
    ("gqa4-d128-bf16-many-pieces", dict(n_q_heads=32, n_kv_heads=8, head_dim=128, dtype=1, n_seqs=16,
                                        lengths=tuple(8192 - 509 * i for i in range(16))), [-1, 3001], [0, 5, 15]),
    ("gqa8-d128-bf16", dict(n_q_heads=16, n_kv_heads=2, head_dim=128, dtype=1, lengths=(5000, 1300, 17)),
     [-1, 700], None),
    ("gqa2-d128-f16", dict(n_q_heads=4, n_kv_heads=2, head_dim=128, lengths=(4100, 260)), [-1, 500], None),
    ("gqa4-d128-f16", dict(n_q_heads=8, n_kv_heads=2, head_dim=128, lengths=(3333,)), [-1, 100], None),
    ("gqa1-d64", dict(n_q_heads=2, n_kv_heads=2, head_dim=64, lengths=(2600, 999)), [-1, 40], None),
    ("gqa8-d64-bf16", dict(n_q_heads=16, n_kv_heads=2, head_dim=64, dtype=1, lengths=(3000,)), [-1, 0], None),
]


@pytest.mark.parametrize("name,kw,windows,sample", STEAL_CASES, ids=[c[0] for c in STEAL_CASES])
def test_stealing_blocks(name, kw, windows, sample, monkeypatch):
    """All-ternary decodes through the 12-wave stealing blocks (forced on at these sizes): against
    the oracle, and close to the 4-wave blocks' outputs (the default) on the same cache."""
    w = wl.small_workload(**kw)
    say(f"steal {name}: {w}")
    cache = make_cache(w, decode_kernel=2)
    fill(cache, w)
    ids = list(range(w.n_seqs)) if sample is None else sample
    encs = {}
    for s in ids:
        kb, vb = host_kv(w, 0, s)
        encs[s] = oc.encode_sequence(spec_of(w), kb, vb, w.dtype, seq_calls(w, s))
    q = wl.queries(w, 0, device="cuda")
    for W in windows:
        monkeypatch.setenv("VK_DECODE_STEAL", "2")
        out = cache.decode(q, list(range(w.n_seqs)), 0, window=W)
        torch.cuda.synchronize()
        assert cache.stats()["last_decode_steal"] == 1
        err = check_decode(out, q, w, encs, W)
        monkeypatch.setenv("VK_DECODE_STEAL", "0")
        plain = cache.decode(q, list(range(w.n_seqs)), 0, window=W)
        torch.cuda.synchronize()
        assert cache.stats()["last_decode_steal"] == 0
        diff = float((out - plain).abs().max())
        assert diff <= 2 * ATTN_ATOL
        say(f"steal {name} window {W}: max err {err:.2e}, vs 4-wave blocks {diff:.2e}")
    cache.close()


@pytest.mark.parametrize("dyn", [0, 1], ids=["static-fp8", "dynamic-fp8"])
@pytest.mark.parametrize("kernel", [2, 1], ids=["mfma", "valu"])
def test_incremental_decode_appends_into_recent_tier(kernel, dyn):
    """Prefill, then one-token appends (the recent fp8 tier grows page by page), decoding each step."""
    w = wl.small_workload(n_q_heads=8, n_kv_heads=2, head_dim=128, dtype=1, sink_format=oc.F16,
                          recent_tokens=64, recent_format=oc.FP8E4M3, lengths=(300,))
    steps = [(0, 250)] + [(250 + i, 1) for i in range(50)]
    cache = make_cache(w, slack_pages=(0, 8, 0), decode_kernel=kernel, fp8_dynamic=dyn)
    spec = spec_of(w, fp8_dynamic=dyn)
    kall = wl.kv_block(w, "k", 0, 0, 0, 300, device="cuda")
    vall = wl.kv_block(w, "v", 0, 0, 0, 300, device="cuda")
    kb, vb = wl.to_bits(kall), wl.to_bits(vall)
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    for i, (t0, n) in enumerate(steps):
        cache.append(kall[t0:t0 + n][None, None].contiguous(), vall[t0:t0 + n][None, None].contiguous(), [0])
        if i % 7 == 0 or i == len(steps) - 1:
            L = t0 + n
            enc = oc.encode_sequence(spec, kb[:L], vb[:L], 1, steps[:i + 1])
            q = torch.randn((1, 8, 128), generator=g, device="cuda").to(torch.bfloat16)
            out = cache.decode(q, [0], 0, window=-1)
            torch.cuda.synchronize()
            check_decode(out, q, w, {0: enc}, -1)
    assert cache.seq_length(0) == 300
    cache.close()


RAGGED_CASES = [
    ("mixed-tiers", dict(n_q_heads=8, n_kv_heads=2, head_dim=128, dtype=1, sink_format=oc.F16, recent_tokens=48,
                         recent_format=oc.FP8E4M3, lengths=(700, 31, 250, 1, 64, 17))),
    ("chunked-d64", dict(n_q_heads=4, n_kv_heads=2, head_dim=64, lengths=(200, 64, 130, 5), chunk_tokens=64)),
    ("chunked-dynamic-fp8", dict(n_q_heads=16, n_kv_heads=2, head_dim=128, dtype=1, recent_tokens=40,
                                 recent_format=oc.FP8E4M3, lengths=(333, 100, 48), chunk_tokens=48)),
]


@pytest.mark.parametrize("name,kw", RAGGED_CASES, ids=[c[0] for c in RAGGED_CASES])
def test_ragged_append_matches_per_sequence_appends(name, kw):
    """One vk_append_ragged call per round of chunks writes the same pages (bytes, formats,
    gammas) and gives the same decode outputs, bit for bit, as one vk_append per sequence and
    chunk; and its pages match the oracle."""
    dyn = int("dynamic" in name)
    w_r = wl.small_workload(**kw, batch_appends=False, ragged_appends=True)
    w_s = wl.small_workload(**kw, batch_appends=False)
    assert any(len(set(ns)) > 1 for _, _, ns in w_r.append_batches())
    caches = []
    for w in (w_r, w_s):
        cache = make_cache(w, fp8_dynamic=dyn)
        fill(cache, w)
        caches.append(cache)
    assert caches[0].stats()["append_calls"] == len(w_r.append_batches()) < caches[1].stats()["append_calls"]
    q = wl.queries(w_r, 0, device="cuda")
    for s in range(w_r.n_seqs):
        n = -(-w_r.lengths[s] // w_r.block_size)
        a, b = caches[0].read_pages(0, s, 0, n), caches[1].read_pages(0, s, 0, n)
        for x, y in zip(a, b):
            assert np.array_equal(x, y, equal_nan=True), (name, s)
        kb, vb = host_kv(w_r, 0, s)
        check_pages(caches[0], w_r, 0, s, kb, vb, pages=list(range(n)), fp8_dynamic=dyn)
    for W in (-1, 40):
        o = [c.decode(q, list(range(w_r.n_seqs)), 0, window=W) for c in caches]
        torch.cuda.synchronize()
        assert torch.equal(o[0], o[1]), (name, W)
    for c in caches:
        c.close()


def test_ragged_append_arguments():
    w = wl.small_workload(n_q_heads=4, n_kv_heads=2, head_dim=64, lengths=(32, 16))
    cache = make_cache(w)
    k = torch.zeros((1, 48, 2, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        cache.append_ragged(k, k, [0, 1], [32, 15])          # counts do not add up to the rows
    with pytest.raises(vk.VkError) as e:
        cache.append_ragged(k, k, [0, 1], [48, 0])           # a zero count
    assert e.value.status == vk.ERR_ARG
    with pytest.raises(vk.VkError) as e:
        cache.append_ragged(k, k, [0, 0], [32, 16])          # a repeated id
    assert e.value.status == vk.ERR_ARG
    assert cache.seq_length(0) == 0 and cache.seq_length(1) == 0   # nothing changed
    cache.append_ragged(k, k, [1, 0], [16, 32])
    assert cache.seq_length(0) == 32 and cache.seq_length(1) == 16
    cache.close()


QUERY_RANGES = [
    # (query factor, softmax scale factor): bf16 queries far outside the f16 range, with a
    # softmax scale that brings the scores back to order 1 (so every score matters)
    (1e5, 1e-5), (3e37, 1e-37), (1e-30, 1e30), (1e-36, 1e36), (7.0, 1.0 / 7.0),
]


@pytest.mark.parametrize("kernel", [2, 1], ids=["mfma", "valu"])
@pytest.mark.parametrize("qf,sf", QUERY_RANGES, ids=[f"q{c[0]:g}" for c in QUERY_RANGES])
def test_query_outside_f16_range(kernel, qf, sf):
    """bf16 queries of any magnitude: the decode scales them by a power of two before the f16
    products and takes the scale back out of the scores."""
    w = wl.small_workload(n_q_heads=8, n_kv_heads=2, head_dim=128, dtype=1, sink_format=oc.F16,
                          recent_tokens=48, recent_format=oc.FP8E4M3, lengths=(700, 31, 250),
                          batch_appends=False)
    cache = make_cache(w, decode_kernel=kernel)
    fill(cache, w)
    encs = {}
    for s in range(w.n_seqs):
        kb, vb = host_kv(w, 0, s)
        encs[s] = oc.encode_sequence(spec_of(w), kb, vb, w.dtype, seq_calls(w, s))
    q = (wl.queries(w, 0, device="cuda").float() * qf).to(torch.bfloat16)
    assert torch.isfinite(q.float()).all() and float(q.float().abs().max()) > 0
    scale = sf / np.sqrt(w.head_dim)
    for W in (-1, 60):
        out = cache.decode(q, list(range(w.n_seqs)), 0, window=W, softmax_scale=scale)
        torch.cuda.synchronize()
        err = check_decode(out, q, w, encs, W, scale=scale)
        say(f"query x {qf:g}, scale x {sf:g}, window {W}: max err {err:.2e}")
    cache.close()


@pytest.mark.parametrize("kernel", [2, 1], ids=["mfma", "valu"])
def test_page_placement_and_repeats_are_bit_identical(kernel):
    w = wl.small_workload(n_q_heads=8, n_kv_heads=2, head_dim=128, dtype=1, sink_format=oc.F16,
                          recent_tokens=100, lengths=(900, 455, 1200), batch_appends=False)
    outs = []
    for shuffle in (0, 1004, 77):
        cache = make_cache(w, shuffle=shuffle, slack_pages=(50, 50, 50), decode_kernel=kernel)
        fill(cache, w)
        q = wl.queries(w, 0, device="cuda")
        for W in (-1, 300):
            outs.append((shuffle, W, cache.decode(q, [0, 1, 2], 0, window=W).cpu()))
            again = cache.decode(q, [0, 1, 2], 0, window=W).cpu()
            assert torch.equal(outs[-1][2], again)
        cache.close()
    for W in (-1, 300):
        ref = [o for s, ww, o in outs if ww == W]
        assert all(torch.equal(ref[0], r) for r in ref[1:])


@pytest.mark.parametrize("kernel", [2, 1], ids=["mfma", "valu"])
def test_many_sequences_subset_and_order(kernel):
    """More sequences than one launch holds; decode a reordered subset."""
    w = wl.small_workload(n_q_heads=4, n_kv_heads=2, head_dim=64, n_seqs=70, lengths=tuple(range(20, 90)),
                          batch_appends=False)
    cache = make_cache(w, decode_kernel=kernel)
    fill(cache, w)
    q = wl.queries(w, 0, device="cuda")
    encs = {}
    for s in (0, 33, 64, 69):
        kb, vb = host_kv(w, 0, s)
        encs[s] = oc.encode_sequence(spec_of(w), kb, vb, 0, seq_calls(w, s))
    out = cache.decode(q, list(range(70)), 0, window=-1)
    torch.cuda.synchronize()
    check_decode(out, q, w, encs, -1)
    ids = [69, 0, 33, 64]
    sub = cache.decode(q[ids].contiguous(), ids, 0, window=-1)
    torch.cuda.synchronize()
    assert float((sub - out[ids]).abs().max()) <= 1e-5
    cache.close()


def test_empty_and_zero_length_calls():
    """A decode of no sequences is a no-op; appends of no tokens and empty tensors are refused;
    the cache is unchanged and still decodes."""
    w = wl.small_workload(n_q_heads=4, n_kv_heads=2, head_dim=64, lengths=(40,))
    cache = make_cache(w, decode_kernel=2)
    fill(cache, w)
    q = wl.queries(w, 0, device="cuda")
    before = cache.decode(q, [0], 0).cpu()
    out = cache.decode(torch.empty((0, 4, 64), dtype=torch.float16, device="cuda"), [], 0)
    assert out.shape == (0, 4, 64)
    k0 = torch.zeros((1, 1, 0, 2, 64), dtype=torch.float16, device="cuda")
    with pytest.raises((vk.VkError, ValueError)):
        cache.append(k0, k0, [0])
    with pytest.raises((vk.VkError, ValueError)):
        vk.quantize_pack(torch.empty(0, dtype=torch.float16, device="cuda"))
    assert cache.seq_length(0) == 40
    assert torch.equal(cache.decode(q, [0], 0).cpu(), before)
    cache.close()


def test_errors_leave_cache_unchanged_and_usable():
    w = wl.small_workload(n_q_heads=4, n_kv_heads=2, head_dim=64, lengths=(64, 64), n_seqs=2)
    cache = make_cache(w, max_tokens=256)  # exactly the pages two 64-token sequences need (+2 slack)
    fill(cache, w)
    before = cache.stats()
    k = torch.zeros((1, 1, 64, 2, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(vk.VkError) as e:
        cache.append(k, k, [0])                 # pool exhausted
    assert e.value.status == vk.ERR_CAPACITY
    with pytest.raises(vk.VkError) as e:
        cache.append(k, k, [5])                 # id out of range
    assert e.value.status == vk.ERR_ARG
    with pytest.raises(vk.VkError) as e:
        cache.append(k[:, :, :3].contiguous(), k[:, :, :3].contiguous(), [0], layer_begin=1)
    assert e.value.status == vk.ERR_ARG
    after = cache.stats()
    assert after["pages_used"] == before["pages_used"] and cache.seq_length(0) == 64
    q = wl.queries(w, 0, device="cuda")
    ok = cache.decode(q, [0, 1], 0).cpu()
    cache.reset([1])
    assert cache.seq_length(1) == 0
    with pytest.raises(vk.VkError) as e:
        cache.decode(q, [0, 1], 0)              # seq 1 is empty now
    assert e.value.status == vk.ERR_ARG
    fill_one = wl.append_inputs(w, [1], 0, 64, device="cuda")
    cache.append(fill_one[0], fill_one[1], [1])  # freed pages are reused
    again = cache.decode(q, [0, 1], 0).cpu()
    assert torch.equal(ok, again)
    small = wl.small_workload(n_q_heads=4, n_kv_heads=2, head_dim=64, lengths=(20,))
    c2 = make_cache(small, slack_pages=(4, 0, 0), max_tokens=64)
    fill(c2, small)                              # page 1 ternary, partly filled
    kk = torch.zeros((1, 1, 4, 2, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(vk.VkError) as e:
        c2.append(kk, kk, [0])
    assert e.value.status == vk.ERR_ALIGN
    c2.close()
    cache.close()


@pytest.mark.parametrize("kernel", [2, 1], ids=["mfma", "valu"])
def test_dynamic_fp8_mixed_tiers_with_extreme_rows(kernel):
    """Dynamic FP8 recent pages holding zero rows, tiny rows and rows near the bfloat16 range
    next to ordinary ones; pages (codes and scales) exact, decode within tolerance."""
    w = wl.small_workload(n_q_heads=8, n_kv_heads=2, head_dim=128, dtype=1, sink_format=oc.F16,
                          recent_tokens=80, recent_format=oc.FP8E4M3, lengths=(211, 37, 160),
                          page_shuffle_seed=5, batch_appends=False)
    cache = make_cache(w, decode_kernel=kernel, fp8_dynamic=1)
    encs = {}
    for ids, t0, n in w.appends():
        k, v = wl.append_inputs(w, ids, t0, n, device="cuda")
        k[0, 0, -3] = 0.0                         # a zero key row for both heads (scale 0)
        v[0, 0, -5, 1] = 1e-30                    # a tiny value row
        k[0, 0, -7, 0] *= 1e4                     # a large key row
        cache.append(k.contiguous(), v.contiguous(), ids)
        kb, vb = wl.to_bits(k[0, 0]), wl.to_bits(v[0, 0])
        encs[ids[0]] = check_pages(cache, w, 0, ids[0], kb, vb, fp8_dynamic=1,
                                   pages=list(range(-(-n // w.block_size))))
    q = wl.queries(w, 0, device="cuda")
    for W in (-1, 70, 0):
        out = cache.decode(q, [0, 1, 2], 0, window=W)
        torch.cuda.synchronize()
        err = check_decode(out, q, w, encs, W)
        say(f"dynamic fp8 window {W}: max err {err:.2e}")
    cache.close()


# ------------------------------------------------------ lossless tier ---

@pytest.mark.parametrize("dim", [128, 64])
@pytest.mark.parametrize("arrangement", ["sorted", "strided", "shuffled"])
def test_lossless_route_every_bf16_pattern(dim, arrangement):
    """Every bfloat16 pattern (infinities and NaNs included) through the lossless page route, keys and
    values: page bytes equal the oracle's (centre, codes, exception order; coded and raw groups)
    and read back to the input bits."""
    n_tok = 65536 // dim
    w = wl.small_workload(n_kv_heads=1, n_q_heads=1, head_dim=dim, dtype=1, block_size=16, sink_tokens=n_tok,
                          sink_format=oc.LOSSLESS, lengths=(n_tok,))
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    if arrangement == "strided":
        bits = bits.reshape(16 * dim, -1).T.ravel().copy()
    elif arrangement == "shuffled":
        bits = np.random.default_rng(9).permutation(bits)
    kb = bits.reshape(n_tok, 1, dim)
    vb = np.ascontiguousarray(bits[::-1]).reshape(n_tok, 1, dim)
    cache = make_cache(w)
    k = to_dev(kb.ravel(), 1).view(1, 1, n_tok, 1, dim)
    v = to_dev(vb.ravel(), 1).view(1, 1, n_tok, 1, dim)
    cache.append(k, v, [0])
    enc = check_pages(cache, w, 0, 0, kb, vb, pages=list(range(n_tok // 16)))
    assert set(enc.page_format) == {oc.LOSSLESS}
    buf, fmt, _ = cache.read_pages(0, 0, 0, n_tok // 16)
    modes = {int(buf[p, 1]) for p in range(n_tok // 16)}
    assert modes == ({0} if arrangement == "sorted" else ({1} if arrangement == "strided" else modes))
    cache.close()


LOSSLESS_CASES = [
    ("anchor-d128-g4", dict(n_q_heads=8, n_kv_heads=2, head_dim=128, dtype=1, sink_format=oc.LOSSLESS,
                            lengths=(700, 31, 250, 1), batch_appends=False), [-1, 60, 0]),
    ("anchor-recent-d64-g8", dict(n_q_heads=16, n_kv_heads=2, head_dim=64, dtype=1, sink_tokens=40,
                                  sink_format=oc.LOSSLESS, recent_tokens=48, recent_format=oc.LOSSLESS,
                                  block_size=32, lengths=(400, 90), batch_appends=False), [-1, 100]),
    ("anchor-lossless-recent-fp8-g2", dict(n_q_heads=4, n_kv_heads=2, head_dim=128, dtype=1, sink_format=oc.LOSSLESS,
                                           recent_tokens=64, recent_format=oc.FP8E4M3, lengths=(1000, 300),
                                           batch_appends=False), [-1, 200]),
    ("outliers-and-zeros", dict(n_q_heads=8, n_kv_heads=2, head_dim=128, dtype=1, sink_tokens=64,
                                sink_format=oc.LOSSLESS, lengths=(500,), outlier_frac=0.2), [-1, 30]),
]


@pytest.mark.parametrize("dyn", [0, 1], ids=["static-fp8", "dynamic-fp8"])
@pytest.mark.parametrize("name,kw,windows", LOSSLESS_CASES, ids=[c[0] for c in LOSSLESS_CASES])
def test_lossless_tier_pages_and_decode(name, kw, windows, dyn):
    """Lossless anchor (and recent) pages beside ternary and fp8 pages: every page against the
    oracle, decode against the oracle's float64 attention over the exact bfloat16 values."""
    w = wl.small_workload(**kw)
    cache = make_cache(w, fp8_dynamic=dyn)
    fill(cache, w)
    encs = {}
    for s in range(w.n_seqs):
        kb, vb = host_kv(w, 0, s)
        encs[s] = check_pages(cache, w, 0, s, kb, vb, pages=list(range(-(-w.lengths[s] // w.block_size))),
                              fp8_dynamic=dyn)
    assert cache.stats()["pages_used"][oc.LOSSLESS] > 0
    q = wl.queries(w, 0, device="cuda")
    for W in windows:
        out = cache.decode(q, list(range(w.n_seqs)), 0, window=W)
        torch.cuda.synchronize()
        err = check_decode(out, q, w, encs, W)
        assert cache.stats()["last_decode_units"][oc.LOSSLESS] > 0
        say(f"lossless {name} window {W}: max err {err:.2e}")
    cache.close()


def test_lossless_tier_errors():
    """float16 input into lossless pages, the vector-ALU kernel with lossless pages and an append
    into a partly filled lossless page are refused; the cache stays usable."""
    w = wl.small_workload(n_q_heads=4, n_kv_heads=2, head_dim=64, dtype=1, block_size=32, sink_tokens=32,
                          sink_format=oc.LOSSLESS, lengths=(64,))
    with pytest.raises(vk.VkError) as e:
        make_cache(w, decode_kernel=1)
    assert e.value.status == vk.ERR_ARG
    cache = make_cache(w)
    k16 = torch.zeros((1, 1, 20, 2, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(vk.VkError) as e:
        cache.append(k16, k16, [0])
    assert e.value.status == vk.ERR_ARG and cache.seq_length(0) == 0
    kb = torch.randn((1, 1, 20, 2, 64), device="cuda").to(torch.bfloat16)
    cache.append(kb, kb, [0])
    with pytest.raises(vk.VkError) as e:
        cache.append(kb, kb, [0])
    assert e.value.status == vk.ERR_ALIGN and cache.seq_length(0) == 20
    cache.close()
