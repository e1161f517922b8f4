"""GPU parity of retiering (FP8 recent pages that left the window -> ternary pages).

Every page of the sampled (layer, sequence) pairs is compared with the oracle
after retiering: formats and block-table flips, the per-page gamma (2^-22
relative), the packed bytes (bit-exact, re-encoded with the device's gamma);
decode over the retiered cache against the oracle's attention (max-abs 2e-3),
with the matrix-core and vector-ALU kernels.
"""
import numpy as np
import pytest
import torch

from bit_ternary_attention_amd import vk
from bit_ternary_attention_amd import workloads as wl
from oracle import attention as oa
from oracle import cache as oc
from oracle import ternary as ot

from gpu_harness import ATTN_ATOL, GAMMA_RTOL, check_partial_page, read_page, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


class Stream:
    """Seeded K/V/q for a hand-driven append schedule, kept as host bits for the oracle."""

    def __init__(self, n_layers, n_seqs, hkv, hq, dim, dtype, seed):
        self.n_layers, self.n_seqs, self.hkv, self.hq, self.dim = n_layers, n_seqs, hkv, hq, dim
        self.dtype = dtype
        self.tdtype = torch.float16 if dtype == wl.DTYPE_F16 else torch.bfloat16
        self.gen = torch.Generator(device="cuda")
        self.gen.manual_seed(seed)
        self.k = [[[] for _ in range(n_seqs)] for _ in range(n_layers)]
        self.v = [[[] for _ in range(n_seqs)] for _ in range(n_layers)]
        self.calls = [[] for _ in range(n_seqs)]
        self.length = [0] * n_seqs

    def draw(self, ids, n, scale=1.0):
        shape = (self.n_layers, len(ids), n, self.hkv, self.dim)
        k = (torch.randn(shape, generator=self.gen, device="cuda") * scale).to(self.tdtype).contiguous()
        v = (torch.randn(shape, generator=self.gen, device="cuda") * scale).to(self.tdtype).contiguous()
        kb, vb = wl.to_bits(k), wl.to_bits(v)
        for j, s in enumerate(ids):
            for layer in range(self.n_layers):
                self.k[layer][s].append(kb[layer, j])
                self.v[layer][s].append(vb[layer, j])
            self.calls[s].append((self.length[s], n))
            self.length[s] += n
        return k, v

    def bits(self, layer, s):
        return np.concatenate(self.k[layer][s]), np.concatenate(self.v[layer][s])

    def query(self):
        return torch.randn((self.n_seqs, self.hq, self.dim), generator=self.gen, device="cuda").to(self.tdtype)


def make(stream, bs, S, sinkf, R, cap, fp8_scale=1.0, decode_kernel=0, max_tokens=4096, fp8_dynamic=0):
    cfg = vk.make_config(n_layers=stream.n_layers, n_kv_heads=stream.hkv, n_q_heads=stream.hq,
                         head_dim=stream.dim, block_size=bs, max_seqs=stream.n_seqs, max_tokens_per_seq=max_tokens,
                         sink_tokens=S, sink_format=sinkf, recent_tokens=R, recent_format=vk.FMT_FP8E4M3,
                         pages_ternary=cap[0], pages_fp8=cap[1], pages_f16=cap[2], fp8_scale=fp8_scale,
                         page_shuffle_seed=77, decode_kernel=decode_kernel, fp8_dynamic=fp8_dynamic)
    return vk.Cache(cfg)


def spec_for(stream, bs, S, sinkf, R, fp8_scale=1.0, fp8_dynamic=0):
    return oc.CacheSpec(n_kv_heads=stream.hkv, head_dim=stream.dim, block_size=bs, sink_tokens=S,
                        sink_format=sinkf, recent_tokens=R, recent_format=oc.FP8E4M3, fp8_scale=fp8_scale,
                        fp8_dynamic=bool(fp8_dynamic))


def check_retiered(cache, stream, spec, layer, s):
    """Every page of (layer, s) against the oracle retiered at the current length; returns the encoding."""
    kb, vb = stream.bits(layer, s)
    calls = stream.calls[s]
    bs = spec.block_size
    enc = oc.encode_sequence(spec, kb, vb, stream.dtype, calls)
    ref = oc.retier(spec, enc)
    n_pages = len(enc.page_format)
    # device gamma: per append call (pages written ternary) and per retiered page
    call_g = [(np.nan, np.nan)] * len(calls)
    for ci in range(len(calls)):
        toks = np.nonzero((enc.token_call == ci) & (enc.token_format == oc.TERNARY2))[0]
        if toks.size:
            _, fmt, gam = read_page(cache, layer, s, int(toks[0]) // bs)
            assert fmt == oc.TERNARY2
            call_g[ci] = (float(gam[0]), float(gam[1]))
            for j in range(2):
                want = float(enc.gamma[ci][j])
                assert abs(call_g[ci][j] - want) <= GAMMA_RTOL * want
    page_g = {}
    for p, (gk, gv) in ref.page_gamma.items():
        _, fmt, gam = read_page(cache, layer, s, p)
        assert fmt == oc.TERNARY2, (layer, s, p, fmt)
        for got, want in ((gam[0], gk), (gam[1], gv)):
            assert abs(float(got) - float(want)) <= GAMMA_RTOL * float(want), (layer, s, p, got, want)
        page_g[p] = (float(gam[0]), float(gam[1]))
    dev = oc.retier(spec, oc.encode_sequence(spec, kb, vb, stream.dtype, calls, gamma_override=call_g),
                    gamma_override=page_g)
    assert dev.page_format == ref.page_format
    for p in range(n_pages):
        buf, fmt, _ = read_page(cache, layer, s, p)
        assert fmt == ref.page_format[p], (layer, s, p, fmt, ref.page_format[p])
        nb = oc.page_bytes(spec, fmt)
        lo, hi = p * bs, min((p + 1) * bs, enc.length)
        if hi - lo == bs:
            want = oc.page_tiles(spec, dev, p)
            if not np.array_equal(buf[:nb], want):
                bad = np.nonzero(buf[:nb] != want)[0]
                raise AssertionError(f"layer {layer} seq {s} page {p} fmt {fmt}: {bad.size} bytes differ, "
                                     f"first {bad[0]}")
        else:
            check_partial_page(spec, dev, p, buf[:nb], fmt, hi - lo)
    return ref


def check_decode(cache, stream, encs, layer, window, S):
    q = stream.query()
    ids = list(range(stream.n_seqs))
    out = cache.decode(q, ids, layer, window=window)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    qv = ot.values16(wl.to_bits(q), stream.dtype)
    worst = 0.0
    for s in ids:
        e = encs[s]
        ref = oa.decode_attention(qv[s], e.k_hat, e.v_hat, e.length, S, window)
        err = float(np.max(np.abs(o[s] - ref)))
        assert err <= ATTN_ATOL, (layer, s, window, err)
        worst = max(worst, err)
    return worst


@pytest.mark.parametrize("dim,bs,S,sinkf,R,scale,dyn", [(128, 16, 4, wl.FMT_F16, 48, 1.0, 0),
                                                         (64, 32, 4, wl.FMT_TERNARY2, 40, 1.0, 0),
                                                         (128, 64, 0, wl.FMT_TERNARY2, 100, 0.3, 0),
                                                         (64, 16, 20, wl.FMT_FP8E4M3, 16, 0.25, 0),
                                                         (128, 16, 4, wl.FMT_F16, 48, 1.0, 1),
                                                         (64, 32, 4, wl.FMT_TERNARY2, 40, 1.0, 1),
                                                         (128, 64, 20, wl.FMT_FP8E4M3, 100, 1.0, 1),
                                                         (256, 16, 4, wl.FMT_F16, 48, 1.0, 0),
                                                         (256, 64, 4, wl.FMT_TERNARY2, 100, 0.5, 0),
                                                         (256, 32, 20, wl.FMT_FP8E4M3, 40, 1.0, 1)])
def test_retier_ragged_appends(dim, bs, S, sinkf, R, scale, dyn):
    """Ragged appends per sequence, retiering after every call; every page checked."""
    say(f"retier ragged: dim {dim} bs {bs} S {S} sink fmt {sinkf} R {R} scale {scale} dynamic {dyn}")
    st = Stream(2, 3, 2, 8, dim, wl.DTYPE_BF16, seed=dim + bs + R)
    rng = np.random.default_rng(dim * bs + R)
    cache = make(st, bs, S, sinkf, R, (600, 200, 40), fp8_scale=scale, fp8_dynamic=dyn)
    spec = spec_for(st, bs, S, sinkf, R, scale, dyn)
    done = 0
    for _ in range(14):
        s = int(rng.integers(0, 3))
        n = int(rng.integers(1, 90))
        sink_end = bs * -(-S // bs)
        if sinkf == wl.FMT_TERNARY2 and st.length[s] < sink_end:
            n = max(n, sink_end)                   # a ternary (sink) page is written by one append
        k, v = st.draw([s], n, scale=2.0)
        cache.append(k, v, [s])
        done += cache.retier([s])
    for s in range(3):
        if st.length[s] == 0:
            k, v = st.draw([s], 5 * bs)
            cache.append(k, v, [s])
    done += cache.retier([0, 1, 2])
    torch.cuda.synchronize()
    assert cache.stats()["pages_retiered"] == done > 0
    for layer in range(2):
        encs = {s: check_retiered(cache, st, spec, layer, s) for s in range(3)}
        for window in (-1, R // 2):
            err = check_decode(cache, st, encs, layer, window, S)
            say(f"  layer {layer} window {window}: max abs err {err:.3e}")


@pytest.mark.parametrize("kernel", [2, 1], ids=["mfma", "valu"])
def test_retier_decode_loop(kernel):
    """Prefill, then one token per step for every sequence with a retier after each append;
    decode over sinks (fp16) + ternary history + the FP8 recent pages at several steps."""
    S, R, bs = 4, 48, 16
    st = Stream(2, 4, 2, 16, 128, wl.DTYPE_BF16, seed=99)
    cache = make(st, bs, S, wl.FMT_F16, R, (400, 40, 8), decode_kernel=kernel)
    spec = spec_for(st, bs, S, wl.FMT_F16, R)
    ids = [0, 1, 2, 3]
    k, v = st.draw(ids, 200)
    cache.append(k, v, ids)
    converted = cache.retier(ids)
    for step in range(70):
        k, v = st.draw(ids, 1)
        cache.append(k, v, ids)
        converted += cache.retier(ids)
        if step in (13, 69):
            torch.cuda.synchronize()
            for layer in (0, 1):
                encs = {s: check_retiered(cache, st, spec, layer, s) for s in ids}
                for window in (-1, 40):
                    err = check_decode(cache, st, encs, layer, window, S)
                    say(f"  step {step} layer {layer} window {window}: max abs err {err:.3e}")
    # the prefill wrote pages 1..8 ternary and 9..12 fp8; those four leave the window by the end
    s0 = cache.stats()
    assert converted == s0["pages_retiered"] and converted >= 4 * 4
    assert s0["pages_used"][1] <= 4 * (-(-R // bs) + 1)   # the FP8 tier stays bounded


def test_retier_capacity_error_leaves_cache_unchanged():
    st = Stream(1, 1, 2, 8, 64, wl.DTYPE_F16, seed=5)
    S, R, bs = 4, 16, 16
    cache = make(st, bs, S, wl.FMT_F16, R, (2, 30, 2))
    spec = spec_for(st, bs, S, wl.FMT_F16, R)
    for _ in range(12):                          # 16 tokens per call: every page but page 0 is fp8
        k, v = st.draw([0], 16)
        cache.append(k, v, [0])
    with pytest.raises(vk.VkError) as e:
        cache.retier([0])                        # 10 pages to convert, 2 free ternary pages
    assert e.value.status == vk.ERR_CAPACITY
    kb, vb = st.bits(0, 0)
    enc = oc.encode_sequence(spec, kb, vb, st.dtype, st.calls[0])
    _, fmt, _ = cache.read_pages(0, 0, 0, 12)
    assert fmt.tolist() == enc.page_format        # nothing flipped
    err = check_decode(cache, st, {0: enc}, 0, -1, S)
    say(f"capacity error: decode still matches, max abs err {err:.3e}")


def test_retier_every_fp8_code_exact_gamma():
    """Pages holding every finite e4m3fn value (through the FP8 route, exactly) in three mixes;
    with fp8_scale 1 the page sum is exact on both sides, so gamma must match bit for bit."""
    from oracle import fp8 as of
    hkv, dim, bs = 2, 128, 16
    vals = of.E4M3_POS[:127]                                   # 0 .. 448, every magnitude
    rng = np.random.default_rng(3)
    mixes = [np.concatenate([vals, -vals]),                    # everything, both signs
             np.concatenate([vals[:40], -vals[:40]]),          # subnormals and small normals
             np.concatenate([vals[100:], -vals[100:], np.zeros(10)])]  # large values and zeros
    st = Stream(1, len(mixes), hkv, 8, dim, wl.DTYPE_BF16, seed=1)
    cache = make(st, bs, 0, wl.FMT_TERNARY2, bs, (8, 8, 2))
    spec = spec_for(st, bs, 0, wl.FMT_TERNARY2, bs)
    for s, mix in enumerate(mixes):
        k = rng.choice(mix, size=(bs, hkv, dim))
        v = rng.choice(mix, size=(bs, hkv, dim))[:, :, ::-1] * 0.5
        for part in ((k, v), (np.ones((bs, hkv, dim)), np.ones((bs, hkv, dim)))):
            kt = torch.tensor(np.ascontiguousarray(part[0]), dtype=torch.float32).to(torch.bfloat16)
            vt = torch.tensor(np.ascontiguousarray(part[1]), dtype=torch.float32).to(torch.bfloat16)
            assert np.array_equal(kt.float().numpy(), part[0]) and np.array_equal(vt.float().numpy(), part[1])
            kb, vb = wl.to_bits(kt), wl.to_bits(vt)
            for arr, store in ((kb, st.k[0][s]), (vb, st.v[0][s])):
                store.append(arr)
            st.calls[s].append((st.length[s], bs))
            st.length[s] += bs
            cache.append(kt[None, None].cuda().contiguous(), vt[None, None].cuda().contiguous(), [s])
    assert cache.retier(list(range(len(mixes)))) == len(mixes)
    torch.cuda.synchronize()
    for s in range(len(mixes)):
        kb, vb = st.bits(0, s)
        ref = oc.retier(spec, oc.encode_sequence(spec, kb, vb, st.dtype, st.calls[s]))
        buf, fmt, gam = cache.read_pages(0, s, 0, 1)
        assert int(fmt[0]) == oc.TERNARY2
        assert (float(gam[0, 0]), float(gam[0, 1])) == tuple(float(x) for x in ref.page_gamma[0]), s
        assert np.array_equal(buf[0][:oc.page_bytes(spec, oc.TERNARY2)], oc.page_tiles(spec, ref, 0)), s
