"""Head dim 256 on the GPU against the CPU oracle.

At head dim 256 the cache is written by the same pack kernel (value chunks of 16
bytes: two head-dim-128 chunks side by side) and read by either decode kernel
(the matrix-core one, the default, with a 4-slot ring of 2 KB rows and no
stealing blocks; or the vector-ALU one).  Every page is compared
bit for bit with the oracle's encoding and every decode output within the
attention tolerance, over group sizes 1-8, ragged lengths, windows, fp16 and
fp8 tiers (static and dynamic scales), block sizes and both input dtypes, plus
one long multi-sequence launch with several splits per sequence.
"""
import pytest
import torch

from bit_ternary_attention_amd import vk
from bit_ternary_attention_amd import workloads as wl
from oracle import cache as oc

from gpu_harness import check_decode, check_pages, fill, host_kv, make_cache, run_workload, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

D256_CASES = [
    # (name, workload kwargs, windows)
    ("gqa1-f16", dict(n_q_heads=2, n_kv_heads=2, lengths=(300, 17)), [-1, 40]),
    ("gqa2-bf16", dict(n_q_heads=4, n_kv_heads=2, dtype=1, lengths=(1030, 5, 260)), [-1, 0, 500]),
    ("gqa4-f16-bs32", dict(n_q_heads=8, n_kv_heads=2, block_size=32, lengths=(777, 64)), [-1, 100]),
    ("gqa8-bf16", dict(n_q_heads=16, n_kv_heads=2, dtype=1, lengths=(1100, 1)), [-1, 300]),
    ("gqa8-no-sinks", dict(n_q_heads=16, n_kv_heads=2, sink_tokens=0, lengths=(333,)), [-1, 1, 17]),
    ("mixed-tiers-f16-fp8", dict(n_q_heads=8, n_kv_heads=2, dtype=1, sink_format=oc.F16, recent_tokens=48,
                                 recent_format=oc.FP8E4M3, lengths=(700, 31, 250), page_shuffle_seed=99,
                                 batch_appends=False), [-1, 60, 0]),
    ("recent-f16-sink-fp8", dict(n_q_heads=4, n_kv_heads=2, sink_tokens=20, sink_format=oc.FP8E4M3,
                                 recent_tokens=32, recent_format=oc.F16, lengths=(400,)), [-1, 33]),
    ("chunked-bs64", dict(n_q_heads=8, n_kv_heads=4, block_size=64, lengths=(640, 130), chunk_tokens=128),
     [-1, 200]),
    ("ragged-appends", dict(n_q_heads=8, n_kv_heads=2, dtype=1, sink_format=oc.F16, recent_tokens=48,
                            recent_format=oc.FP8E4M3, lengths=(333, 100, 48), chunk_tokens=48,
                            ragged_appends=True), [-1, 70]),
]


def _has_fp8(kw):
    return oc.FP8E4M3 in (kw.get("sink_format"), kw.get("recent_format"))


# dynamic FP8 scales only where the case holds fp8 pages
D256_PARAMS = [pytest.param(name, kw, windows, kernel, dyn,
                            id=f"{name}-{kid}-{'dynamic' if dyn else 'static'}-fp8")
               for name, kw, windows in D256_CASES
               for kernel, kid in ((2, "mfma"), (1, "valu"))
               for dyn in ((0, 1) if _has_fp8(kw) else (0,))]


@pytest.mark.parametrize("name,kw,windows,kernel,dyn", D256_PARAMS)
def test_head_dim_256(name, kw, windows, kernel, dyn):
    w = wl.small_workload(head_dim=256, **kw)
    say(f"d256 {name} kernel {kernel} dynamic fp8 {dyn}: {w}")
    cache = make_cache(w, decode_kernel=kernel, fp8_dynamic=dyn)
    fill(cache, w)
    encs = {}
    for s in range(w.n_seqs):
        kb, vb = host_kv(w, 0, s)
        encs[s] = check_pages(cache, w, 0, s, kb, vb, pages=list(range(-(-w.lengths[s] // w.block_size))),
                              fp8_dynamic=dyn)
    q = wl.queries(w, 0, device="cuda")
    for W in windows:
        if w.sink_tokens == 0 and W == 0:
            continue
        out = cache.decode(q, list(range(w.n_seqs)), 0, window=W)
        torch.cuda.synchronize()
        err = check_decode(out, q, w, encs, W)
        say(f"d256 {name} window {W}: max err {err:.2e}")
    cache.close()


@pytest.mark.parametrize("kernel", [2, 1], ids=["mfma", "valu"])
def test_head_dim_256_long_launch(kernel):
    """Eight sequences of 6k-16k bfloat16 tokens, 16 query / 8 KV heads (group 2), shuffled
    pages, full retention: several splits per (sequence, KV head), merged; the matrix-core
    waves walk their ring many times over."""
    lengths = (16384, 12000, 9001, 16000, 6000, 15999, 8192, 11111)
    w = wl.small_workload(n_q_heads=16, n_kv_heads=8, head_dim=256, dtype=wl.DTYPE_BF16, lengths=lengths,
                          page_shuffle_seed=21, number=11)
    r = run_workload(w, page_layers=[0], decode_layers=[0], decode_kernel=kernel)
    assert r["seqs_decoded"] == w.n_seqs
    assert r["pages"] == sum(-(-L // w.block_size) for L in lengths)
    assert r["stats"]["last_decode_splits"] > 1
    say(f"d256 long launch ({kernel}): {r['stats']['last_decode_splits']} splits, max err {r['max_err']:.3e}")


def test_head_dim_256_stealing_blocks_not_taken(monkeypatch):
    """VK_DECODE_STEAL=2 asks for stealing blocks wherever the shape allows; head dim 256 has
    no such instance, so the 4-wave blocks run and the outputs stay on the oracle."""
    monkeypatch.setenv("VK_DECODE_STEAL", "2")
    w = wl.small_workload(n_q_heads=8, n_kv_heads=2, head_dim=256, dtype=1, lengths=(3000,))
    cache = make_cache(w, decode_kernel=2)
    fill(cache, w)
    kb, vb = host_kv(w, 0, 0)
    enc = check_pages(cache, w, 0, 0, kb, vb, pages=[0, 1, 100, 187])
    q = wl.queries(w, 0, device="cuda")
    out = cache.decode(q, [0], 0, window=-1)
    torch.cuda.synchronize()
    assert cache.stats()["last_decode_steal"] == 0
    say(f"d256 steal refused: max err {check_decode(out, q, w, {0: enc}, -1):.2e}")
    cache.close()


def test_head_dim_256_refuses_lossless():
    base = dict(n_layers=1, n_kv_heads=2, n_q_heads=4, head_dim=256, block_size=16, max_seqs=1,
                max_tokens_per_seq=64, pages_ternary=8, pages_lossless=2)
    for bad in (dict(sink_format=wl.FMT_LOSSLESS), dict(recent_tokens=16, recent_format=wl.FMT_LOSSLESS)):
        with pytest.raises(vk.VkError):
            vk.Cache(vk.make_config(**base, **bad))
