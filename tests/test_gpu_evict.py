"""GPU checks of bounded-memory eviction: a long single-token stream per sequence with
retiering and eviction after every append, in pools far smaller than the stream.

Decode over sinks + window (no wider than the eviction window) must match the oracle's
attention over the full, never-evicted sequence (max-abs 2e-3) with both decode
kernels; wider windows are refused; the pages in use stay within the bound.
"""
import numpy as np
import pytest
import torch

from bit_ternary_attention_amd import vk
from bit_ternary_attention_amd import workloads as wl
from oracle import attention as oa
from oracle import cache as oc
from oracle import ternary as ot

from gpu_harness import ATTN_ATOL, say
from test_gpu_retier import Stream, make, spec_for

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def decode_errors(cache, st, spec, window, S):
    q = st.query()
    ids = list(range(st.n_seqs))
    worst = 0.0
    for layer in range(st.n_layers):
        out = cache.decode(q, ids, layer, window=window).cpu().numpy()
        qv = ot.values16(wl.to_bits(q), st.dtype)
        for s in ids:
            kb, vb = st.bits(layer, s)
            enc = oc.retier(spec, oc.encode_sequence(spec, kb, vb, st.dtype, st.calls[s]))
            ref = oa.decode_attention(qv[s], enc.k_hat, enc.v_hat, enc.length, S, window)
            err = float(np.max(np.abs(out[s] - ref)))
            assert err <= ATTN_ATOL, (layer, s, window, err)
            worst = max(worst, err)
    return worst


@pytest.mark.parametrize("kernel", [2, 1], ids=["mfma", "valu"])
def test_streaming_with_eviction(kernel):
    S, R, W, bs = 4, 48, 128, 16
    st = Stream(2, 4, 2, 16, 128, wl.DTYPE_BF16, seed=7)
    n = st.n_seqs
    per_seq = -(-S // bs) + -(-W // bs) + 2
    cache = make(st, bs, S, wl.FMT_F16, R, (n * per_seq, n * (-(-R // bs) + 2), n), decode_kernel=kernel)
    spec = spec_for(st, bs, S, wl.FMT_F16, R)
    ids = list(range(n))
    k, v = st.draw(ids, 150)
    cache.append(k, v, ids)
    cache.retier(ids)
    freed = cache.evict(ids, W)
    bound = n * (-(-S // bs) + -(-W // bs) + 1)
    for step in range(250):
        k, v = st.draw(ids, 1)
        cache.append(k, v, ids)
        cache.retier(ids)
        freed += cache.evict(ids, W)
        used = sum(cache.stats()["pages_used"])
        assert used <= bound, (step, used, bound)
        if step in (30, 249):
            torch.cuda.synchronize()
            for window in (W, 50):
                err = decode_errors(cache, st, spec, window, S)
                say(f"  step {step} window {window}: max abs err {err:.3e}, pages in use {used}")
    assert freed == cache.stats()["pages_evicted"] == n * len(oc.evict_pages(spec, 400, W))
    # 400 tokens per sequence would need 25 pages each without eviction; the pools hold per_seq
    assert st.length[0] == 400 and 400 // bs > per_seq
    for window in (-1, W + bs):
        with pytest.raises(vk.VkError) as e:
            cache.decode(st.query(), ids, 0, window=window)
        assert e.value.status == vk.ERR_ARG
    _, fmt, _ = cache.read_pages(0, 0, 0, 400 // bs)
    gone = [p for p, f in enumerate(fmt) if f == -1]
    assert gone == oc.evict_pages(spec, 400, W)
