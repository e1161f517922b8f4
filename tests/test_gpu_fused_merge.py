"""The matrix-core decode's fused split merge against the two-launch path.

With several parts per (sequence, KV head) and no lossless pages, the last block of each pair
to finish combines the parts itself (device-coherent part stores, a device-scope part counter)
instead of a k_merge launch.  It must give the same outputs bit for bit as the merge launch
(VK_DECODE_FUSED_MERGE=0), call after call (the counters return to zero), on launches whose
parts are splits, fp8 / fp16 blocks or both, over group sizes 1-8 and head dims 64, 128 and
256, and when one call holds more sequences than a launch (several launches in a row reuse
the counters).  The oracle comparison of the same path is in the parity tests, which run it
by default.
"""
import os

import numpy as np
import pytest
import torch

from bit_ternary_attention_amd import workloads as wl
from oracle import cache as oc

from gpu_harness import fill, make_cache, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

CASES = [
    ("full-retention-like", dict(n_q_heads=32, n_kv_heads=8, head_dim=128, dtype=wl.DTYPE_BF16,
                                 lengths=(4096,) * 6), [-1]),
    ("mixed-tiers-g8", dict(n_q_heads=16, n_kv_heads=2, head_dim=128, dtype=wl.DTYPE_BF16, sink_format=oc.F16,
                            recent_tokens=256, recent_format=oc.FP8E4M3, lengths=(3000, 700, 257, 40),
                            page_shuffle_seed=7), [-1, 300]),
    ("g1-d64-ragged", dict(n_q_heads=2, n_kv_heads=2, head_dim=64, lengths=(9000, 1, 3000, 33)), [-1, 100]),
    ("g2-d256", dict(n_q_heads=4, n_kv_heads=2, head_dim=256, dtype=wl.DTYPE_BF16, lengths=(2048, 513)), [-1]),
    ("many-seqs", dict(n_q_heads=8, n_kv_heads=2, head_dim=128, lengths=tuple(200 + 37 * i for i in range(70))),
     [-1]),
]


def _decode(cache, q, ids, W, fused):
    old = os.environ.get("VK_DECODE_FUSED_MERGE")
    os.environ["VK_DECODE_FUSED_MERGE"] = "1" if fused else "0"
    try:
        return cache.decode(q, ids, 0, window=W).cpu().numpy()
    finally:
        if old is None:
            os.environ.pop("VK_DECODE_FUSED_MERGE", None)
        else:
            os.environ["VK_DECODE_FUSED_MERGE"] = old


@pytest.mark.parametrize("name,kw,windows", CASES, ids=[c[0] for c in CASES])
def test_fused_merge_equals_merge_launch(name, kw, windows):
    w = wl.small_workload(**kw)
    cache = make_cache(w, decode_kernel=2)
    fill(cache, w)
    q = wl.queries(w, 0, device="cuda")
    ids = list(range(w.n_seqs))
    for W in windows:
        ref = _decode(cache, q, ids, W, fused=False)
        splits = cache.stats()["last_decode_splits"]
        for rep in range(3):
            got = _decode(cache, q, ids, W, fused=True)
            assert np.array_equal(got, ref), f"{name} window {W} call {rep}: fused merge differs"
        say(f"fused merge {name} window {W} ({splits} splits): equal to the merge launch over 3 calls")
    cache.close()
