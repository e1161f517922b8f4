"""The pipelined all-ternary pack kernel against the oracle and against the one-task kernel.

Short all-ternary appends at head dims 64 and 128 run k_pack_tern, whose blocks walk a run of
tasks with the next task's loads in flight; VK_PACK_PIPE=0 makes the same calls run k_pack's
one-task blocks.  Both caches must hold the same bytes and gammas in every page, and the
pipelined one must equal the oracle's encoding (page bytes bit for bit).  The cases cross
sequence and layer boundaries inside a block's run (ragged calls, several layers per call,
block-per-CU settings that give runs of 1 to 16 tasks), and end calls inside a unit.
"""
import os

import numpy as np
import pytest
import torch

from bit_ternary_attention_amd import vk
from bit_ternary_attention_amd import workloads as wl

from gpu_harness import check_pages, fill, host_kv, make_cache, read_all_pages, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

CASES = [
    # (name, workload kwargs, VK_PACK_BLOCKS_PER_CU)
    ("d128-bf16-4seq-chunks", dict(n_q_heads=8, n_kv_heads=4, head_dim=128, dtype=wl.DTYPE_BF16,
                                   lengths=(1024, 1024, 1024, 1024), chunk_tokens=256), 16),
    ("d128-f16-3layers-ragged", dict(n_layers=3, n_q_heads=8, n_kv_heads=2, head_dim=128,
                                     lengths=(700, 33, 1, 250), chunk_tokens=96, ragged_appends=True), 1),
    ("d64-bf16-ragged-tail", dict(n_q_heads=4, n_kv_heads=2, head_dim=64, dtype=wl.DTYPE_BF16,
                                  lengths=(517, 16, 95), chunk_tokens=64, ragged_appends=True), 3),
    ("d64-f16-2layers-bs64", dict(n_layers=2, n_q_heads=8, n_kv_heads=8, head_dim=64, block_size=64,
                                  lengths=(640, 130)), 64),
]


def _fill_with(w, pipe, per_cu):
    old = {k: os.environ.get(k) for k in ("VK_PACK_PIPE", "VK_PACK_BLOCKS_PER_CU")}
    os.environ["VK_PACK_PIPE"] = "1" if pipe else "0"
    os.environ["VK_PACK_BLOCKS_PER_CU"] = str(per_cu)
    try:
        cache = make_cache(w)
        fill(cache, w)
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    return cache


@pytest.mark.parametrize("name,kw,per_cu", CASES, ids=[c[0] for c in CASES])
def test_pipelined_pack_matches_one_task_kernel_and_oracle(name, kw, per_cu):
    w = wl.small_workload(**kw)
    say(f"pack pipe {name}: {w}, {per_cu} blocks per CU")
    a = _fill_with(w, True, per_cu)
    b = _fill_with(w, False, per_cu)
    for layer in range(w.n_layers):
        for s in range(w.n_seqs):
            ga, gb = read_all_pages(a, layer, s), read_all_pages(b, layer, s)
            for x, y in zip(ga, gb):
                np.testing.assert_array_equal(x, y)
            kb, vb = host_kv(w, layer, s)
            check_pages(a, w, layer, s, kb, vb, pages=list(range(-(-w.lengths[s] // w.block_size))))
    a.close()
    b.close()
