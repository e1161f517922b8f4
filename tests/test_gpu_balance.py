"""GPU parity of the balanced split plan.

24 equal-length sequences x 8 KV heads of 2048 tokens (head dim 128 with bfloat16
queries, head dim 64 with float16 ones): the plain plan (about two blocks per
compute unit) takes 3 splits, 576 blocks, which puts 3 blocks on some compute units and 2 on
others; the balanced plan takes 4 splits, 768 blocks, 3 on every compute unit.  Both plans'
outputs are compared with the float64 oracle for every sequence (exact attention over the
pages read directly: Minima-KV, "How mixed-format attention works").
"""

import pytest
import torch

from bit_ternary_attention_amd import workloads as wl

from gpu_harness import run_workload, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

def _workload(window, head_dim, dtype):
    return wl.small_workload(n_q_heads=32, n_kv_heads=8, head_dim=head_dim, dtype=dtype, window=window,
                             lengths=(2048,) * 24, page_shuffle_seed=5, number=11)

def _n_cu():
    return torch.cuda.get_device_properties(0).multi_processor_count

@pytest.mark.parametrize("balance", [True, False], ids=["balanced", "plain"])
@pytest.mark.parametrize("window", [-1, 1500])
@pytest.mark.parametrize("head_dim,dtype", [(128, wl.DTYPE_BF16), (64, wl.DTYPE_F16)], ids=["d128-bf16", "d64-f16"])
def test_balanced_split_plan_parity(balance, window, head_dim, dtype, monkeypatch):
    if not balance:
        monkeypatch.setenv("VK_DECODE_BALANCE", "0")
    monkeypatch.delenv("VK_DECODE_BLOCKS_PER_CU", raising=False)
    w = _workload(window, head_dim, dtype)
    r = run_workload(w, page_layers=[], decode_layers=[0])
    assert r["seqs_decoded"] == w.n_seqs
    splits = r["stats"]["last_decode_splits"]
    if _n_cu() == 256 and window == -1:
        assert splits == (4 if balance else 3), splits
    say(f"24 x 2048 tokens, head dim {head_dim}, window {window}, balance {balance}: {splits} splits, "
        f"max err {r['max_err']:.3e}")
