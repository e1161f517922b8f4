"""GPU parity of the five seeded workloads against the CPU oracle.

Each test runs the workload at its full size through the C ABI, in the same
launch configuration the benchmark times, and compares every sequence with the
oracle: every page's stored codes, fp8 bytes and fp16 values bit-exactly (and
every ternary page's gamma within 2^-22), and every sequence's decode output
within max-abs 2e-3 of the float64 oracle.
"""
import dataclasses

import pytest
import torch

from bit_ternary_attention_amd import workloads as wl

from gpu_harness import run_workload, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

# 2 = matrix-core decode (the default), 1 = vector-ALU decode
KERNELS = pytest.mark.parametrize("kernel", [2, 1], ids=["mfma", "valu"])


def total_pages(w, layers):
    return len(layers) * sum(-(-L // w.block_size) for L in w.lengths)


def check_all(w, r, page_layers, decode_layers):
    assert r["pages"] == total_pages(w, page_layers)
    assert r["seqs_decoded"] == w.n_seqs * len(decode_layers)


@KERNELS
def test_workload1_tiny(kernel):
    w = wl.workload(1)
    r = run_workload(w, page_layers=[0], decode_layers=[0], decode_kernel=kernel)
    check_all(w, r, [0], [0])
    assert r["stats"]["last_decode_units"] == [17, 0, 0, 0]   # units holding tokens 0..3 and 256..511
    say(f"workload 1: {r}")


@KERNELS
def test_workload2_qwen_shaped_36_layers(kernel):
    w = wl.workload(2)
    layers = list(range(36))
    r = run_workload(w, page_layers=layers, decode_layers=layers, decode_kernel=kernel)
    check_all(w, r, layers, layers)
    assert r["stats"]["pages_used"] == [256, 0, 0, 0]
    say(f"workload 2: max err {r['max_err']:.3e}")


@KERNELS
def test_workload3_full_retention_outliers(kernel):
    w = wl.workload(3)
    r = run_workload(w, page_layers=[0], decode_layers=[0], decode_kernel=kernel)
    check_all(w, r, [0], [0])
    assert r["stats"]["last_decode_steal"] == 0   # stealing blocks are opt-in
    assert r["stats"]["last_decode_ordered"] == 0  # equal lengths: the plain grid
    say(f"workload 3: max err {r['max_err']:.3e}")


@KERNELS
def test_workload4_mixed_format_paged(kernel):
    w = wl.workload(4)
    r = run_workload(w, page_layers=[0], decode_layers=[0], decode_kernel=kernel)
    check_all(w, r, [0], [0])
    units = r["stats"]["last_decode_units"]
    assert units[0] > 0 and units[1] > 0 and units[2] == 64   # every route ran
    # ragged lengths and fp8 / fp16 parts: the matrix-core launch dispatches from its order table
    assert r["stats"]["last_decode_ordered"] == (0 if kernel == 1 else 1)
    say(f"workload 4: max err {r['max_err']:.3e} units {units}")


@KERNELS
def test_workload4_dynamic_fp8(kernel):
    """Workload 4 with the recent tier in dynamic FP8 (one scale per token and KV head)."""
    w = wl.workload(4)
    r = run_workload(w, page_layers=[0], decode_layers=[0], decode_kernel=kernel, fp8_dynamic=1)
    check_all(w, r, [0], [0])
    assert r["stats"]["last_decode_units"][1] > 0
    say(f"workload 4 dynamic fp8: max err {r['max_err']:.3e}")


def test_workload4_lossless_anchor_tier():
    """Workload 4 with its sink pages in the lossless bfloat16 tier instead of fp16 (matrix-core
    decode: the vector-ALU kernel does not read lossless pages)."""
    w = dataclasses.replace(wl.workload(4), sink_format=wl.FMT_LOSSLESS)
    r = run_workload(w, page_layers=[0], decode_layers=[0], decode_kernel=2)
    check_all(w, r, [0], [0])
    units = r["stats"]["last_decode_units"]
    assert units[wl.FMT_LOSSLESS] == 64 and units[wl.FMT_F16] == 0 and units[wl.FMT_FP8E4M3] > 0
    say(f"workload 4 lossless anchors: max err {r['max_err']:.3e} units {units}")


@KERNELS
def test_workload5_prefill_128k_chunked(kernel):
    w = wl.workload(5)
    r = run_workload(w, page_layers=[0], decode_layers=[0], decode_kernel=kernel)
    check_all(w, r, [0], [0])
    assert r["stats"]["append_calls"] == 32
    assert r["stats"]["last_decode_steal"] == 0
    say(f"workload 5: max err {r['max_err']:.3e}")


@pytest.mark.parametrize("head_dim", [128, 256])
def test_long_windowed_ranges_take_the_long_path(head_dim):
    """Sinks plus a recent window over long sequences of different lengths, in a launch large
    enough that every wave walks more than one ring of units (the long-range path, whose
    ternary scores use the fp4 product): the attended set is two unit ranges with the window's
    first unit partly attended.  Every sequence's output against the oracle."""
    lengths = (20000, 19000, 18007, 20000, 17555, 19999, 20000, 18888)
    w = wl.small_workload(n_q_heads=32, n_kv_heads=8, head_dim=head_dim, dtype=wl.DTYPE_BF16, window=9001,
                          lengths=lengths, page_shuffle_seed=11, number=10)
    r = run_workload(w, page_layers=[], decode_layers=[0])
    assert r["seqs_decoded"] == w.n_seqs
    max_units = 1 + -(-(9001 + 15) // 16)  # the sink unit and the window's units (an upper bound)
    splits = r["stats"]["last_decode_splits"]
    ring = 8 if head_dim == 128 else 4    # ring slots per wave
    assert max_units / splits > 4 * ring, "the launch must give its waves more than one ring of units"
    say(f"long windowed ranges, head dim {head_dim}: {splits} splits, max err {r['max_err']:.3e}")
