"""GPU parity of the five seeded workloads against the CPU oracle.

Each test runs the workload at its full size through the C ABI, in the same
launch configuration the benchmark times, and checks sampled sequences,
layers and pages bit-exactly (codes, bytes), gamma within 2^-22 and decode
outputs within max-abs 2e-3 of the float64 oracle.
"""
import pytest
import torch

from bit_ternary_attention_amd import workloads as wl

from gpu_harness import run_workload, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

# 2 = matrix-core decode (the default), 1 = vector-ALU decode
KERNELS = pytest.mark.parametrize("kernel", [2, 1], ids=["mfma", "valu"])


@KERNELS
def test_workload1_tiny(kernel):
    w = wl.workload(1)
    r = run_workload(w, sample_seqs=[0], page_layers=[0], decode_layers=[0], decode_kernel=kernel)
    assert r["stats"]["last_decode_units"] == [17, 0, 0]   # units holding tokens 0..3 and 256..511
    say(f"workload 1: {r}")


@KERNELS
def test_workload2_qwen_shaped_36_layers(kernel):
    w = wl.workload(2)
    r = run_workload(w, sample_seqs=[0], page_layers=[0, 17, 35], decode_layers=list(range(36)), decode_kernel=kernel)
    assert r["stats"]["pages_used"] == [256, 0, 0]
    say(f"workload 2: max err {r['max_err']:.3e}")


@KERNELS
def test_workload3_full_retention_outliers(kernel):
    w = wl.workload(3)
    r = run_workload(w, sample_seqs=[0, 13, 31], page_layers=[0], decode_layers=[0], decode_kernel=kernel)
    assert r["stats"]["last_decode_steal"] == 0   # stealing blocks are opt-in
    say(f"workload 3: max err {r['max_err']:.3e}")


@KERNELS
def test_workload4_mixed_format_paged(kernel):
    w = wl.workload(4)
    lengths = list(w.lengths)
    sample = sorted({lengths.index(min(lengths)), lengths.index(max(lengths)), 5, 40})
    r = run_workload(w, sample_seqs=sample, page_layers=[0], decode_layers=[0], decode_kernel=kernel)
    units = r["stats"]["last_decode_units"]
    assert units[0] > 0 and units[1] > 0 and units[2] == 64   # every route ran
    say(f"workload 4: max err {r['max_err']:.3e} units {units}")


@KERNELS
def test_workload4_dynamic_fp8(kernel):
    """Workload 4 with the recent tier in dynamic FP8 (one scale per token and KV head)."""
    w = wl.workload(4)
    lengths = list(w.lengths)
    sample = sorted({lengths.index(max(lengths)), 7, 40})
    r = run_workload(w, sample_seqs=sample, page_layers=[0], decode_layers=[0], decode_kernel=kernel, fp8_dynamic=1)
    assert r["stats"]["last_decode_units"][1] > 0
    say(f"workload 4 dynamic fp8: max err {r['max_err']:.3e}")


@KERNELS
def test_workload5_prefill_128k_chunked(kernel):
    w = wl.workload(5)
    r = run_workload(w, sample_seqs=[2], page_layers=[0], decode_layers=[0], decode_kernel=kernel)
    assert r["stats"]["append_calls"] == 32
    assert r["stats"]["last_decode_steal"] == 0
    say(f"workload 5: max err {r['max_err']:.3e}")
