"""Benchmark: quantize+pack into the packed ternary KV cache, then decode attention over it.

One step is one pass of the whole hot path over one batch of synthetic input:
every append call of the workload (absmean pass, gamma finalize, quantise +
pack + page scatter) followed by one decode step of every layer.  The default
workload is the Qwen2.5-3B-shaped cache (36 layers, 16 query / 2 KV heads,
head_dim 128, 4096 bf16 tokens, sinks 4 + window 256).  Other workloads are
selectable with --workload for reference numbers.

Prints one JSON line.  `value` is whole-step algorithmic bytes / step time
(GB/s): both passes of the write side over the input, every stored byte, and
the attended page bytes the decode reads.  Inputs are resident in HBM before
the timed region; several input sets rotate so that no step reads inputs still
held in the 256 MB Infinity Cache from an earlier step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MIN_WARMUP_S = 0.3   # untimed warm-up lasts at least this long (and at least --warmup steps)
METRIC = "decode-attn over packed KV: GB/s & % HBM peak; quantize+pack GB/s"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", type=int, default=2, help="1..5 (default 2: Qwen2.5-3B-shaped)")
    ap.add_argument("--decode-kernel", type=int, default=0, help="0 default, 1 vector ALU, 2 matrix cores")
    ap.add_argument("--fp8-dynamic", action="store_true",
                    help="FP8 pages with one scale per token and KV head instead of the static scale")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-layers", type=int, default=0, help="0 = workload's own sample rule")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (counter calibration)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import numpy as np
    import torch

    from bit_ternary_attention_amd import vk
    from bit_ternary_attention_amd import workloads as wl

    torch.cuda.set_device(0)
    if args.calibration_copy_mib:
        # a plain copy of known size (read n bytes, write n bytes) under a kernel name of its
        # own, to scale the FETCH_SIZE / WRITE_SIZE counters
        n = args.calibration_copy_mib * 2 ** 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    w = wl.workload(args.workload)
    calls = w.appends()
    ids_all = list(range(w.n_seqs))

    # pages per format needed by one step (format rule of the cache config)
    cfg = vk.make_config(n_layers=w.n_layers, n_kv_heads=w.n_kv_heads, n_q_heads=w.n_q_heads,
                         head_dim=w.head_dim, block_size=w.block_size, max_seqs=w.n_seqs,
                         max_tokens_per_seq=w.max_len, sink_tokens=w.sink_tokens, sink_format=w.sink_format,
                         recent_tokens=w.recent_tokens, recent_format=w.recent_format,
                         page_shuffle_seed=w.page_shuffle_seed, decode_kernel=args.decode_kernel,
                         fp8_dynamic=int(args.fp8_dynamic))
    need = [0, 0, 0]
    bs = w.block_size
    for s in range(w.n_seqs):
        for ids, t0, n in calls:
            if s not in ids:
                continue
            for p in range(-(-t0 // bs), -(-(t0 + n) // bs)):
                lo = p * bs
                if p < -(-w.sink_tokens // bs):
                    f = w.sink_format
                elif w.recent_tokens > 0 and lo < t0 + n and lo + bs > t0 + n - w.recent_tokens:
                    f = w.recent_format
                else:
                    f = vk.FMT_TERNARY2
                need[f] += 1
    cfg.pages_ternary, cfg.pages_fp8, cfg.pages_f16 = need
    cache = vk.Cache(cfg)

    # inputs resident in HBM: rotate enough sets to exceed the 256 MB Infinity Cache
    in_bytes = sum(2 * w.n_layers * len(ids) * n * w.n_kv_heads * w.head_dim * 2 for ids, _, n in calls)
    n_sets = max(1, min(3, -(-768 * 2 ** 20 // in_bytes)))
    sets = []
    for r in range(n_sets):
        per_call = []
        for ci, (ids, t0, n) in enumerate(calls):
            k, v = wl.append_inputs(w, ids, t0, n, device="cuda")
            if r:  # other sets: same shapes, different draws
                k = k[:, :, torch.randperm(n, device="cuda")].contiguous()
                v = v[:, :, torch.randperm(n, device="cuda")].contiguous()
            per_call.append((ids, k, v))
        sets.append(per_call)
    qs = [wl.queries(w, layer, device="cuda") for layer in range(w.n_layers)]
    outs = [torch.empty(q.shape, dtype=torch.float32, device="cuda") for q in qs]
    torch.cuda.synchronize()

    def step(i, seg=None):
        cache.reset(ids_all)
        for ids, k, v in sets[i % n_sets]:
            cache.append(k, v, ids)
        if seg is not None:
            seg[0].record()
        for layer in range(w.n_layers):
            cache.decode(qs[layer], ids_all, layer, window=w.window, out=outs[layer])
        if seg is not None:
            seg[1].record()

    # W warm-up steps, then more untimed steps until the warm-up has lasted MIN_WARMUP_S: a
    # GPU coming out of idle needs some time under load before its throughput is steady
    tw = time.perf_counter()
    warm = 0
    while warm < args.warmup or time.perf_counter() - tw < MIN_WARMUP_S:
        step(warm)
        warm += 1
        if warm >= args.warmup:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps

    # the same steps with one event pair per step around its decode launches (the launch stream
    # is torch's current one): the decode segment's device time without a pair of events around
    # every launch
    segs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, segs[i])
    torch.cuda.synchronize()
    decode_seg_ms = sum(a.elapsed_time(b) for a, b in segs) / args.steps

    # same steps again with per-kernel HIP event timing (library hooks on the launch stream)
    cache.kernel_timing(True)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    kt = cache.kernel_times()
    cache.kernel_timing(False)
    ms_step_timed = (t3 - t2) * 1e3 / args.steps
    stats = cache.stats()

    kernels = {}
    for name, (launches, ms, by) in kt.items():
        if launches == 0:
            continue
        avg_us = ms * 1e3 / launches
        gbps = by / (ms * 1e-3) / 1e9 if ms > 0 else 0.0
        kernels[name] = {"launches_per_step": launches / args.steps, "avg_us": round(avg_us, 3),
                         "bytes_per_launch": by / launches, "GBps": round(gbps, 1),
                         "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
                         "ms_per_step": round(ms / args.steps, 4)}
    step_bytes = sum(by for (_, _, by) in kt.values()) / args.steps
    write_bytes = sum(kt[k][2] for k in ("absmean", "finalize", "pack")) / args.steps
    write_ms = sum(kt[k][1] for k in ("absmean", "finalize", "pack")) / args.steps
    read_bytes = sum(kt[k][2] for k in ("decode", "merge")) / args.steps
    read_ms = sum(kt[k][1] for k in ("decode", "merge")) / args.steps
    dominant = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    dk = dict(kernels[dominant])
    if dominant == "decode" and "merge" not in kernels:
        # decode launches back to back with nothing between them: their average duration from
        # the segment's events (an event pair around each launch adds a few microseconds to a
        # launch this short)
        dk["avg_us_per_launch_events"] = dk["avg_us"]
        dk["avg_us"] = round(decode_seg_ms * 1e3 / dk["launches_per_step"], 3)
        dk["GBps"] = round(dk["bytes_per_launch"] / (dk["avg_us"] * 1e-6) / 1e9, 1)
        dk["hbm_frac"] = round(dk["GBps"] / HBM_PEAK_GBPS, 4)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    kv_tokens = sum(len(ids) * n for ids, _, n in calls)

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "dtype_detail": ("bf16/f16 inputs; 2-bit codes, 4 per u8; f16 x f16 -> f32 dot products; "
                         "f32 softmax and accumulation"),
        "data": "synthetic (seeded torch.randn, see bit_ternary_attention_amd/workloads.py)",
        "config": {"workload": w.name, "layers": w.n_layers, "seqs": w.n_seqs,
                   "tokens_per_seq": list(sorted(set(w.lengths))) if len(set(w.lengths)) > 1 else w.lengths[0],
                   "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size, "sink_tokens": w.sink_tokens, "window": w.window,
                   "append_calls": len(calls), "input_sets": n_sets,
                   "fp8": "dynamic per (token, head)" if args.fp8_dynamic else "static scale"},
        "quantize_pack": {"GBps": round(write_bytes / (write_ms * 1e-3) / 1e9, 1),
                          "hbm_frac": round(write_bytes / (write_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                          "bytes_per_step": write_bytes, "device_ms_per_step": round(write_ms, 4),
                          "kv_tokens_per_s": round(kv_tokens * w.n_layers / (write_ms * 1e-3), 1)},
        "decode_attn": {"GBps": round(read_bytes / (read_ms * 1e-3) / 1e9, 1),
                        "hbm_frac": round(read_bytes / (read_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                        "bytes_per_step": read_bytes, "device_ms_per_step": round(read_ms, 4),
                        "us_per_layer": round(read_ms * 1e3 / w.n_layers, 3),
                        "segment_us_per_layer": round(decode_seg_ms * 1e3 / w.n_layers, 3),
                        "splits": stats["last_decode_splits"], "units_by_format": stats["last_decode_units"],
                        "kernel": {0: "default (matrix cores)", 1: "vector ALU", 2: "matrix cores"}[args.decode_kernel]},
        "kernels": kernels,
        "ms_per_step_with_kernel_timing": round(ms_step_timed, 4),
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": dk["GBps"], "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": dk["hbm_frac"], "traffic": measured_traffic(dominant, w.name),
                     "bytes_per_launch": dk["bytes_per_launch"], "avg_launch_us": dk["avg_us"],
                     "timing": ("decode segment events over the timed steps / launches"
                                if "avg_us_per_launch_events" in dk else "event pair around each launch"),
                     **({"avg_launch_us_event_pairs": dk["avg_us_per_launch_events"]}
                        if "avg_us_per_launch_events" in dk else {})},
    }

    result["decode_step"] = decode_step_leg(cache, qs, outs, w, ids_all)

    if w.recent_tokens > 0 and w.recent_format == vk.FMT_FP8E4M3:
        cache.close()
        result["retier"] = retier_leg(w, args.steps, args.warmup, args.fp8_dynamic)
        result["stream"] = stream_leg(w, args.steps, args.warmup, fp8_dynamic=args.fp8_dynamic)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, calls, args.cpu_sample_layers)
    print(json.dumps(result), flush=True)
    cache.close()


def attended_tokens(L, S, W):
    """Tokens a decode attends: the first S and the last W (W = -1: all), counted once."""
    if W < 0:
        return L
    a = min(S, L)
    return a + (L - max(a, L - W))


def decode_step_leg(cache, qs, outs, w, ids, reps=20):
    """One decode step of every layer, timed with events on the launch stream (median of reps),
    warm (right after the previous step) and cold: the 256 MB Infinity Cache and the L2s are
    first refilled by reading 1 GiB of other data (a read, so that no dirty lines are left to be
    written back during the timed step)."""
    import torch
    flush = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    res = {}
    for mode in ("warm", "cold"):
        times = []
        for r in range(reps):
            if mode == "cold":
                flush.sum()
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record()
            for layer in range(w.n_layers):
                cache.decode(qs[layer], ids, layer, window=w.window, out=outs[layer])
            t1.record()
            torch.cuda.synchronize()
            times.append(t0.elapsed_time(t1))
        times.sort()
        res[mode + "_us"] = round(1e3 * times[len(times) // 2], 2)
    del flush
    toks = sum(attended_tokens(L, w.sink_tokens, w.window) for L in w.lengths) * w.n_layers
    res.update({"layers": w.n_layers, "attended_tokens": toks, "reps": reps,
                "kv_tokens_per_s_warm": round(toks / (res["warm_us"] * 1e-6), 1),
                "kv_tokens_per_s_cold": round(toks / (res["cold_us"] * 1e-6), 1),
                "decode_steps_per_s_warm": round(w.n_seqs / (res["warm_us"] * 1e-6), 1),
                "decode_steps_per_s_cold": round(w.n_seqs / (res["cold_us"] * 1e-6), 1)})
    return res


def retier_leg(w, steps, warmup, fp8_dynamic=False):
    """FP8 -> ternary retiering on the workload's shape: every sequence gets R tokens (all
    in FP8 pages but the sink page), then R more, so the first R tokens' pages leave the
    recent window; one vk_retier call over all sequences converts them.  Only that call
    is timed (HIP events around its kernel)."""
    import torch

    from bit_ternary_attention_amd import vk

    R, bs = w.recent_tokens, w.block_size
    ids = list(range(w.n_seqs))
    n_sink = -(-w.sink_tokens // bs)
    cfg = vk.make_config(n_layers=w.n_layers, n_kv_heads=w.n_kv_heads, n_q_heads=w.n_q_heads,
                         head_dim=w.head_dim, block_size=bs, max_seqs=w.n_seqs, max_tokens_per_seq=2 * R,
                         sink_tokens=w.sink_tokens, sink_format=w.sink_format, recent_tokens=R,
                         recent_format=vk.FMT_FP8E4M3, fp8_dynamic=int(fp8_dynamic))
    per_seq = -(-2 * R // bs)
    cfg.pages_ternary = per_seq * w.n_seqs
    cfg.pages_fp8 = per_seq * w.n_seqs
    cfg.pages_f16 = n_sink * w.n_seqs
    cache = vk.Cache(cfg)
    g = torch.Generator(device="cuda")
    g.manual_seed(5000 + w.number)
    shape = (w.n_layers, w.n_seqs, R, w.n_kv_heads, w.head_dim)
    kv = [torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16) for _ in range(4)]
    converted = []

    def one(timed):
        cache.reset(ids)
        cache.append(kv[0], kv[1], ids)
        cache.append(kv[2], kv[3], ids)
        if timed:
            cache.kernel_timing(True)
        converted.append(cache.retier(ids))
        if timed:
            launches, ms, by = cache.kernel_times()["retier"]
            cache.kernel_timing(False)
            return launches, ms, by
        return None

    for _ in range(warmup):
        one(False)
    tot = [0, 0.0, 0.0]
    for _ in range(steps):
        la, ms, by = one(True)
        tot[0] += la
        tot[1] += ms
        tot[2] += by
    torch.cuda.synchronize()
    cache.close()
    gbps = tot[2] / (tot[1] * 1e-3) / 1e9
    return {"kernel": "retier", "pages_per_call": converted[-1], "layers": w.n_layers,
            "launches": tot[0], "avg_us": round(tot[1] * 1e3 / tot[0], 3),
            "bytes_per_launch": tot[2] / tot[0], "GBps": round(gbps, 1),
            "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
            "config": f"{w.n_seqs} seqs x {w.n_kv_heads} KV heads x head_dim {w.head_dim}, block {bs}: "
                      f"{R} + {R} tokens appended, pages {n_sink}..{R // bs - 1} of every sequence retiered"}


def stream_leg(w, steps, warmup, prefill=1024, window=512, fp8_dynamic=False):
    """A bounded-memory serving loop on the workload's shape (its sequences, heads, head dim,
    block size, sinks and FP8 recent tier): after a prefill, every step appends one token
    to every sequence, evicts the pages between the sinks and the last `window` tokens
    (max_active_tokens), retiers the FP8 pages that left the recent tier (evicting first
    spares converting pages that are about to go), and decodes one layer with that window.  Reports steps per second, the library's device time per
    kernel, the host time of the two page-table calls, and the pages in use (constant)."""
    import torch

    from bit_ternary_attention_amd import vk

    bs = w.block_size
    ids = list(range(w.n_seqs))
    n_steps = warmup + steps
    n_sink = -(-w.sink_tokens // bs)
    per_seq = n_sink + -(-window // bs) + 2
    cfg = vk.make_config(n_layers=1, n_kv_heads=w.n_kv_heads, n_q_heads=w.n_q_heads, head_dim=w.head_dim,
                         block_size=bs, max_seqs=w.n_seqs, max_tokens_per_seq=prefill + n_steps,
                         sink_tokens=w.sink_tokens, sink_format=w.sink_format, recent_tokens=w.recent_tokens,
                         recent_format=vk.FMT_FP8E4M3, fp8_dynamic=int(fp8_dynamic))
    chunk = 64  # prefill chunk: retier and evict after each, as the loop does per token
    cfg.pages_ternary = (per_seq + chunk // bs) * w.n_seqs
    cfg.pages_fp8 = ((w.recent_tokens + chunk) // bs + 3) * w.n_seqs
    cfg.pages_f16 = n_sink * w.n_seqs
    cache = vk.Cache(cfg)
    g = torch.Generator(device="cuda")
    g.manual_seed(6000 + w.number)
    shape = (prefill // chunk, 2, 1, w.n_seqs, chunk, w.n_kv_heads, w.head_dim)
    pre = torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16)
    tok = torch.randn((n_steps, 2, 1, w.n_seqs, 1, w.n_kv_heads, w.head_dim), generator=g,
                      device="cuda").to(torch.bfloat16)
    q = torch.randn((n_steps, w.n_seqs, w.n_q_heads, w.head_dim), generator=g, device="cuda").to(torch.bfloat16)
    out = torch.empty((w.n_seqs, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    for c in range(prefill // chunk):
        cache.append(pre[c, 0], pre[c, 1], ids)
        cache.evict(ids, window)
        cache.retier(ids)
    del pre
    host_s = [0.0, 0.0]

    def one(i):
        cache.append(tok[i, 0], tok[i, 1], ids)
        t = time.perf_counter()
        cache.evict(ids, window)
        host_s[1] += time.perf_counter() - t
        t = time.perf_counter()
        cache.retier(ids)
        host_s[0] += time.perf_counter() - t
        cache.decode(q[i], ids, 0, window=window, out=out)

    for i in range(warmup):
        one(i)
    torch.cuda.synchronize()
    host_s[0] = host_s[1] = 0.0
    cache.kernel_timing(True)
    t0 = time.perf_counter()
    for i in range(warmup, n_steps):
        one(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kt = cache.kernel_times()
    cache.kernel_timing(False)
    st = cache.stats()
    cache.close()
    ms = (t1 - t0) * 1e3 / steps
    return {"steps": steps, "seqs": w.n_seqs, "window": window, "prefill": prefill,
            "ms_per_step": round(ms, 4), "tokens_per_s": round(w.n_seqs / (ms * 1e-3), 1),
            "device_us_per_step": {k: round(v[1] * 1e3 / steps, 3) for k, v in kt.items() if v[0]},
            "host_us_per_call": {"retier": round(host_s[0] * 1e6 / steps, 2), "evict": round(host_s[1] * 1e6 / steps, 2)},
            "pages_in_use": st["pages_used"], "page_bound": (per_seq - 1) * w.n_seqs,
            "pages_retiered": st["pages_retiered"], "pages_evicted": st["pages_evicted"]}


def measured_traffic(kind, workload_name):
    """HBM bytes per launch of this kernel on this workload, from the FETCH_SIZE / WRITE_SIZE
    counter record kept with the profiles (calibrated by a plain copy), or None when there
    is no record or the kernel's sources have changed since it was taken."""
    from bit_ternary_attention_amd import profsum

    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(f"{kind}|{workload_name}")
    if rec is None:
        return None
    srcs = [os.path.join(ROOT, p) for p in rec["sources"]]
    if not all(os.path.exists(p) for p in srcs) or profsum.sources_sha256(srcs) != rec["source_sha256"]:
        return None
    return round(rec["hbm_bytes_per_dispatch"])


def cpu_baseline(w, calls, sample_layers):
    """The CPU oracle, as written, on a bounded sample of the same workload (one thread)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from bit_ternary_attention_amd import workloads as wl
    from oracle import attention as oa
    from oracle import cache as oc
    from oracle import ternary as ot

    spec = oc.CacheSpec(n_kv_heads=w.n_kv_heads, head_dim=w.head_dim, block_size=w.block_size,
                        sink_tokens=w.sink_tokens, sink_format=w.sink_format, recent_tokens=w.recent_tokens,
                        recent_format=w.recent_format)
    # sample: whole layers of whole sequences, about 10-30 s of oracle work
    layers = sample_layers or min(w.n_layers, 36)
    seqs = [0]
    if w.max_len > 8192:
        layers = 1
    total_in = 0.0
    total_bytes = 0.0
    elapsed = 0.0
    n_tok = 0
    passes = 0
    with threadpool_limits(limits=1):
      while passes < 3 and (passes == 0 or elapsed < 10.0):
        passes += 1
        for layer in range(layers):
            q = wl.queries(w, layer, device="cpu")
            for s in seqs:
                L = w.lengths[s]
                # bounded: at most 16384 tokens of a long sequence
                Ls = min(L, 16384)
                kb = wl.to_bits(wl.kv_block(w, "k", layer, s, 0, L, device="cpu")[:Ls])
                vb = wl.to_bits(wl.kv_block(w, "v", layer, s, 0, L, device="cpu")[:Ls])
                scalls = [(t0, min(n, Ls - t0)) for ids, t0, n in calls if s in ids and t0 < Ls]
                qv = ot.values16(wl.to_bits(q[s]), w.dtype)
                t0 = time.perf_counter()
                enc = oc.encode_sequence(spec, kb, vb, w.dtype, scalls)
                pages = [oc.page_tiles(spec, enc, p) for p in range(len(enc.page_format))]
                out = oa.decode_attention(qv, enc.k_hat, enc.v_hat, Ls, w.sink_tokens, w.window)
                elapsed += time.perf_counter() - t0
                stored = sum(p.size for p in pages)
                n_att = len(oa.attended_tokens(Ls, w.sink_tokens, w.window))
                att_bytes = n_att * w.n_kv_heads * 2 * (w.head_dim / 4)
                total_bytes += 2 * kb.nbytes * 2 + stored + att_bytes
                total_in += kb.nbytes * 2
                n_tok += Ls
                del enc, pages, out
    return {"value": round(total_bytes / elapsed / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "seconds": round(elapsed, 2),
            "sample": f"{passes} pass(es) over {layers} layer(s) x seq {seqs} x {n_tok // max(1, layers * passes)} tokens: oracle quantize+pack "
                      f"(every page) + float64 decode attention, algorithmic bytes counted as on the GPU"}


if __name__ == "__main__":
    main()
