"""Benchmark: quantize+pack into the packed ternary KV cache, then decode attention over it.

One step is one pass of the whole hot path over one batch of synthetic input:
every append call of the workload (absmean pass, then quantise + pack + page
scatter, whose waves derive each segment's gamma) followed by one decode step of
every layer.  The default
workload is the full-retention long-context batch (32 sequences of 32768 bf16
tokens, 32 query / 8 KV heads, head_dim 128, 2% outlier channels, every token
attended): the largest workload that is bandwidth-bound on one GPU.  Other
workloads are selectable with --workload.

Prints one JSON line.  `value` is the decode attention's rate: the algorithmic
bytes of one decode step (the attended pages in their stored formats, their
gammas, the queries and the outputs) divided by the device time of the step's
decode launches (decode + split merge), from HIP event pairs around each
launch on the launch stream, over the timed steps.  The quantize+pack
rate (algorithmic bytes of the write side over the device time of its two
kernels) stands beside it, with a roofline for the decode kernel, the pack
kernel and the absmean kernel.  Inputs are resident in HBM before the timed
region; several input sets rotate when one set would fit in the 256 MB
Infinity Cache.
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
FORMATS = {"ternary": 0, "fp8": 1, "f16": 2, "lossless": 3}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", type=int, default=3, help="1..5 (default 3: full retention, 32 x 32K tokens); 6: head dim 256, 32 x 16K tokens")
    ap.add_argument("--decode-kernel", type=int, default=0, help="0 default, 1 vector ALU, 2 matrix cores")
    ap.add_argument("--sink-format", choices=sorted(FORMATS), default=None,
                    help="page format of the sink pages instead of the workload's own (lossless: the exact "
                         "bfloat16 tier)")
    ap.add_argument("--recent-format", choices=sorted(FORMATS), default=None,
                    help="page format of the recent tier instead of the workload's own")
    ap.add_argument("--fp8-dynamic", action="store_true",
                    help="FP8 pages with one scale per token and KV head instead of the static scale")
    ap.add_argument("--page-order", choices=["workload", "sequential", "shuffled"], default="workload",
                    help="page placement in the pools: the workload's own, in allocation order, or a seeded "
                         "random permutation")
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
    if args.sink_format or args.recent_format:
        import dataclasses
        w = dataclasses.replace(w, sink_format=FORMATS[args.sink_format] if args.sink_format else w.sink_format,
                                recent_format=FORMATS[args.recent_format] if args.recent_format else w.recent_format)
    if args.page_order != "workload":
        import dataclasses
        w = dataclasses.replace(w, page_shuffle_seed=0 if args.page_order == "sequential" else 12345)
    calls = w.appends()
    ids_all = list(range(w.n_seqs))

    # format of every page of every sequence (the cache's format rule, decided by the append
    # call that first writes the page), and the pages per format one step needs
    cfg = vk.make_config(n_layers=w.n_layers, n_kv_heads=w.n_kv_heads, n_q_heads=w.n_q_heads,
                         head_dim=w.head_dim, block_size=w.block_size, max_seqs=w.n_seqs,
                         max_tokens_per_seq=w.max_len, sink_tokens=w.sink_tokens, sink_format=w.sink_format,
                         recent_tokens=w.recent_tokens, recent_format=w.recent_format,
                         page_shuffle_seed=w.page_shuffle_seed, decode_kernel=args.decode_kernel,
                         fp8_dynamic=int(args.fp8_dynamic))
    formats = page_formats(w, calls)
    need = [sum(f.count(x) for f in formats) for x in range(4)]
    cfg.pages_ternary, cfg.pages_fp8, cfg.pages_f16, cfg.pages_lossless = need
    cache = vk.Cache(cfg)

    # inputs resident in HBM: rotate enough sets to exceed the 256 MB Infinity Cache
    batches = w.append_batches()
    in_bytes = sum(2 * w.n_layers * sum(ns) * w.n_kv_heads * w.head_dim * 2 for _, _, ns in batches)
    n_sets = max(1, min(3, -(-768 * 2 ** 20 // in_bytes)))
    sets = []
    for r in range(n_sets):
        per_call = []
        for ids, t0s, ns in batches:
            if w.ragged_appends:
                k, v = wl.append_inputs_ragged(w, ids, t0s, ns, device="cuda")
                ax = 1
            else:
                k, v = wl.append_inputs(w, ids, t0s[0], ns[0], device="cuda")
                ax = 2
            if r:  # other sets: same shapes, different draws
                k = k.index_select(ax, torch.randperm(k.shape[ax], device="cuda")).contiguous()
                v = v.index_select(ax, torch.randperm(v.shape[ax], device="cuda")).contiguous()
            per_call.append((ids, ns, k, v))
        sets.append(per_call)
    qs = [wl.queries(w, layer, device="cuda") for layer in range(w.n_layers)]
    outs = [torch.empty(q.shape, dtype=torch.float32, device="cuda") for q in qs]
    torch.cuda.synchronize()

    def step(i, seg=None):
        cache.reset(ids_all)
        for ids, ns, k, v in sets[i % n_sets]:
            if w.ragged_appends:
                cache.append_ragged(k, v, ids, ns)
            else:
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

    # The timed steps.  Inside them: the library's per-kernel HIP event pairs on the launch
    # stream (torch's current stream), and one more event pair per step around the step's
    # decode launches, whose elapsed time is the decode attention's device time.
    segs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    cache.kernel_timing(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, segs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    kt = cache.kernel_times()
    cache.kernel_timing(False)
    decode_seg_ms = sum(a.elapsed_time(b) for a, b in segs) / args.steps
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
    write_bytes = sum(kt[k][2] for k in ("absmean", "finalize", "pack")) / args.steps
    write_ms = sum(kt[k][1] for k in ("absmean", "finalize", "pack")) / args.steps
    dec_bytes = decode_step_bytes(w, formats, args.fp8_dynamic)
    # device time of the decode attention: its decode and merge launches (event pairs around
    # each); the segment events around the step's decode launches also hold the gaps the
    # per-launch events open between them
    dec_ms = sum(kt[k][1] for k in ("decode", "merge")) / args.steps
    dec_gbps = dec_bytes / (dec_ms * 1e-3) / 1e9
    kv_tokens = sum(len(ids) * n for ids, _, n in calls)
    att_tokens = sum(attended_tokens(L, w.sink_tokens, w.window) for L in w.lengths) * w.n_layers

    def roofline(kind):
        k = kernels[kind]
        small = k["bytes_per_launch"] < 64 * 2 ** 20
        return {"bound": "hbm", "kernel": kind, "achieved": k["GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": k["hbm_frac"], "traffic": measured_traffic(kind, w.name),
                "bytes_per_launch": k["bytes_per_launch"], "avg_launch_us": k["avg_us"],
                "launches_per_step": k["launches_per_step"],
                "timing": "HIP event pair around each launch on the launch stream, over the timed steps",
                **({"regime": "latency-bound: one launch moves too few bytes to fill the GPU"} if small else {})}

    result = {
        "metric": METRIC,
        "value": round(dec_gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16 in; 2-bit codes (4 per u8); scores fp4 codes x two e4m3 query terms (head dims 128 "
                  "and 256, bf16 queries; f16 operands otherwise), P*V f16-operand MFMA; f32 accumulate and softmax"),
        "dtype_detail": ("write side: 16-bit inputs, float64 absmean sums, codes by integer thresholds equal to "
                         "float32 RoundClip(x / (gamma + eps)); decode: ternary key codes as e2m1 operands against "
                         "the bf16 query held exactly as two e4m3 terms (scaled MFMA, head dims 128 and 256), other keys, "
                         "the values and f16 queries as f16 operands, probabilities as f16 (scaled by 2^14), "
                         "f32 scores, softmax state and accumulation"),
        "data": "synthetic (seeded torch.randn, see bit_ternary_attention_amd/workloads.py)",
        "config": {"workload": w.name, "layers": w.n_layers, "seqs": w.n_seqs,
                   "tokens_per_seq": list(sorted(set(w.lengths))) if len(set(w.lengths)) > 1 else w.lengths[0],
                   "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size, "sink_tokens": w.sink_tokens, "window": w.window,
                   "page_order": "shuffled" if w.page_shuffle_seed else "sequential",
                   "append_calls": len(batches), "ragged_appends": w.ragged_appends, "input_sets": n_sets,
                   "fp8": "dynamic per (token, head)" if args.fp8_dynamic else "static scale",
                   "sink_format": next(k for k, f in FORMATS.items() if f == w.sink_format),
                   "recent_format": (next(k for k, f in FORMATS.items() if f == w.recent_format)
                                     if w.recent_tokens > 0 else None)},
        "decode_attn": {"GBps": round(dec_gbps, 1), "hbm_frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
                        "bytes_per_step": dec_bytes, "device_us_per_step": round(dec_ms * 1e3, 3),
                        "us_per_layer": round(dec_ms * 1e3 / w.n_layers, 3),
                        "kv_tokens_per_s": round(att_tokens / (dec_ms * 1e-3), 1),
                        "decode_steps_per_s": round(w.n_seqs / (dec_ms * 1e-3), 1),
                        "segment_us_per_step": round(decode_seg_ms * 1e3, 3),
                        "segment_GBps": round(dec_bytes / (decode_seg_ms * 1e-3) / 1e9, 1),
                        "splits": stats["last_decode_splits"], "units_by_format": stats["last_decode_units"],
                        "ordered_dispatch": bool(stats["last_decode_ordered"]),
                        "timing": ("decode + merge launches, HIP event pair around each on the launch stream, "
                                   "over the timed steps; segment_*: one event pair per step around the step's "
                                   "decode launches"),
                        "kernel": {0: "default (matrix cores)", 1: "vector ALU", 2: "matrix cores"}[args.decode_kernel]},
        "quantize_pack": {"GBps": round(write_bytes / (write_ms * 1e-3) / 1e9, 1),
                          "hbm_frac": round(write_bytes / (write_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                          "bytes_per_step": write_bytes, "device_us_per_step": round(write_ms * 1e3, 3),
                          "kv_tokens_per_s": round(kv_tokens * w.n_layers / (write_ms * 1e-3), 1),
                          "timing": "sum of the absmean and pack launches' event pairs"},
        "step_GBps": round((dec_bytes + write_bytes) / (ms_step * 1e-3) / 1e9, 1),
        "kernels": kernels,
        "roofline": {**roofline("decode"), "counters": measured_counters("decode", w.name)},
        "roofline_pack": roofline("pack"),
        "roofline_absmean": roofline("absmean"),
    }

    result["decode_step"] = decode_step_leg(cache, qs, outs, w, ids_all)
    if stats["pages_used"][3] > 0:
        result["lossless_tier"] = lossless_bytes(cache, w, ids_all)

    if w.recent_tokens > 0 and w.recent_format == vk.FMT_FP8E4M3:
        cache.close()
        result["retier"] = retier_leg(w, args.steps, args.warmup, args.fp8_dynamic)
        result["stream"] = stream_leg(w, args.steps, args.warmup, fp8_dynamic=args.fp8_dynamic)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, calls, args.cpu_sample_layers, args.fp8_dynamic)
    print(json.dumps(result), flush=True)
    cache.close()


def page_formats(w, calls):
    """Format of every page of every sequence: the cache's rule, applied by the append call that
    first writes the page (sink pages, pages meeting the last recent_tokens tokens of that call's
    end, else ternary)."""
    bs = w.block_size
    out = []
    for s in range(w.n_seqs):
        fm = []
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
                    f = 0
                fm.append(f)
        out.append(fm)
    return out


def decode_step_bytes(w, formats, fp8_dynamic=False):
    """Algorithmic bytes of one decode step of every layer: per attended token and KV head the
    key and value in their stored format (ternary D/4 bytes each, fp8 D (+4 B of scale when
    dynamic), fp16 2D, lossless 1.5 D + 1 (its two coded streams and a 16-byte header per 16
    tokens; exceptions not counted)), a gamma pair (8 B) per attended ternary page, the queries
    (16-bit) and the float32 outputs."""
    D, hkv, bs = w.head_dim, w.n_kv_heads, w.block_size
    per_tok = {0: 2 * D / 4, 1: 2 * (D + (4 if fp8_dynamic else 0)), 2: 2 * 2 * D, 3: 2 * (1.5 * D + 1)}
    import numpy as np
    total = 0.0
    for s, L in enumerate(w.lengths):
        fm = np.asarray(formats[s])
        lo = np.arange(fm.size) * bs
        hi = np.minimum(lo + bs, L)
        if w.window < 0:
            n_att = hi - lo
        else:   # tokens of the page in [0, min(S, L)) or [max(S, L - W), L): each counted once
            a = min(w.sink_tokens, L)
            b = max(a, L - w.window)
            n_att = np.clip(np.minimum(hi, a) - lo, 0, None) + np.clip(hi - np.maximum(lo, b), 0, None)
        for f, per in per_tok.items():
            total += per * hkv * float(n_att[fm == f].sum())
        total += 8 * int(np.count_nonzero((fm == 0) & (n_att > 0)))
    total += w.n_seqs * w.n_q_heads * D * (2 + 4)
    return total * w.n_layers


def lossless_bytes(cache, w, ids):
    """Bytes a decode reads from the lossless pages of layer 0 (each 16-token group's header, its
    two coded streams and its exceptions, or its raw values) against their bfloat16 size, read
    back from the device after the timed steps."""
    import numpy as np
    slot = 32 * w.head_dim + 16
    read = raw = groups = raw_groups = 0
    for s in ids:
        n = -(-cache.seq_length(s) // w.block_size)
        buf, fmt, _ = cache.read_pages(0, s, 0, n)
        for p in np.nonzero(fmt == 3)[0]:
            hdr = buf[p, :2 * w.n_kv_heads * (w.block_size // 16) * slot].reshape(-1, slot)[:, :8]
            for h in hdr:
                groups += 1
                if h[1] == 1:
                    raw_groups += 1
                    read += 16 + 32 * w.head_dim
                else:
                    read += 16 + 24 * w.head_dim + int(h[4:8].view("<u4")[0])
                raw += 32 * w.head_dim
    return {"groups": groups, "raw_groups": raw_groups, "bytes_read": read, "bf16_bytes": raw,
            "bf16_over_read": round(raw / read, 4) if read else None,
            "note": "every 16-token group of every lossless page of layer 0, including units past a "
                    "sequence's end inside its last page"}


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
    cfg.pages_lossless = n_sink * w.n_seqs if w.sink_format == vk.FMT_LOSSLESS else 0
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
    cfg.pages_lossless = n_sink * w.n_seqs if w.sink_format == vk.FMT_LOSSLESS else 0
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


def measured_counters(kind, workload_name):
    """Hardware counters of this kernel on this workload (VALU busy, matrix-core busy, LDS bank
    conflicts, L2 hits and misses, instructions per attended 16-token unit), from the record kept
    with the profiles, or None when there is none or the kernel's sources have changed since."""
    from bit_ternary_attention_amd import profsum

    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(f"{kind}|{workload_name}")
    if rec is None:
        return None
    srcs = [os.path.join(ROOT, p) for p in rec["sources"]]
    if not all(os.path.exists(p) for p in srcs) or profsum.sources_sha256(srcs) != rec["source_sha256"]:
        return None
    c = rec["counters"]
    keep = ("VALUBusy", "VALUUtilization", "MfmaUtil", "LDSBankConflict")
    out = {k: c[k] for k in keep if k in c}
    if "TCC_HIT_sum" in c and "TCC_MISS_sum" in c:
        out["L2_hit_rate"] = round(c["TCC_HIT_sum"] / max(1.0, c["TCC_HIT_sum"] + c["TCC_MISS_sum"]), 4)
    out["per_unit"] = rec["per_unit"]
    out["source"] = "profiles/counters.json (rocprofv3 --pmc, one run per counter set)"
    return out


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


def cpu_baseline(w, calls, sample_layers, fp8_dynamic=False):
    """The CPU oracle, as written, on a bounded sample of the same workload, on one thread.

    The oracle's decode attention (float64 softmax attention over its dequantised pages) gives
    `value`, in the unit of the GPU's `value`: the sample's algorithmic decode bytes (counted
    as on the GPU) per second.  Its write side (absmean, codes and every page's bytes) is
    reported beside it as quantize+pack GB/s.
    """
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from bit_ternary_attention_amd import workloads as wl
    from oracle import attention as oa
    from oracle import cache as oc
    from oracle import ternary as ot

    spec = oc.CacheSpec(n_kv_heads=w.n_kv_heads, head_dim=w.head_dim, block_size=w.block_size,
                        sink_tokens=w.sink_tokens, sink_format=w.sink_format, recent_tokens=w.recent_tokens,
                        recent_format=w.recent_format, fp8_dynamic=bool(fp8_dynamic))
    blas_default = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    # sample: whole layers of sequence 0, at most 16384 tokens of it, about 10-30 s of oracle work
    layers = sample_layers or min(w.n_layers, 36)
    if w.max_len > 8192:
        layers = 1
    dec_s = enc_s = dec_bytes = enc_bytes = 0.0
    n_tok = passes = 0
    with threadpool_limits(limits=1):
        while passes < 3 and (passes == 0 or dec_s + enc_s < 10.0):
            passes += 1
            for layer in range(layers):
                q = wl.queries(w, layer, device="cpu")
                L = w.lengths[0]
                Ls = min(L, 16384)
                kb = wl.to_bits(wl.kv_block(w, "k", layer, 0, 0, L, device="cpu")[:Ls])
                vb = wl.to_bits(wl.kv_block(w, "v", layer, 0, 0, L, device="cpu")[:Ls])
                scalls = [(t0, min(n, Ls - t0)) for ids, t0, n in calls if 0 in ids and t0 < Ls]
                qv = ot.values16(wl.to_bits(q[0]), w.dtype)
                t0 = time.perf_counter()
                enc = oc.encode_sequence(spec, kb, vb, w.dtype, scalls)
                pages = [oc.page_tiles(spec, enc, p) for p in range(len(enc.page_format))]
                t1 = time.perf_counter()
                oa.decode_attention(qv, enc.k_hat, enc.v_hat, Ls, w.sink_tokens, w.window)
                t2 = time.perf_counter()
                enc_s += t1 - t0
                dec_s += t2 - t1
                enc_bytes += 2 * (kb.nbytes + vb.nbytes) + sum(p.size for p in pages)
                idx = oa.attended_tokens(Ls, w.sink_tokens, w.window)
                fmt = enc.token_format[idx]
                per_tok = {0: 2 * w.head_dim / 4, 1: 2 * (w.head_dim + (4 if fp8_dynamic else 0)), 2: 4 * w.head_dim,
                           3: 2 * (1.5 * w.head_dim + 1)}
                dec_bytes += sum(per_tok[f] * w.n_kv_heads * int(np.count_nonzero(fmt == f)) for f in per_tok)
                dec_bytes += 8 * len(set(int(t) // w.block_size for t in idx[fmt == 0]))
                dec_bytes += w.n_q_heads * w.head_dim * (2 + 4)
                n_tok += Ls
                del enc, pages
    return {"value": round(dec_bytes / dec_s / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "seconds": round(dec_s + enc_s, 2),
            "quantize_pack_GBps": round(enc_bytes / enc_s / 1e9, 4),
            "decode_seconds": round(dec_s, 3), "quantize_pack_seconds": round(enc_s, 3),
            "host_cpu_count": os.cpu_count(), "blas_threads_default": blas_default, "blas_threads_used": 1,
            "sample": f"{passes} pass(es) over {layers} layer(s) x sequence 0 x {n_tok // max(1, layers * passes)} "
                      f"tokens: oracle decode attention in float64 (value) and oracle quantize+pack with every "
                      f"page's bytes (quantize_pack_GBps), algorithmic bytes counted as on the GPU, one thread"}


if __name__ == "__main__":
    main()
