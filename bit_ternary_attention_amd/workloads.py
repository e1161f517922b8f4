"""Seeded synthetic workloads for the packed ternary KV cache.

This module only draws random numbers and lays them out; it holds none of the
cache's arithmetic (no scale, no quantisation, no attention).  Both the test
oracle and the HIP path are fed from here, so the two see identical inputs.

The five workloads follow the shapes the pages measure on: a tiny GQA cache,
a Qwen2.5-3B-shaped cache (36 layers, 16 query / 2 KV heads, head_dim 128,
4096 tokens; Show HN: Vantage-V-AI, multi-GPU benchmark section, where that
model is run with a 1024-token prompt), a full-retention long-context batch,
a mixed-format paged batch (Minima-KV, "Recent, Anchor and Stale" tiers) and
a 128K-token prefill appended in 4096-token chunks.

Recipe: every (layer, sequence, append-chunk) block of K (or V) is its own
``torch.randn`` draw in float32 from a generator seeded with
``SeedSequence([base, layer, seq, chunk])``, optionally multiplied by 10 on a
seeded set of outlier channels, then rounded to the 16-bit input dtype
(round-to-nearest-even).  Bases: K = 1000+c, V = 2000+c, q = 3000+c,
sequence lengths = 4000+c, outlier channels = 1007, for workload number c.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

FMT_TERNARY2 = 0
FMT_FP8E4M3 = 1
FMT_F16 = 2
FMT_LOSSLESS = 3

DTYPE_F16 = 0
DTYPE_BF16 = 1

_TORCH_DTYPES = {DTYPE_F16: torch.float16, DTYPE_BF16: torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    number: int
    name: str
    n_layers: int
    n_seqs: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: int
    block_size: int
    sink_tokens: int
    window: int                 # recent window in tokens, -1 = whole context
    sink_format: int
    recent_tokens: int          # tokens kept in the recent tier's format (0 = none)
    recent_format: int
    page_shuffle_seed: int
    lengths: Tuple[int, ...]    # final length of every sequence
    chunk_tokens: int           # tokens per append call (0 = whole sequence)
    outlier_frac: float = 0.0
    outlier_mult: float = 10.0
    batch_appends: bool = True  # one append call carries every sequence's chunk
    ragged_appends: bool = False  # sequences of different lengths share one (ragged) append call

    @property
    def gqa(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def max_len(self) -> int:
        return max(self.lengths)

    def appends(self) -> List[Tuple[List[int], int, int]]:
        """The append calls, in order: (sequence ids, first token, n_tokens).

        Sequences of different lengths are appended one call each, since a
        call appends the same number of tokens to every sequence it names.
        """
        calls = []
        if self.batch_appends and len(set(self.lengths)) == 1:
            total = self.lengths[0]
            step = self.chunk_tokens or total
            for t0 in range(0, total, step):
                calls.append((list(range(self.n_seqs)), t0, min(step, total - t0)))
        else:
            for s, total in enumerate(self.lengths):
                step = self.chunk_tokens or total
                for t0 in range(0, total, step):
                    calls.append(([s], t0, min(step, total - t0)))
        return calls


    def append_batches(self) -> List[Tuple[List[int], List[int], List[int]]]:
        """The append calls as issued: (sequence ids, first token of each, token count of each).

        With ragged_appends the k-th append of every sequence goes into one call (vk_append_ragged);
        otherwise each entry of appends() is one call with the same count for every sequence.
        """
        if not self.ragged_appends:
            return [(ids, [t0] * len(ids), [n] * len(ids)) for ids, t0, n in self.appends()]
        per_seq = [[(t0, n) for ids, t0, n in self.appends() if s in ids] for s in range(self.n_seqs)]
        out = []
        for k in range(max(len(c) for c in per_seq)):
            ids = [s for s in range(self.n_seqs) if k < len(per_seq[s])]
            out.append((ids, [per_seq[s][k][0] for s in ids], [per_seq[s][k][1] for s in ids]))
        return out


def _c4_lengths() -> Tuple[int, ...]:
    rng = np.random.Generator(np.random.PCG64(4004))
    return tuple(int(x) for x in rng.integers(1024, 16385, size=64))


def workload(number: int) -> Workload:
    """The five seeded workloads, numbered 1..5, and number 6: head dim 256 at workload 3's page
    bytes (32 sequences of 16384 bfloat16 tokens, 32 query / 8 KV heads, full retention)."""
    if number == 1:
        return Workload(1, "tiny-gqa4-d64-512tok", 1, 1, 8, 2, 64, DTYPE_F16, 512, 4, 256,
                        FMT_TERNARY2, 0, FMT_FP8E4M3, 0, (512,), 0)
    if number == 2:
        return Workload(2, "qwen2.5-3b-shaped-36L-4096tok", 36, 1, 16, 2, 128, DTYPE_BF16, 16, 4, 256,
                        FMT_TERNARY2, 0, FMT_FP8E4M3, 0, (4096,), 0)
    if number == 3:
        return Workload(3, "full-retention-b32-32k-outliers", 1, 32, 32, 8, 128, DTYPE_BF16, 16, 4, -1,
                        FMT_TERNARY2, 0, FMT_FP8E4M3, 0, (32768,) * 32, 0, outlier_frac=0.02)
    if number == 4:
        return Workload(4, "mixed-format-paged-64seq", 1, 64, 64, 8, 128, DTYPE_BF16, 16, 4, -1,
                        FMT_F16, 256, FMT_FP8E4M3, 1004, _c4_lengths(), 0, ragged_appends=True)
    if number == 5:
        return Workload(5, "prefill-128k-b4-chunk4096", 1, 4, 32, 8, 128, DTYPE_BF16, 16, 4, -1,
                        FMT_TERNARY2, 0, FMT_FP8E4M3, 0, (131072,) * 4, 4096)
    if number == 6:
        return Workload(6, "head-dim-256-b32-16k", 1, 32, 32, 8, 256, DTYPE_BF16, 16, 4, -1,
                        FMT_TERNARY2, 0, FMT_FP8E4M3, 0, (16384,) * 32, 0)
    raise ValueError(f"no workload {number}")


def outlier_channels(w: Workload) -> np.ndarray:
    """Flat (kv_head * head_dim + d) indices of the channels scaled as outliers."""
    n = w.n_kv_heads * w.head_dim
    k = int(round(w.outlier_frac * n))
    if k == 0:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.Generator(np.random.PCG64(1007))
    return np.sort(rng.choice(n, size=k, replace=False))


def _seed(base: int, *idx: int) -> int:
    return int(np.random.SeedSequence([base, *idx]).generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def _randn(shape, seed: int, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32, device=device)


def kv_block(w: Workload, which: str, layer: int, seq: int, t0: int, n: int,
             device="cpu") -> torch.Tensor:
    """K or V values of tokens [t0, t0+n) of (layer, seq): shape [n, Hkv, D], input dtype.

    Blocks are drawn per append chunk, so a block must start on a chunk edge
    of the workload's append schedule (tests may ask for any aligned block).
    """
    base = (1000 if which == "k" else 2000) + w.number
    step = w.chunk_tokens or w.lengths[seq]
    if t0 % step != 0:
        raise ValueError("kv_block must start on an append-chunk edge")
    parts = []
    t = t0
    while t < t0 + n:
        ci = t // step
        m = min(step - (t - ci * step), t0 + n - t)
        full = min(step, w.lengths[seq] - ci * step)
        x = _randn((full, w.n_kv_heads, w.head_dim), _seed(base, layer, seq, ci), device)[:m]
        parts.append(x)
        t += m
    x = torch.cat(parts, 0) if len(parts) > 1 else parts[0]
    oc = outlier_channels(w)
    if oc.size:
        flat = x.view(x.shape[0], -1)
        idx = torch.as_tensor(oc, device=x.device)
        flat[:, idx] *= w.outlier_mult
    return x.to(_TORCH_DTYPES[w.dtype])


def append_inputs(w: Workload, seq_ids: Sequence[int], t0: int, n: int, device="cpu"):
    """(K, V) for one append call: [n_layers][n_seqs][n][Hkv][D] each, contiguous."""
    ks, vs = [], []
    for layer in range(w.n_layers):
        ks.append(torch.stack([kv_block(w, "k", layer, s, t0, n, device) for s in seq_ids]))
        vs.append(torch.stack([kv_block(w, "v", layer, s, t0, n, device) for s in seq_ids]))
    return torch.stack(ks).contiguous(), torch.stack(vs).contiguous()


def append_inputs_ragged(w: Workload, seq_ids: Sequence[int], t0s: Sequence[int], ns: Sequence[int], device="cpu"):
    """(K, V) for one ragged append call: [n_layers][sum(ns)][Hkv][D] each, contiguous; within a
    layer, sequence i's tokens [t0s[i], t0s[i] + ns[i]) follow sequence i-1's."""
    ks, vs = [], []
    for layer in range(w.n_layers):
        ks.append(torch.cat([kv_block(w, "k", layer, s, t0, n, device) for s, t0, n in zip(seq_ids, t0s, ns)]))
        vs.append(torch.cat([kv_block(w, "v", layer, s, t0, n, device) for s, t0, n in zip(seq_ids, t0s, ns)]))
    return torch.stack(ks).contiguous(), torch.stack(vs).contiguous()


def queries(w: Workload, layer: int, device="cpu") -> torch.Tensor:
    """One decode query per sequence for ``layer``: [n_seqs][Hq][D], input dtype."""
    x = _randn((w.n_seqs, w.n_q_heads, w.head_dim), _seed(3000 + w.number, layer), device)
    return x.to(_TORCH_DTYPES[w.dtype])


def to_bits(x: torch.Tensor) -> np.ndarray:
    """Raw 16-bit patterns of a float16/bfloat16 tensor, as a host uint16 array."""
    return x.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def small_workload(n_layers=1, n_seqs=None, n_q_heads=8, n_kv_heads=2, head_dim=64,
                   dtype=DTYPE_F16, block_size=16, sink_tokens=4, window=-1,
                   sink_format=FMT_TERNARY2, recent_tokens=0, recent_format=FMT_FP8E4M3,
                   page_shuffle_seed=0, lengths=(64,), chunk_tokens=0, number=9,
                   outlier_frac=0.0, batch_appends=True, ragged_appends=False) -> Workload:
    """A custom small workload for edge-case tests (same generators)."""
    if n_seqs is None:
        n_seqs = len(lengths)
    return Workload(number, "custom", n_layers, n_seqs, n_q_heads, n_kv_heads, head_dim, dtype,
                    block_size, sink_tokens, window, sink_format, recent_tokens, recent_format,
                    page_shuffle_seed, tuple(lengths), chunk_tokens, outlier_frac=outlier_frac,
                    batch_appends=batch_appends, ragged_appends=ragged_appends)
