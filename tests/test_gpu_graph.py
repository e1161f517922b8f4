"""Decode steps captured into a HIP graph and replayed.

vk_decode_attn only enqueues kernel launches on its stream, so a serving loop can capture
a decode step (one call per layer) once and replay it while the sequences keep their
lengths.  Every replay, with eager work and synchronisations between replays, must give
the eager step's outputs bit for bit (the default decode path repeats exactly), and the
outputs must match the oracle.
"""
import pytest
import torch

from bit_ternary_attention_amd import workloads as wl
from oracle import cache as oc

from gpu_harness import check_decode, fill, host_kv, make_cache, say, seq_calls, spec_of

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

GRAPH_CASES = [
    # (name, workload kwargs, window): mixed tiers (an fp8 / fp16 block and a merge launch)
    # and an all-ternary cache whose decode writes its output directly
    ("mixed-tiers", dict(n_layers=3, n_q_heads=8, n_kv_heads=2, head_dim=128, dtype=1, sink_format=oc.F16,
                         recent_tokens=48, recent_format=oc.FP8E4M3, lengths=(700, 95), batch_appends=False), -1),
    ("ternary-window", dict(n_layers=4, n_q_heads=16, n_kv_heads=2, head_dim=128, dtype=1,
                            lengths=(4096,)), 256),
]


@pytest.mark.parametrize("name,kw,W", GRAPH_CASES, ids=[c[0] for c in GRAPH_CASES])
def test_decode_step_graph_replays_match_eager(name, kw, W):
    w = wl.small_workload(**kw)
    say(f"graph {name}: {w}")
    cache = make_cache(w, decode_kernel=2)
    fill(cache, w)
    ids = list(range(w.n_seqs))
    qs = [wl.queries(w, layer, device="cuda") for layer in range(w.n_layers)]
    outs = [torch.empty(q.shape, dtype=torch.float32, device="cuda") for q in qs]

    def step():
        for layer in range(w.n_layers):
            cache.decode(qs[layer], ids, layer, window=W, out=outs[layer])

    step()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    for layer in (0, w.n_layers - 1):
        encs = {}
        for s in ids:
            kb, vb = host_kv(w, layer, s)
            encs[s] = oc.encode_sequence(spec_of(w), kb, vb, w.dtype, seq_calls(w, s))
        check_decode(want[layer], qs[layer], w, encs, W)

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for layer in range(w.n_layers):
            assert torch.equal(outs[layer], want[layer]), (name, rep, layer)
        # eager work between replays: another decode step and an unrelated kernel
        step()
        torch.sum(torch.ones(1 << 20, device="cuda")).item()
        torch.cuda.synchronize()
    say(f"graph {name}: 4 replays equal the eager step")
    cache.close()
