"""The decode step captured into hipGraphs: confkv_step only enqueues its two
launches (no host synchronisation, no allocation, no memset), so a run of
steps can be captured and replayed. The position is a launch argument, so a
graph covers one run of consecutive positions and is replayed once.

Three graphs of consecutive steps are captured, then replayed in order with
eager work and synchronisations between the replays; after every replay the
outputs, confidences, budgets and the whole cache must be bit-identical to a
twin cache stepped eagerly on the same inputs.
"""

import pytest
import torch

from gpu_lockstep import DEV, log
from kv_cache_eviction_04_amd import confkv, synth

pytestmark = pytest.mark.gpu


def same(a, b, what):
    if a.dtype.is_floating_point:
        a = a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16)
        b = b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16)
    assert torch.equal(a, b), what


@pytest.mark.parametrize("name,over", [("toy", dict(prefill=100)), ("gpt2_small", dict(num_layers=3))])
def test_graph_replays_equal_eager_steps(name, over):
    w = synth.workload(name, **over)
    pk, pv = synth.prefill(w, 0, DEV) if w["prefill"] else (None, None)
    eager = confkv.Cache(w, pk, pv)
    graphed = confkv.Cache(w, pk, pv)
    B, n_graphs, per_graph = w["batch"], 3, 12
    inputs = [synth.step_inputs(w, 0, i, DEV) for i in range(n_graphs * per_graph)]
    outs = [torch.empty_like(x["q"]) for x in inputs]
    confs = [torch.empty(B, dtype=torch.float32, device=DEV) for _ in inputs]
    buds = [torch.empty(B, dtype=torch.int32, device=DEV) for _ in inputs]
    torch.cuda.synchronize()
    graphs = []
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        for g in range(n_graphs):
            cg = torch.cuda.CUDAGraph()
            with torch.cuda.graph(cg, stream=cap):
                for i in range(g * per_graph, (g + 1) * per_graph):
                    x = inputs[i]
                    graphed.step(x["logits"], x["q"], x["k"], x["v"], out=outs[i], conf_out=confs[i],
                                 budget_out=buds[i])
            graphs.append(cg)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    assert graphed.position == eager.position + n_graphs * per_graph
    for g, cg in enumerate(graphs):
        cg.replay()
        out_e, conf_e, bud_e = [], [], []
        for i in range(g * per_graph, (g + 1) * per_graph):  # eager twin, between the replays
            x = inputs[i]
            c = torch.empty(B, dtype=torch.float32, device=DEV)
            bb = torch.empty(B, dtype=torch.int32, device=DEV)
            out_e.append(eager.step(x["logits"], x["q"], x["k"], x["v"], conf_out=c, budget_out=bb))
            conf_e.append(c)
            bud_e.append(bb)
        torch.cuda.synchronize()
        for j, i in enumerate(range(g * per_graph, (g + 1) * per_graph)):
            same(outs[i], out_e[j], f"graph {g} step {i}: output")
            same(confs[i], conf_e[j], f"graph {g} step {i}: confidence")
            same(buds[i], bud_e[j], f"graph {g} step {i}: budget")
        ra, rb = graphed.read_cache(), eager.read_cache()
        for k in ra:
            same(ra[k], rb[k], f"after graph {g}: cache field {k}")
    assert graphed.status() == confkv.OK and eager.status() == confkv.OK
    assert graphed.stats() == eager.stats()
    log(f"{name}: {n_graphs} graphs of {per_graph} steps replayed, bit-identical to eager steps")
