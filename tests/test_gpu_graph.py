"""Decode calls captured in a HIP graph (a layer loop replayed as one step) give
the eager results on every replay (needs an MI355X)."""
from __future__ import annotations

import pytest
import torch

import oracle
import sparse_mla_top_amd as smla
import workloads as W
from parity import assert_parity
from workloads.device import upload

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-test] {msg}", flush=True)


@pytest.mark.parametrize("plan", [{"nsplit": 1}, {"nsplit": 4, "merge": smla.MERGE_IN_KERNEL},
                                  {"nsplit": 3, "merge": smla.MERGE_SEPARATE}, {"nsplit": 8, "merge": smla.MERGE_SPREAD}],
                         ids=["ns1", "ns4_fused", "ns3_sep", "ns8_spread"])
def test_graph_replay_equals_eager(plan):
    """Every replay gives the eager bits, and the first replay of every layer
    matches the oracle (the layer loop of one decode step as one graph)."""
    _say(f"graph replay plan={plan}")
    layers = 6
    ws_list, per = [], None
    sets, pool, hosts = [], None, []
    for l in range(layers):
        w = W.make(2, layer=l, page_base=0 if per is None else l * per).subset(8)
        if per is None:
            per = W.make(2, layer=0).pool_pages
            pool = torch.empty(per * layers * W.PAGE * w.row_bytes, dtype=torch.uint8, device="cuda")
        sets.append(upload(w, pool=pool))
        hosts.append(w)
    B = 8
    shape = smla.make_shape(B, sets[0].kv_format, sets[0].page_table.shape[1], per * layers)
    _, ws_bytes = smla.plan_for(shape, plan)
    ws = smla.new_workspace(ws_bytes)
    outs = [torch.empty((B, 64, 512), dtype=torch.bfloat16, device="cuda") for _ in range(layers)]
    lses = [torch.empty((B, 64), dtype=torch.float32, device="cuda") for _ in range(layers)]

    def step():
        for l, d in enumerate(sets):
            rc = smla.decode_raw(d.q, d.pool, d.page_table, d.topk_idx, d.ctx_len, d.scale, outs[l], lses[l],
                                 shape, plan, ws)
            assert rc == 0

    step()
    torch.cuda.synchronize()
    eager = [(o.clone(), l.clone()) for o, l in zip(outs, lses)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step()                                   # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    for rep in range(4):
        for o, l in zip(outs, lses):
            o.fill_(7)
            l.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, ((eo, el), o, l) in enumerate(zip(eager, outs, lses)):
            assert torch.equal(o, eo) and torch.equal(l, el), f"replay {rep} layer {i}"
            if rep == 0:
                ref_o, ref_l = oracle.decode_workload(hosts[i])
                assert_parity(o, l, ref_o, ref_l, f"graph replay plan={plan} layer {i}")
        step()                                   # eager work between replays
        torch.cuda.synchronize()
