"""The in-kernel split merge's give-up path (needs an MI355X).

The merging workgroup polls a bounded number of times for the other splits'
partials; the environment variable SMLA_MERGE_SPIN_LIMIT lowers that bound,
here to zero, so the give-up happens from the host side with every kernel still
running to completion.  A give-up sets the workspace's status word: lse is NaN
for that call and every later in-kernel merge on the workspace, validate mode
turns the word into SMLA_ERR_MERGE, the separate combine launch (which uses no
counters) is unaffected, and smla_workspace_init restores normal operation."""
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


def test_merge_give_up_marks_the_workspace_until_init(monkeypatch):
    w = W.build("merge_status", 990, 0, 5, [65536, 3000, 300, 131072, 20000], W.FMT_FP8, "uniform")
    d = upload(w)
    shape = smla.make_shape(w.B, d.kv_format, d.page_table.shape[1], d.pool_pages)
    fused = {"nsplit": 4, "merge": smla.MERGE_IN_KERNEL}
    separate = {"nsplit": 4, "merge": smla.MERGE_SEPARATE}
    _, ws_bytes = smla.plan_for(shape, fused)
    ws = smla.new_workspace(ws_bytes)
    out = torch.empty((w.B, 64, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, 64), dtype=torch.float32, device="cuda")
    ref_o, ref_l = oracle.decode_workload(w)

    def call(plan):
        rc = smla.decode_raw(d.q, d.pool, d.page_table, d.topk_idx, d.ctx_len, d.scale, out, lse, shape, plan, ws)
        torch.cuda.synchronize()
        return rc

    monkeypatch.delenv("SMLA_VALIDATE", raising=False)
    _say("merge status: healthy workspace")
    assert call(fused) == smla.OK
    assert_parity(out, lse, ref_o, ref_l, "before the give-up")

    _say("merge status: spin limit 0 (every merge gives up)")
    monkeypatch.setenv("SMLA_MERGE_SPIN_LIMIT", "0")
    assert call(fused) == smla.OK
    assert torch.isnan(lse).all(), "a merge that gave up must leave NaN in lse"
    monkeypatch.delenv("SMLA_MERGE_SPIN_LIMIT")

    _say("merge status: sticky after the limit is lifted")
    out.fill_(3)
    lse.fill_(3)
    assert call(fused) == smla.OK
    assert torch.isnan(lse).all(), "the status word must keep later in-kernel merges at NaN"
    assert (out == 3).all(), "a marked workspace leaves out as it was"

    _say("merge status: validate mode reports it")
    monkeypatch.setenv("SMLA_VALIDATE", "1")
    assert call(fused) == smla.ERR_MERGE
    monkeypatch.delenv("SMLA_VALIDATE")

    _say("merge status: the separate combine ignores the counters")
    assert call(separate) == smla.OK
    assert_parity(out, lse, ref_o, ref_l, "separate combine on a marked workspace")

    _say("merge status: smla_workspace_init clears it")
    smla.workspace_init(ws)
    monkeypatch.setenv("SMLA_VALIDATE", "1")
    assert call(fused) == smla.OK
    assert_parity(out, lse, ref_o, ref_l, "after smla_workspace_init")
    assert call(fused) == smla.OK                # counters left at zero again
    assert_parity(out, lse, ref_o, ref_l, "second call after smla_workspace_init")


def test_spread_merge_give_up_marks_the_workspace_until_init(monkeypatch):
    """The spread merge (every split waits for the others, then merges a share):
    a give-up writes NaN into the share of out and into lse, and sets the same
    status word, with the same later behaviour."""
    w = W.build("merge_status_spread", 991, 0, 5, [65536, 3000, 300, 131072, 20000], W.FMT_FP8, "uniform")
    d = upload(w)
    shape = smla.make_shape(w.B, d.kv_format, d.page_table.shape[1], d.pool_pages)
    spread = {"nsplit": 4, "merge": smla.MERGE_SPREAD}
    _, ws_bytes = smla.plan_for(shape, spread)
    ws = smla.new_workspace(ws_bytes)
    out = torch.empty((w.B, 64, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, 64), dtype=torch.float32, device="cuda")
    ref_o, ref_l = oracle.decode_workload(w)

    def call(plan):
        rc = smla.decode_raw(d.q, d.pool, d.page_table, d.topk_idx, d.ctx_len, d.scale, out, lse, shape, plan, ws)
        torch.cuda.synchronize()
        return rc

    monkeypatch.delenv("SMLA_VALIDATE", raising=False)
    _say("spread merge status: healthy workspace")
    assert call(spread) == smla.OK
    assert_parity(out, lse, ref_o, ref_l, "spread merge before the give-up")

    _say("spread merge status: spin limit 0 (every split gives up)")
    monkeypatch.setenv("SMLA_MERGE_SPIN_LIMIT", "0")
    assert call(spread) == smla.OK
    assert torch.isnan(lse).all(), "a give-up must leave NaN in lse"
    assert torch.isnan(out.float()).all(), "a give-up must leave NaN in its share of out"
    monkeypatch.delenv("SMLA_MERGE_SPIN_LIMIT")

    _say("spread merge status: sticky, reported in validate mode")
    out.fill_(3)
    lse.fill_(3)
    assert call(spread) == smla.OK
    assert torch.isnan(lse).all() and (out == 3).all()
    monkeypatch.setenv("SMLA_VALIDATE", "1")
    assert call(spread) == smla.ERR_MERGE
    monkeypatch.delenv("SMLA_VALIDATE")

    _say("spread merge status: smla_workspace_init clears it")
    smla.workspace_init(ws)
    monkeypatch.setenv("SMLA_VALIDATE", "1")
    for k in range(2):
        assert call(spread) == smla.OK
        assert_parity(out, lse, ref_o, ref_l, f"spread merge call {k} after smla_workspace_init")
