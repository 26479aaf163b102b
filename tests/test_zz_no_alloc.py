"""sparse_mla_decode_noalloc (workspace in the library's own device array) gives
the bits of sparse_mla_decode with a caller's workspace, and the oracle's
result, on two calls in a row, the second with a smaller input; a plan whose
workspace exceeds the array is refused before any launch (needs an MI355X)."""
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


def _both(w, plan):
    d = upload(w)
    shape = smla.make_shape(w.B, d.kv_format, d.page_table.shape[1], d.pool_pages, w.q_len)
    lead = (w.B, w.q_len) if w.q_len > 1 else (w.B,)
    o_ref = torch.empty(lead + (64, 512), dtype=torch.bfloat16, device="cuda")
    l_ref = torch.empty(lead + (64,), dtype=torch.float32, device="cuda")
    o_na, l_na = torch.full_like(o_ref, 7), torch.full_like(l_ref, 7)
    _, ws_bytes = smla.plan_for(shape, plan)
    ws = smla.new_workspace(ws_bytes)
    assert smla.decode_raw(d.q, d.pool, d.page_table, d.topk_idx, d.ctx_len, d.scale, o_ref, l_ref, shape, plan,
                           ws) == smla.OK
    assert smla.decode_noalloc_raw(d.q, d.pool, d.page_table, d.topk_idx, d.ctx_len, d.scale, o_na, l_na, shape,
                                   plan) == smla.OK
    torch.cuda.synchronize()
    return o_ref, l_ref, o_na, l_na


@pytest.mark.parametrize("plan", [{"nsplit": 4, "merge": smla.MERGE_IN_KERNEL},
                                  {"nsplit": 3, "merge": smla.MERGE_SEPARATE}, None],
                         ids=["ns4_in_kernel", "ns3_separate", "auto"])
def test_noalloc_equals_workspace_entry_on_shrinking_inputs(plan):
    big = W.build("noalloc_big", 970, 0, 12, [65536] * 6 + [4096, 700, 300, 513, 131072, 20000], W.FMT_FP8,
                  "uniform")
    small = W.build("noalloc_small", 971, 0, 3, [3000, 200, 40000], W.FMT_FP8, "uniform")
    for w in (big, small):
        _say(f"noalloc {w.name} B={w.B} plan={plan}")
        o_ref, l_ref, o_na, l_na = _both(w, plan)
        assert torch.equal(o_ref, o_na) and torch.equal(l_ref, l_na), f"{w.name} plan={plan}"
        ref_o, ref_l = oracle.decode_workload(w)
        assert_parity(o_na, l_na, ref_o, ref_l, f"noalloc {w.name} plan={plan}")


def test_noalloc_several_query_tokens_and_bf16_rows():
    w = W.with_query_tokens(W.build("noalloc_mtp", 972, 0, 4, [8192, 300, 65536, 1000], W.FMT_BF16, "uniform"), 2)
    plan = {"nsplit": 5, "merge": smla.MERGE_IN_KERNEL}
    o_ref, l_ref, o_na, l_na = _both(w, plan)
    assert torch.equal(o_ref, o_na) and torch.equal(l_ref, l_na)


def test_noalloc_refuses_a_plan_beyond_its_array():
    """20 requests x 16 splits need 40 MiB of partials, more than the 32 MiB
    array: SMLA_ERR_WORKSPACE, outputs untouched."""
    w = W.build("noalloc_over", 973, 0, 20, [2048] * 20, W.FMT_FP8, "uniform")
    d = upload(w)
    shape = smla.make_shape(w.B, d.kv_format, d.page_table.shape[1], d.pool_pages)
    plan = {"nsplit": 16, "merge": smla.MERGE_SEPARATE}
    assert smla.plan_for(shape, plan)[1] > smla.NOALLOC_SCRATCH_BYTES
    out = torch.full((w.B, 64, 512), 7, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((w.B, 64), 7, dtype=torch.float32, device="cuda")
    rc = smla.decode_noalloc_raw(d.q, d.pool, d.page_table, d.topk_idx, d.ctx_len, d.scale, out, lse, shape, plan)
    torch.cuda.synchronize()
    assert rc == smla.ERR_WORKSPACE
    assert torch.all(out == 7) and torch.all(lse == 7)
