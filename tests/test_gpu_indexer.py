"""The top-k indexer (smla_indexer_topk) against the oracle (needs an MI355X).

The selection is integer work decided by floating-point scores: the kernel's
selection must equal the oracle's selection rule applied to the kernel's own
fp32 scores (same precision for the decision), the scores must match the fp64
oracle closely, and the fp64 oracle's selection may differ only at scores
within that tolerance of the threshold."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import sparse_mla_top_amd as smla
import workloads as W
from parity import assert_parity
from workloads.device import upload

pytestmark = pytest.mark.gpu
SCORE_TOL = 2e-5       # relative to the request's largest |score|


def _say(msg):
    print(f"[gpu-test] {msg}", flush=True)


def _run(inp):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    idx, sc = smla.indexer_topk(t(inp.q).view(torch.bfloat16), t(inp.w), t(inp.keys).view(torch.bfloat16),
                                t(inp.page_table), t(inp.ctx_len), pool_pages=inp.pool_pages)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), sc.cpu().numpy()


def _check(inp, what):
    _say(what)
    idx, sc = _run(inp)
    ref_sc, ref_idx = oracle.indexer(inp.q, inp.w, inp.keys, inp.pool_pages, inp.page_table, inp.ctx_len)
    valid = ~np.isnan(ref_sc)
    for b in range(idx.shape[0]):
        v = valid[b]
        scale = max(np.abs(ref_sc[b][v]).max(), 1e-30) if v.any() else 1.0
        err = np.abs(sc[b][v].astype(np.float64) - ref_sc[b][v]).max() if v.any() else 0.0
        assert err <= SCORE_TOL * scale, f"{what}: request {b} score error {err / scale:.2e}"
        n = int(v.sum())
        tail = np.nonzero(~v[:min(int(inp.ctx_len[b]), sc.shape[1])])[0]
        assert np.all(np.isneginf(sc[b][tail])), f"{what}: excluded positions must score -inf"
    # the selection rule applied to the kernel's own scores: identical
    own = np.where(valid, sc.astype(np.float64), np.nan)
    assert np.array_equal(idx, oracle.topk_select(own, inp.pool_pages, inp.page_table, inp.ctx_len)), what
    # against the fp64 selection: differences only at the threshold
    for b in range(idx.shape[0]):
        a, r = set(idx[b][idx[b] >= 0]), set(ref_idx[b][ref_idx[b] >= 0])
        assert len(a) == len(r)
        if a != r:
            v = valid[b]
            scale = np.abs(ref_sc[b][v]).max()
            thr = min(ref_sc[b][list(r)])
            for s in a ^ r:
                assert abs(ref_sc[b][s] - thr) <= 2 * SCORE_TOL * scale, f"{what}: request {b} position {s}"
    return idx, sc


def test_indexer_random():
    inp = W.indexer_inputs(4, [20000, 513, 300, 7000], 11)
    inp.page_table[0, 17] = inp.pool_pages + 9          # invalid page: 64 positions excluded
    inp.page_table[3, 2] = -1
    idx, _ = _check(inp, "indexer random")
    assert np.all(idx[2][300:] == -1) and np.all(idx[2][:300] >= 0)
    assert not np.any((idx[0] >= 17 * 64) & (idx[0] < 18 * 64))


def test_indexer_closed_form_and_ties():
    inp = W.indexer_inputs(2, [3000, 700], 12)
    inp.q[1] = 0                                        # request 1: every score 0 -> first 512 positions
    slot = lambda b, s: int(inp.page_table[b, s // W.PAGE]) * W.PAGE + s % W.PAGE
    for s in (1000, 1500, 2999):                        # exact ties in request 0
        inp.keys[slot(0, s)] = inp.keys[slot(0, 5)]
    idx, sc = _check(inp, "indexer closed form and ties")
    assert list(idx[1]) == list(range(512))
    assert sc[0][5] == sc[0][1000] == sc[0][1500] == sc[0][2999]


def test_indexer_long_context():
    inp = W.indexer_inputs(2, [131072, 65536 + 17], 13)
    _check(inp, "indexer long context")


def test_indexer_feeds_decode():
    """The indexer's output is a valid topk_idx for the decode kernel."""
    inp = W.indexer_inputs(3, [9000, 2000, 400], 14)
    idx, _ = _run(inp)
    w = W.build("from_indexer", 961, 0, 3, list(inp.ctx_len), W.FMT_FP8, "given", topk_idx=idx)
    d = upload(w)
    out, lse = smla.decode(d.q, d.pool, d.page_table, d.topk_idx, d.ctx_len, d.scale, kv_format=d.kv_format,
                           pool_pages=d.pool_pages)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.decode_workload(w)
    assert_parity(out, lse, ref_o, ref_l, "decode over the indexer's selection")


def test_indexer_heavy_ties():
    """Ties at the threshold: the lowest positions win, whether the tied key
    fits the kernel's candidate set or not."""
    inp = W.indexer_inputs(3, [9000, 20000, 20000], 15)
    inp.q[0] = 0                                        # request 0: 9000 equal scores
    ref_sc, _ = oracle.indexer(inp.q, inp.w, inp.keys, inp.pool_pages, inp.page_table, inp.ctx_len)
    slot = lambda b, s: int(inp.page_table[b, s // W.PAGE]) * W.PAGE + s % W.PAGE
    for b, copies in ((1, 6000), (2, 1000)):           # the 301st best key copied onto low scorers
        order = np.argsort(-ref_sc[b][:inp.ctx_len[b]], kind="stable")
        src = int(order[300])
        for s in order[-copies:]:
            inp.keys[slot(b, int(s))] = inp.keys[slot(b, src)]
    idx, sc = _check(inp, "indexer heavy ties")
    assert list(idx[0]) == list(range(512))
    for b in (1, 2):
        t = sc[b][int(np.argsort(-ref_sc[b][:inp.ctx_len[b]], kind="stable")[300])]
        assert (sc[b][idx[b]] >= t).all() and (sc[b][idx[b]] == t).sum() > 100


def test_indexer_long_context_fallbacks():
    """Long contexts where an estimate from a sample of the scores cannot stand:
    every score equal (far too many candidates, then ties by position), almost
    every page invalid (too few valid keys), and invalid pages scattered."""
    inp = W.indexer_inputs(3, [65536, 65536, 40000], 16)
    inp.q[0] = 0
    keep = [3, 200, 511, 700, 1023]
    for p in range(inp.page_table.shape[1]):
        if p not in keep:
            inp.page_table[1, p] = -1
    for p in range(0, 625, 37):
        inp.page_table[2, p] = inp.pool_pages + p
    idx, _ = _check(inp, "indexer long-context fallbacks")
    assert list(idx[0]) == list(range(512))
    got = sorted(int(s) for s in idx[1] if s >= 0)
    assert got == sorted(p * W.PAGE + i for p in keep for i in range(W.PAGE)) and np.all(idx[1][320:] == -1)
    assert not np.any(np.isin(idx[2] // W.PAGE, list(range(0, 625, 37))))
