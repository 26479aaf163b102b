"""HIP path vs the fp64 oracle, through the C ABI (needs an MI355X)."""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import sparse_mla_top_amd as smla
import workloads as W
from parity import assert_parity, TOL
from workloads.device import upload

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-test] {msg}", flush=True)


def _run(d, plan=None):
    out, lse = smla.decode(d.q, d.pool, d.page_table, d.topk_idx, d.ctx_len, d.scale,
                           kv_format=d.kv_format, pool_pages=d.pool_pages, plan=plan)
    torch.cuda.synchronize()
    return out, lse


def _check(w, plan=None, what=None):
    what = what or f"{w.name} plan={plan}"
    _say(what)
    pool = w.host_pool()
    d = upload(w)
    out, lse = _run(d, plan)
    ref_o, ref_l = oracle.decode_workload(w, pool=pool)
    return assert_parity(out, lse, ref_o, ref_l, what)


# --------------------------------------------------------------------------- gather
@pytest.mark.parametrize("wid", [1, 2, 3, 4])
def test_gather_bit_exact(wid):
    w = W.make(wid)
    _say(f"gather {w.name}")
    pool = w.host_pool()
    d = upload(w)
    rows, slots = smla.gather_rows(d.pool, d.page_table, d.topk_idx, d.ctx_len, kv_format=d.kv_format,
                                   pool_pages=d.pool_pages)
    torch.cuda.synchronize()
    ref_slots, ref_rows = oracle.gather_workload(w, pool=pool)
    assert np.array_equal(slots.cpu().numpy(), ref_slots)
    assert np.array_equal(rows.cpu().numpy(), ref_rows)


def test_gather_edge_indices():
    B = 4
    rng = np.random.default_rng(8)
    idx = np.stack([rng.integers(-3, 760, W.TOPK) for _ in range(B)]).astype(np.int32)
    w = W.build("edge", 920, 0, B, [700, 64, 3, 200], W.FMT_FP8, "given", topk_idx=idx, max_pages=12)
    w.page_table[0, 3] = w.pool_pages + 5
    w.page_table[3, 1] = -2
    _say("gather edge indices")
    pool = w.host_pool()
    d = upload(w)
    rows, slots = smla.gather_rows(d.pool, d.page_table, d.topk_idx, d.ctx_len, kv_format=d.kv_format,
                                   pool_pages=d.pool_pages)
    torch.cuda.synchronize()
    ref_slots, ref_rows = oracle.gather_workload(w, pool=pool)
    assert np.array_equal(slots.cpu().numpy(), ref_slots)
    assert np.array_equal(rows.cpu().numpy(), ref_rows)


# --------------------------------------------------------------------------- decode
@pytest.mark.parametrize("wid", [1, 2, 3, 4])
def test_decode_workloads(wid):
    _check(W.make(wid))


def test_decode_b1_in_fp8_format():
    _check(W.make(1, kv_format=W.FMT_FP8))


@pytest.mark.parametrize("nsplit", [1, 2, 3, 4, 5, 8, 16])
@pytest.mark.parametrize("fmt", [W.FMT_FP8, W.FMT_BF16])
def test_decode_forced_nsplit(nsplit, fmt):
    w = W.build("nsplit", 930, fmt, 6, [65536, 4096, 700, 513, 300, 131072], fmt, "uniform")
    for merge in (smla.MERGE_IN_KERNEL, smla.MERGE_SEPARATE, smla.MERGE_SPREAD):
        _check(w, plan={"nsplit": nsplit, "merge": merge}, what=f"forced nsplit={nsplit} merge={merge} fmt={fmt}")


@pytest.mark.parametrize("nsplit", [6, 16])
def test_one_tile_splits_under_load(nsplit):
    """Splits holding a single 32-token tile (all of them at 16 splits, the
    last one at 6) read that tile in their first iteration: at B = 96 the row
    loads are slow enough that a missing wait for them shows."""
    w = W.make(4)
    for merge in (smla.MERGE_IN_KERNEL, smla.MERGE_SEPARATE):
        _check(w, plan={"nsplit": nsplit, "merge": merge}, what=f"one-tile splits nsplit={nsplit} merge={merge}")


def test_nsplit_results_agree():
    w = W.build("agree", 931, 0, 5, [65536, 4096, 700, 300, 131072], W.FMT_FP8, "uniform")
    d = upload(w)
    outs = [(_run(d, ns)) for ns in (1, 2, 4, 8, 16)]
    o0 = outs[0][0].float()
    for o, l in outs[1:]:
        denom = o0.abs().amax(dim=-1).clamp_min(1e-30)
        assert ((o.float() - o0).abs().amax(dim=-1) / denom).max().item() <= 2 * TOL


@pytest.mark.parametrize("fmt", [W.FMT_FP8, W.FMT_BF16])
def test_sweep_sampled_layers(fmt):
    """512K-context sweep workload: sampled layers at B = 96 and prefixes."""
    for layer in (0, 41):
        w = W.make(5, layer=layer, kv_format=fmt)
        _check(w, what=f"sweep layer {layer} B=96 fmt={fmt}")
        for b in (1, 8, 33):
            _check(w.subset(b), what=f"sweep layer {layer} B={b} fmt={fmt}")


def test_masked_and_degenerate_requests():
    idx = np.full((6, W.TOPK), -1, np.int32)
    rng = np.random.default_rng(12)
    idx[1, 100] = 7                                   # single valid token
    idx[2] = rng.permutation(W.TOPK).astype(np.int32) # dense ctx = 512
    idx[3, ::2] = rng.choice(5000, 256, replace=False)
    idx[3, 1::2] = 5000 + rng.integers(0, 100, 256)   # >= ctx -> masked
    idx[4] = rng.integers(0, 50, W.TOPK)              # duplicates (count per slot)
    idx[5, 480:] = rng.choice(3000, 32, replace=False)  # only the last tile valid
    w = W.build("degenerate", 940, 0, 6, [1000, 8, 512, 5000, 50, 3000], W.FMT_FP8, "given", topk_idx=idx)
    for ns in (1, 4, 16):
        _check(w, plan=ns, what=f"degenerate nsplit={ns}")
    # splits that hold no valid slot at all (lse -inf) under every merge placement
    for merge in (smla.MERGE_IN_KERNEL, smla.MERGE_SEPARATE, smla.MERGE_SPREAD):
        _check(w, plan={"nsplit": 16, "merge": merge}, what=f"degenerate nsplit=16 merge={merge}")


def test_q_zero_and_single_token_closed_forms():
    w = W.build("q0", 941, 0, 3, [4096, 100, 600], W.FMT_FP8, "uniform", q_zero=True)
    _check(w, plan=4, what="q=0")


@pytest.mark.parametrize("fmt", [W.FMT_FP8, W.FMT_BF16])
def test_page_table_longer_than_the_staged_part(fmt):
    """1.5M-token contexts: the page-table row (23,438 entries) is longer than
    the part the kernel stages in LDS, so tokens on the last pages are looked up
    in global memory instead."""
    w = W.build("longpt", 944, fmt, 3, [1_500_000, 1_499_000, 700], fmt, "uniform", compact=True)
    assert w.max_pages > 22272
    for ns in (1, 3):
        _check(w, plan=ns, what=f"page table longer than staged, nsplit={ns} fmt={fmt}")


def test_invalid_page_ids_are_masked():
    w = W.build("badpages", 942, 0, 3, [3000, 3000, 3000], W.FMT_FP8, "uniform")
    w.page_table[0, :10] = -5
    w.page_table[1, 5:20] = w.pool_pages + 100
    _check(w, plan=2, what="invalid page ids")


def test_validate_mode(monkeypatch):
    """SMLA_VALIDATE=1: inputs the kernels would silently mask (an index other
    than -1 outside [0, ctx_len), a page id outside the pool) are reported as
    SMLA_ERR_INDEX before any launch, outputs untouched; -1 padding and valid
    inputs pass and give the same bits as without the check."""
    monkeypatch.setenv("SMLA_VALIDATE", "1")
    w = W.build("validate", 944, 0, 3, [3000, 300, 5000], W.FMT_FP8, "uniform")   # request 1: -1 padding
    d = upload(w)
    shape = smla.make_shape(w.B, d.kv_format, d.page_table.shape[1], d.pool_pages)
    ok_out, ok_lse = _run(d, plan=2)
    monkeypatch.delenv("SMLA_VALIDATE")
    ref_out, ref_lse = _run(d, plan=2)
    assert torch.equal(ok_out, ref_out) and torch.equal(ok_lse, ref_lse)
    monkeypatch.setenv("SMLA_VALIDATE", "1")
    smla.gather_rows(d.pool, d.page_table, d.topk_idx, d.ctx_len, kv_format=d.kv_format, pool_pages=d.pool_pages)
    idx0, pt0 = w.topk_idx.copy(), w.page_table.copy()
    bad_cases = []
    for what, edit in (("index -2", lambda i, p: i.__setitem__((0, 7), -2)),
                       ("index = ctx_len", lambda i, p: i.__setitem__((2, 100), w.ctx_len[2])),
                       ("page id = pool_pages", lambda i, p: p.__setitem__((0, int(i[0, 3]) // W.PAGE), w.pool_pages)),
                       ("page id -1", lambda i, p: p.__setitem__((2, int(i[2, 0]) // W.PAGE), -1))):
        i, p = idx0.copy(), pt0.copy()
        edit(i, p)
        bad_cases.append((what, i, p))
    for what, i, p in bad_cases:
        _say(f"validate mode: {what}")
        topk = torch.from_numpy(i).cuda()
        pt = torch.from_numpy(p).cuda()
        out = torch.full((w.B, 64, 512), 7, dtype=torch.bfloat16, device="cuda")
        lse = torch.full((w.B, 64), 7, dtype=torch.float32, device="cuda")
        for plan in (1, 2):
            ws = smla.new_workspace(smla.plan_for(shape, plan)[1] + 256)
            rc = smla.decode_raw(d.q, d.pool, pt, topk, d.ctx_len, d.scale, out, lse, shape, plan, ws)
            assert rc == smla.ERR_INDEX, (what, plan, rc)
        with pytest.raises(smla.SmlaError):
            smla.gather_rows(d.pool, pt, topk, d.ctx_len, kv_format=d.kv_format, pool_pages=d.pool_pages)
        torch.cuda.synchronize()
        assert torch.all(out == 7) and torch.all(lse == 7), what      # nothing launched
        monkeypatch.delenv("SMLA_VALIDATE")                            # without the check: masked, no error
        _run(dataclasses.replace(d, topk_idx=topk, page_table=pt), plan=2)
        monkeypatch.setenv("SMLA_VALIDATE", "1")


def test_permutation_invariance_on_gpu():
    w = W.make(2)
    d = upload(w)
    out0, lse0 = _run(d)
    rng = np.random.default_rng(1)
    perm = np.stack([rng.permutation(W.TOPK) for _ in range(w.B)])
    d.topk_idx = torch.from_numpy(np.take_along_axis(w.topk_idx, perm, axis=1)).cuda()
    out1, lse1 = _run(d)
    denom = out0.float().abs().amax(dim=-1)
    assert ((out1.float() - out0.float()).abs().amax(dim=-1) / denom).max().item() <= 2 * TOL
    assert (lse1 - lse0).abs().max().item() <= 2 * TOL


def test_deterministic_rerun():
    w = W.make(3)
    d = upload(w)
    a = _run(d)
    b = _run(d)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_empty_batch_and_errors():
    w = W.build("err", 943, 0, 2, [3000, 3000], W.FMT_FP8, "uniform")
    d = upload(w)
    shape = smla.make_shape(2, d.kv_format, d.page_table.shape[1], d.pool_pages)
    out = torch.full((2, 64, 512), 7, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((2, 64), 7, dtype=torch.float32, device="cuda")
    plan, ws = smla.plan_for(shape, 4)
    assert ws > 0
    small = torch.empty(ws - 256, dtype=torch.uint8, device="cuda")
    rc = smla.decode_raw(d.q, d.pool, d.page_table, d.topk_idx, d.ctx_len, d.scale, out, lse, shape, 4, small)
    assert rc == smla.ERR_WORKSPACE
    rc = smla.decode_raw(d.q, d.pool, d.page_table, d.topk_idx, d.ctx_len, d.scale, out, lse, shape, 4, None)
    assert rc == smla.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 7) and torch.all(lse == 7)      # outputs untouched on error
    empty = smla.make_shape(0, d.kv_format, d.page_table.shape[1], d.pool_pages)
    rc = smla.decode_raw(d.q, d.pool, d.page_table, d.topk_idx, d.ctx_len, d.scale, out, lse, empty)
    assert rc == smla.OK


def test_split_and_combine_stages_equal_decode():
    """In-kernel merge, separate-launch merge, the spread merge (where the grid
    fits the device) and the two stages called one by one give identical bits
    (same weights, same split-ordered sums)."""
    w = W.make(2)
    d = upload(w)
    shape = smla.make_shape(w.B, d.kv_format, d.page_table.shape[1], d.pool_pages)
    for ns in (1, 3, 4, 16):
        plan, ws_bytes = smla.plan_for(shape, ns)
        ws = smla.new_workspace(ws_bytes)
        res = []
        merges = (smla.MERGE_IN_KERNEL, smla.MERGE_SEPARATE) + ((smla.MERGE_SPREAD,) if ns in (3, 4) else ())
        for merge in merges:
            o = torch.empty((w.B, 64, 512), dtype=torch.bfloat16, device="cuda")
            l = torch.empty((w.B, 64), dtype=torch.float32, device="cuda")
            pl = {"nsplit": ns, "merge": merge}
            assert smla.decode_raw(d.q, d.pool, d.page_table, d.topk_idx, d.ctx_len, d.scale, o, l, shape, pl, ws) == 0
            res.append((o, l))
        o2, l2 = torch.empty_like(res[0][0]), torch.empty_like(res[0][1])
        assert smla.split_raw(d.q, d.pool, d.page_table, d.topk_idx, d.ctx_len, d.scale, o2, l2, shape, ns, ws) == 0
        assert smla.combine_raw(shape, ns, ws, o2, l2) == 0
        torch.cuda.synchronize()
        res.append((o2, l2))
        for o, l in res[1:]:
            assert torch.equal(res[0][0], o) and torch.equal(res[0][1], l), f"nsplit={ns}"
        if ns == 4:
            ref_o, ref_l = oracle.decode_workload(w)
            assert_parity(res[1][0], res[1][1], ref_o, ref_l, "separate merge nsplit=4")


def test_fused_merge_repeated_calls_share_workspace():
    """One workspace reused across calls, plans and batch sizes: the arrival
    counters must come back to zero after every call."""
    ws = smla.new_workspace(80 << 20)
    for it, (wid, ns) in enumerate([(2, 4), (2, 4), (3, 3), (2, 16), (4, 6), (2, 4)]):
        w = W.make(wid)
        pool = w.host_pool()
        d = upload(w)
        out, lse = smla.decode(d.q, d.pool, d.page_table, d.topk_idx, d.ctx_len, d.scale, kv_format=d.kv_format,
                               pool_pages=d.pool_pages, plan={"nsplit": ns, "merge": smla.MERGE_IN_KERNEL},
                               workspace=ws)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle.decode_workload(w, pool=pool)
        assert_parity(out, lse, ref_o, ref_l, f"fused merge call {it} {w.name} nsplit={ns}")


def test_spread_merge_repeated_calls_share_workspace():
    """The spread merge and the last-split merge take turns on one workspace,
    across plans and batch sizes: each call leaves its counters at zero."""
    ws = smla.new_workspace(80 << 20)
    spread, fused = smla.MERGE_SPREAD, smla.MERGE_IN_KERNEL
    for it, (wid, ns, merge) in enumerate([(2, 4, spread), (2, 4, spread), (2, 4, fused), (1, 16, spread),
                                           (2, 3, spread), (1, 8, fused), (1, 8, spread), (2, 4, spread)]):
        w = W.make(wid)
        pool = w.host_pool()
        d = upload(w)
        out, lse = smla.decode(d.q, d.pool, d.page_table, d.topk_idx, d.ctx_len, d.scale, kv_format=d.kv_format,
                               pool_pages=d.pool_pages, plan={"nsplit": ns, "merge": merge}, workspace=ws)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle.decode_workload(w, pool=pool)
        assert_parity(out, lse, ref_o, ref_l, f"merge {merge} call {it} {w.name} nsplit={ns}")


def test_workspace_init_recovers_dirty_counters():
    w = W.make(2)
    d = upload(w)
    shape = smla.make_shape(w.B, d.kv_format, d.page_table.shape[1], d.pool_pages)
    plan, ws_bytes = smla.plan_for(shape, 4)
    ws = torch.full((ws_bytes,), 0x5A, dtype=torch.uint8, device="cuda")   # garbage everywhere
    smla.workspace_init(ws)
    out, lse = smla.decode(d.q, d.pool, d.page_table, d.topk_idx, d.ctx_len, d.scale, kv_format=d.kv_format,
                           pool_pages=d.pool_pages, plan={"nsplit": 4, "merge": smla.MERGE_IN_KERNEL}, workspace=ws)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.decode_workload(w)
    assert_parity(out, lse, ref_o, ref_l, "after workspace_init")


# --------------------------------------------------------------- several query tokens per request
def _mtp_workload(q_len, fmt=W.FMT_FP8):
    base = W.build("mtp", 950, fmt, 5, [65536, 4096, 700, 300, 131072], fmt, "uniform")
    return W.with_query_tokens(base, q_len)


@pytest.mark.parametrize("q_len", [2, 3, 4])
def test_query_tokens_share_selection(q_len):
    w = _mtp_workload(q_len)
    _check(w, what=f"q_len={q_len} auto plan")
    for ns in (1, 2, 5):
        merges = (smla.MERGE_IN_KERNEL, smla.MERGE_SEPARATE, smla.MERGE_SPREAD) if ns > 1 else (smla.MERGE_AUTO,)
        for merge in merges:
            _check(w, plan={"nsplit": ns, "merge": merge}, what=f"q_len={q_len} nsplit={ns} merge={merge}")


def test_query_tokens_bf16_rows():
    w = W.with_query_tokens(W.make(1), 4)
    for ns in (1, 4):
        _check(w, plan=ns, what=f"q_len=4 bf16 nsplit={ns}")


def test_query_tokens_equal_single_token_calls():
    """Each query token's rows are computed exactly as in a single-token call
    with the same plan (bit-identical), and the two-stage form matches too."""
    w = _mtp_workload(3)
    d = upload(w)
    for ns in (1, 3):
        plan = {"nsplit": ns, "merge": smla.MERGE_IN_KERNEL}
        out, lse = _run(d, plan)
        for t in range(3):
            o1, l1 = smla.decode(d.q[:, t].contiguous(), d.pool, d.page_table, d.topk_idx, d.ctx_len, d.scale,
                                 kv_format=d.kv_format, pool_pages=d.pool_pages, plan=plan)
            torch.cuda.synchronize()
            assert torch.equal(o1, out[:, t]) and torch.equal(l1, lse[:, t]), f"nsplit={ns} token {t}"
    shape = smla.make_shape(w.B, d.kv_format, d.page_table.shape[1], d.pool_pages, 3)
    plan, ws_bytes = smla.plan_for(shape, 4)
    ws = smla.new_workspace(ws_bytes)
    o_a = torch.empty((w.B, 3, 64, 512), dtype=torch.bfloat16, device="cuda")
    l_a = torch.empty((w.B, 3, 64), dtype=torch.float32, device="cuda")
    o_b, l_b = torch.empty_like(o_a), torch.empty_like(l_a)
    assert smla.decode_raw(d.q, d.pool, d.page_table, d.topk_idx, d.ctx_len, d.scale, o_a, l_a, shape,
                           {"nsplit": 4, "merge": smla.MERGE_IN_KERNEL}, ws) == 0
    assert smla.split_raw(d.q, d.pool, d.page_table, d.topk_idx, d.ctx_len, d.scale, o_b, l_b, shape, 4, ws) == 0
    assert smla.combine_raw(shape, 4, ws, o_b, l_b) == 0
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(l_a, l_b)


def test_query_tokens_masked_and_degenerate():
    idx = np.full((4, W.TOPK), -1, np.int32)
    rng = np.random.default_rng(13)
    idx[1, 7] = 3                                      # one valid token
    idx[2] = rng.permutation(W.TOPK).astype(np.int32)  # dense ctx = 512
    idx[3, 480:] = rng.choice(3000, 32, replace=False) # only the last tile valid
    base = W.build("mtp_degenerate", 951, 0, 4, [1000, 8, 512, 3000], W.FMT_FP8, "given", topk_idx=idx)
    w = W.with_query_tokens(base, 2)
    for ns in (1, 4, 16):
        _check(w, plan=ns, what=f"q_len=2 degenerate nsplit={ns}")


# --------------------------------------------------------------- large batches
def test_large_batch_several_dispatch_rounds():
    """600 requests: 1200 workgroups unsplit (several dispatch rounds on 256
    CUs) and 2400 with two splits merged in-kernel (600 sets of counters)."""
    w = W.build("large", 953, 0, 600, [600 + 37 * (b % 50) for b in range(600)], W.FMT_FP8, "uniform")
    for plan in (None, {"nsplit": 1}, {"nsplit": 2, "merge": smla.MERGE_IN_KERNEL}):
        _check(w, plan=plan, what=f"B=600 plan={plan}")


def test_query_sets_beyond_the_in_kernel_merge_limit():
    """1030 requests x 4 query tokens = 4120 query sets, past the 4096 the
    arrival-counter head holds: a split plan merges with the combine launch,
    and forcing the in-kernel merge is refused."""
    base = W.build("qsets", 954, 0, 1030, [520] * 1030, W.FMT_FP8, "uniform")
    w = W.with_query_tokens(base, 4)
    d = upload(w)
    shape = smla.make_shape(w.B, d.kv_format, d.page_table.shape[1], d.pool_pages, 4)
    p, _ = smla.plan_for(shape, {"nsplit": 2})
    assert p.merge == smla.MERGE_SEPARATE
    with pytest.raises(smla.SmlaError):
        smla.plan_for(shape, {"nsplit": 2, "merge": smla.MERGE_IN_KERNEL})
    _check(w, plan={"nsplit": 2}, what="4120 query sets, nsplit 2")


# --------------------------------------------------------------- a dominant token: live rescale and lse spread
def _dominant_workload(fmt, shared=1.5, seed=960):
    """Three requests in which the token at top-k slot 300 + 17b (tile 9 or 10 of
    16) scores about 30 nats above every other selected token, for every head:
    all heads' q share a component `shared * u` on the 512 latent dims (u a
    fixed +-1 pattern) and that token's latent is u with zero rope.  Unsplit,
    the running maximum then jumps after nine tiles have been accumulated (the
    rescale of live accumulators); split, one split's lse lies ~25 nats above
    the others'.  Rows and Q are built here from the generator's own encoders."""
    B = 3
    w = W.build("dominant", seed, fmt, B, [8192, 20000, 4096], fmt, "uniform")
    rng = np.random.default_rng(seed)
    u = rng.choice([-1.0, 1.0], size=W.D_LATENT).astype(np.float32)
    qf = torch.from_numpy(w.q.view(np.int16)).view(torch.bfloat16).float().numpy()
    qf[:, :, :W.D_LATENT] += np.float32(shared) * u
    w.q = W.bf16_bits(qf)
    planted = W.pack_rows(fmt, u[None, :], np.zeros((1, W.D_ROPE), np.float32))[0]
    slots = []
    for b in range(B):
        i = int(w.topk_idx[b, 300 + 17 * b])
        slot = int(w.page_table[b, i // W.PAGE]) * W.PAGE + i % W.PAGE
        k = int(np.searchsorted(w.row_slots, slot))
        assert w.row_slots[k] == slot
        w.row_data[k] = planted
        slots.append(slot)
    return w


@pytest.mark.parametrize("fmt", [W.FMT_FP8, W.FMT_BF16])
def test_dominant_late_token_rescales_live_accumulators(fmt):
    """Unsplit (nsplit = 1) and one tile per split (nsplit = 16): the oracle's
    lse sits ~30 nats up, set by the planted token, and the kernel must match."""
    w = _dominant_workload(fmt)
    ref_o, ref_l = oracle.decode_workload(w)
    assert ref_l.min() > 20.0, ref_l.min()          # the planted token dominates every head
    for ns, merge in ((1, smla.MERGE_AUTO), (16, smla.MERGE_IN_KERNEL), (16, smla.MERGE_SPREAD)):
        _check(w, plan={"nsplit": ns, "merge": merge}, what=f"dominant late token nsplit={ns} merge={merge} fmt={fmt}")


@pytest.mark.parametrize("fmt", [W.FMT_FP8, W.FMT_BF16])
def test_merge_of_splits_with_far_apart_lse(fmt):
    """The dominant token sits in one split, so that split's lse is ~25 nats above
    the others' and their weights underflow to ~1e-11: every merge placement must
    give the oracle's result."""
    w = _dominant_workload(fmt)
    for ns in (2, 4, 16):
        for merge in (smla.MERGE_IN_KERNEL, smla.MERGE_SEPARATE, smla.MERGE_SPREAD):
            _check(w, plan={"nsplit": ns, "merge": merge}, what=f"far-apart lse nsplit={ns} merge={merge} fmt={fmt}")
