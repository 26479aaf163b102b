"""Host-side checks of libsparse_mla.so that need no GPU: exports, validation, selector."""
from __future__ import annotations

import ctypes
import json
import math
import os
import re

import pytest

import sparse_mla_top_amd as smla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_mla.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert {"sparse_mla_decode", "smla_plan_for", "smla_gather_rows", "smla_strerror"} <= set(names)
    L = smla.lib()
    for n in names:
        assert hasattr(L, n), f"{n} declared in sparse_mla.h but not exported"


def test_version_and_row_bytes():
    L = smla.lib()
    assert L.smla_version() >= 100
    assert L.smla_row_bytes(smla.KV_BF16) == 1152
    assert L.smla_row_bytes(smla.KV_FP8) == 656
    assert L.smla_row_bytes(7) == -1
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -99):
        assert smla.strerror(code)
    # every error code has its own message, and the binding's constants are the header's
    assert len({smla.strerror(c) for c in (-1, -2, -3, -4, -5, -6, -7)}) == 7
    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "sparse_mla.h")).read()
    for name in ("INVALID_ARG", "UNSUPPORTED_SHAPE", "WORKSPACE", "PLAN", "HIP", "INDEX"):
        m = re.search(r"#define SMLA_ERR_%s \((-\d+)\)" % name, hdr)
        assert m and int(m.group(1)) == getattr(smla, "ERR_" + name), name


def _shape(**kw):
    s = smla.make_shape(kw.pop("batch", 8), kw.pop("kv_format", smla.KV_FP8), kw.pop("max_pages", 16),
                        kw.pop("pool_pages", 1024))
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def _decode_rc(shape, nonnull=True, scale=1 / 24):
    # pointers are never dereferenced on these paths: validation fails first
    p = ctypes.c_void_p(16) if nonnull else None
    return smla.lib().sparse_mla_decode(p, p, p, p, p, scale, p, p, ctypes.byref(shape), None, None, 0, None)


@pytest.mark.parametrize("field,value,code", [
    ("num_heads", 32, smla.ERR_UNSUPPORTED_SHAPE), ("d_qk", 512, smla.ERR_UNSUPPORTED_SHAPE),
    ("d_v", 576, smla.ERR_UNSUPPORTED_SHAPE), ("topk", 2048, smla.ERR_UNSUPPORTED_SHAPE),
    ("page_size", 16, smla.ERR_UNSUPPORTED_SHAPE), ("batch", -1, smla.ERR_INVALID_ARG),
    ("max_pages_per_req", 0, smla.ERR_INVALID_ARG), ("pool_pages", 0, smla.ERR_INVALID_ARG),
    ("kv_format", 5, smla.ERR_INVALID_ARG), ("q_len", 5, smla.ERR_UNSUPPORTED_SHAPE),
    ("q_len", -1, smla.ERR_INVALID_ARG),
])
def test_shape_validation(field, value, code):
    assert _decode_rc(_shape(**{field: value})) == code


def test_null_pointers_and_bad_scale():
    assert _decode_rc(_shape(), nonnull=False) == smla.ERR_INVALID_ARG
    assert _decode_rc(_shape(), scale=float("nan")) == smla.ERR_INVALID_ARG
    assert smla.lib().sparse_mla_decode(None, None, None, None, None, 1.0, None, None, None, None, None, 0,
                                        None) == smla.ERR_INVALID_ARG


def test_plan_overrides_validated():
    s = _shape()
    for bad in ({"nsplit": 17}, {"nsplit": -1}, {"tile_tokens": 16}, {"heads_per_wg": 64}, {"wg_per_cu": 3},
                {"merge": 4}, {"merge": -1}):
        with pytest.raises(smla.SmlaError) as e:
            smla.plan_for_cus(s, 256, bad)
        assert e.value.code == smla.ERR_PLAN


@pytest.mark.parametrize("forced,expect", [(1, 1), (2, 2), (3, 3), (5, 4), (6, 6), (7, 6), (9, 8), (16, 16)])
def test_forced_nsplit_normalised_to_whole_tiles(forced, expect):
    # splits hold whole 32-token tiles: 16 tiles in chunks of ceil(16/n), no empty split
    p, ws = smla.plan_for_cus(_shape(batch=8), 256, forced)
    assert p.nsplit == expect
    chunk = math.ceil(16 / p.nsplit)
    assert (p.nsplit - 1) * chunk < 16 <= p.nsplit * chunk
    a256 = lambda x: (x + 255) // 256 * 256
    # a fixed head (64 KiB of arrival counters, a 256-byte status block), then
    # partial outputs and partial lse
    assert ws == (0 if expect == 1 else 65536 + 256 + a256(8 * expect * 64 * 512 * 4) + a256(8 * expect * 64 * 4))


def test_selector_is_shape_only_and_bounded():
    for B in (1, 8, 16, 32, 48, 64, 80, 88, 96, 300):
        p, ws = smla.plan_for_cus(_shape(batch=B), 256)
        assert 1 <= p.nsplit <= 16
        # a merge placement exactly when there is something to merge
        assert (p.merge in (smla.MERGE_IN_KERNEL, smla.MERGE_SEPARATE, smla.MERGE_SPREAD)) == (p.nsplit > 1)
        if p.merge == smla.MERGE_SPREAD:   # only when the whole grid is resident at once
            assert B * 2 * p.nsplit <= 256
        p2, ws2 = smla.plan_for_cus(_shape(batch=B), 256)
        assert p.as_dict() == p2.as_dict() and ws == ws2
    # with many requests the grid already fills the device: no split needed
    p, _ = smla.plan_for_cus(_shape(batch=2048), 256)
    assert p.nsplit == 1


def test_selector_fills_compute_units_at_small_batch():
    # at B=1 a single workgroup would idle 255 of 256 CUs
    p, _ = smla.plan_for_cus(_shape(batch=1), 256)
    assert p.nsplit >= 2
    # fewer splits per request as the batch grows
    ns = [smla.plan_for_cus(_shape(batch=B), 256)[0].nsplit for B in (1, 8, 32, 80, 256, 1024)]
    assert ns == sorted(ns, reverse=True), ns


# ---------------------------------------------------------------- pages' grid arithmetic
GOLDEN = os.path.join(ROOT, "tests", "golden", "pages_grid_arithmetic.json")


def pages_nsplit(B: int) -> int:
    """The NSPLIT rule the pages quote for their sm120 Triton kernel."""
    return min(16, math.ceil(256 / (B * 2)))


def dispatch_rounds(grid: int, slots: int) -> float:
    return grid / slots


def test_pages_worked_grid_numbers():
    g = json.load(open(GOLDEN))
    for case in g["nsplit_rule"]:
        B = case["B"]
        grid = B * 2 * pages_nsplit(B)
        assert grid == case["ctas"], case
        if "rounds" in case:
            assert round(dispatch_rounds(grid, g["sm_count"]), 2) == case["rounds"], case
        if "first_round" in case:
            assert min(grid, g["sm_count"]) == case["first_round"]
            assert grid - g["sm_count"] == case["second_round"]
    old = g["unsplit_grid"]
    assert old["B"] * old["H"] == old["blocks"]
    assert round(old["blocks"] / old["sms"], 2) == old["occupancy"]
    sk = g["split_k_target"]
    assert sk["B"] * sk["H"] * sk["nsplit"] == sk["blocks"]


@pytest.mark.parametrize("merge", [1, 2, 3])
def test_forced_merge_placement_is_kept(merge):
    p, ws = smla.plan_for_cus(_shape(batch=8), 256, {"nsplit": 4, "merge": merge})
    assert (p.nsplit, p.merge) == (4, merge)
    # nothing to merge with one split
    p, ws = smla.plan_for_cus(_shape(batch=8), 256, {"nsplit": 1, "merge": merge})
    assert (p.nsplit, p.merge, ws) == (1, 0, 0)


def test_query_tokens_scale_the_workspace_and_grid():
    """q_len query tokens per request: partials and counters per (request,
    token); q_len = 0 reads as 1; the selector sees q_len times the workgroups."""
    for ns in (2, 4):
        ws = {}
        for q in (0, 1, 2, 3, 4):
            s = _shape(batch=6, q_len=q)
            _, ws[q] = smla.plan_for_cus(s, 256, {"nsplit": ns})
        assert ws[0] == ws[1]
        a256 = lambda x: (x + 255) // 256 * 256
        for q in (1, 2, 3, 4):
            Q = 6 * q
            assert ws[q] == 65536 + 256 + a256(Q * ns * 64 * 512 * 4) + a256(Q * ns * 64 * 4)
    # more query tokens never ask for more splits (the grid already fills more of the device)
    for B in (1, 4, 16, 32):
        picks = [smla.plan_for_cus(_shape(batch=B, q_len=q), 256)[0].nsplit for q in (1, 2, 3, 4)]
        assert picks == sorted(picks, reverse=True), (B, picks)


def test_kv_append_validation():
    L = smla.lib()
    p = ctypes.c_void_p(16)
    s = _shape()
    assert L.smla_kv_append(p, p, p, p, p, p, -1, ctypes.byref(s), None) == smla.ERR_INVALID_ARG
    assert L.smla_kv_append(None, None, None, None, None, None, 0, ctypes.byref(s), None) == smla.OK   # nothing to do
    assert L.smla_kv_append(None, p, p, p, p, p, 4, ctypes.byref(s), None) == smla.ERR_INVALID_ARG
    assert L.smla_kv_append(ctypes.c_void_p(20), p, p, p, p, p, 4, ctypes.byref(s), None) == smla.ERR_INVALID_ARG
    assert L.smla_kv_append(p, p, p, p, p, p, 4, ctypes.byref(_shape(num_heads=8)), None) == smla.ERR_UNSUPPORTED_SHAPE
    assert L.smla_kv_append(p, p, p, p, p, p, 4, None, None) == smla.ERR_INVALID_ARG


def test_in_kernel_merge_limited_to_counter_head():
    """The arrival counters live in a fixed 64 KiB head (4096 query sets x two
    head groups x two counters), so the in-kernel merge is never chosen beyond
    4096 query sets and forcing it there is a plan error."""
    p, ws = smla.plan_for_cus(_shape(batch=4096), 256, {"nsplit": 2, "merge": smla.MERGE_IN_KERNEL})
    assert (p.nsplit, p.merge) == (2, smla.MERGE_IN_KERNEL)
    for B, q in ((4097, 1), (1025, 4)):
        p, _ = smla.plan_for_cus(_shape(batch=B, q_len=q), 256, {"nsplit": 2})
        assert p.merge == smla.MERGE_SEPARATE
        with pytest.raises(smla.SmlaError):
            smla.plan_for_cus(_shape(batch=B, q_len=q), 256, {"nsplit": 2, "merge": smla.MERGE_IN_KERNEL})


def test_spread_merge_needs_a_resident_grid():
    """The spread merge has every split wait for its request's other splits, so
    a plan takes it only while the whole grid (query sets x 2 head groups x
    nsplit workgroups, one per compute unit) fits the device at once; forcing
    it beyond that, or beyond the counter head's 4096 query sets, is refused."""
    spread = smla.MERGE_SPREAD
    p, ws = smla.plan_for_cus(_shape(batch=8), 256, {"nsplit": 16, "merge": spread})   # 256 workgroups
    assert (p.nsplit, p.merge) == (16, spread) and ws > 0
    for B, q, ns, cus in ((9, 1, 16, 256), (8, 1, 16, 255), (33, 1, 4, 256), (5, 4, 8, 256), (4097, 1, 2, 20000)):
        with pytest.raises(smla.SmlaError) as e:
            smla.plan_for_cus(_shape(batch=B, q_len=q), cus, {"nsplit": ns, "merge": spread})
        assert e.value.code == smla.ERR_PLAN
    # the automatic choice keeps the grid within half the device, whatever its size
    for cus in (32, 120, 256, 304):
        for B in range(1, 129, 3):
            for q in (1, 2):
                p, _ = smla.plan_for_cus(_shape(batch=B, q_len=q), cus)
                if p.merge == spread:
                    assert B * q * 2 * p.nsplit <= cus // 2, (cus, B, q, p.as_dict())


def test_read_rows_validation():
    """smla_read_rows rejects bad arguments before touching the device."""
    L = smla.lib()
    p = ctypes.c_void_p(256)
    rr = L.smla_read_rows
    assert rr(None, 100, p, 10, 10, 656, 1, p, None) == smla.ERR_INVALID_ARG
    assert rr(p, 100, None, 10, 10, 656, 1, p, None) == smla.ERR_INVALID_ARG
    assert rr(p, 100, p, 10, 10, 656, 1, None, None) == smla.ERR_INVALID_ARG
    assert rr(p, -1, p, 10, 10, 656, 1, p, None) == smla.ERR_INVALID_ARG
    assert rr(p, 0, p, 10, 10, 656, 1, p, None) == smla.ERR_INVALID_ARG       # empty pool
    assert rr(p, 100, p, 10, 4097, 656, 1, p, None) == smla.ERR_INVALID_ARG   # group beyond the staged offsets
    assert rr(p, 100, p, -1, 10, 656, 1, p, None) == smla.ERR_INVALID_ARG
    assert rr(p, 100, p, 10, 0, 656, 1, p, None) == smla.ERR_INVALID_ARG
    assert rr(p, 100, p, 10, 10, 640, 1, p, None) == smla.ERR_INVALID_ARG     # not a row size of this library
    assert rr(ctypes.c_void_p(264), 100, p, 10, 10, 656, 1, p, None) == smla.ERR_INVALID_ARG   # pool unaligned
    assert rr(p, 100, ctypes.c_void_p(260), 10, 10, 656, 1, p, None) == smla.ERR_INVALID_ARG   # slots unaligned
    assert rr(p, 100, p, 10, 4, 656, 2, p, None) == smla.ERR_INVALID_ARG      # 2 groups of 4 cannot cover 10 slots
    assert rr(p, 100, p, 0, 4, 1152, 0, p, None) == smla.OK                    # nothing to read
