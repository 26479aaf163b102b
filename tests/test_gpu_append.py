"""The cache producer (smla_kv_append) vs the oracle's, byte for byte (needs an MI355X)."""
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


def _say(msg):
    print(f"[gpu-test] {msg}", flush=True)


def _inputs(n, seed, B=6, max_pages=40, pool_pages=300):
    rng = np.random.default_rng(seed)
    lat = rng.standard_normal((n, 512)).astype(np.float32)
    rope = rng.standard_normal((n, 64)).astype(np.float32)
    # special blocks
    lat[0, 128:256] = 0.0                                   # all-zero block
    lat[1, :128] = 0.0
    lat[1, 77] = -3.25                                      # one non-zero value
    lat[2] *= np.float32(1e-30)                             # tiny magnitudes
    lat[3] *= np.float32(1e30)                              # huge magnitudes
    codes = np.arange(0, 0x7F, dtype=np.uint8)              # every finite positive e4m3 value ...
    vals = np.array([oracle.e4m3_to_f64(int(c)) for c in codes])
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)  # ... and every midpoint (ties)
    lat[4, :126] = mids[:126]
    lat[4, 126] = 448.0                                     # amax 448: scale exactly 1
    lat[4, 127] = -0.0
    lat[5, 256:384] = -mids[-128:] if mids.size >= 128 else -np.resize(mids, 128)
    lat[5, 300] = -448.0
    rope[0, :8] = np.array([1.00390625, 1.01171875, -1.00390625, 3e-39, -0.0, 65504.0, 1e38, -1e-45], np.float32)
    pt = rng.permutation(pool_pages)[:B * max_pages].astype(np.int32).reshape(B, max_pages)
    pt[B - 1, 5] = -3                                       # invalid page id
    req = rng.integers(0, B, n).astype(np.int32)
    pos = np.empty(n, np.int32)
    for b in range(B):
        ix = np.nonzero(req == b)[0]
        pos[ix] = rng.choice(max_pages * W.PAGE, len(ix), replace=False)
    req[6], req[7], pos[8], pos[9] = -1, B, -1, max_pages * W.PAGE   # invalid destinations
    return lat, rope, req, pos, pt, pool_pages


@pytest.mark.parametrize("fmt", [W.FMT_FP8, W.FMT_BF16])
@pytest.mark.parametrize("n", [1, 10, 2000])
def test_kv_append_bit_exact(fmt, n):
    _say(f"kv_append fmt={fmt} n={n}")
    lat, rope, req, pos, pt, pool_pages = _inputs(max(n, 10), 30 + n)
    lat, rope, req, pos = lat[:n], rope[:n], req[:n], pos[:n]
    rb = W.ROW_BYTES[fmt]
    ref = np.full(pool_pages * W.PAGE * rb, 0xA5, dtype=np.uint8)     # untouched rows keep their bytes
    oracle.kv_append(lat, rope, req, pos, pt, ref, pool_pages, fmt)
    pool = torch.full((pool_pages * W.PAGE * rb,), 0xA5, dtype=torch.uint8, device="cuda")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    smla.kv_append(t(lat), t(rope), t(req), t(pos), t(pt), pool, kv_format=fmt, pool_pages=pool_pages)
    torch.cuda.synchronize()
    got = pool.cpu().numpy()
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"{bad.size} bytes differ, first at row {bad[0] // rb} byte {bad[0] % rb}"


def test_decode_over_appended_rows():
    """Rows written by the producer feed the decode kernel: parity against the oracle
    decoding the oracle-produced pool (which the byte test shows is the same)."""
    w = W.build("append_e2e", 960, 0, 4, [5000, 700, 64, 3000], W.FMT_FP8, "uniform")
    # every selected token's row, re-produced from fresh fp32 values
    rng = np.random.default_rng(61)
    req, pos = [], []
    for b in range(w.B):
        sel = w.topk_idx[b][(w.topk_idx[b] >= 0) & (w.topk_idx[b] < w.ctx_len[b])]
        req += [b] * len(sel)
        pos += list(sel)
    req, pos = np.array(req, np.int32), np.array(pos, np.int32)
    lat = (rng.standard_normal((len(req), 512)) * rng.uniform(0.01, 30, (len(req), 1))).astype(np.float32)
    rope = rng.standard_normal((len(req), 64)).astype(np.float32)
    rb = w.row_bytes
    ref = np.zeros(w.pool_pages * W.PAGE * rb, dtype=np.uint8)
    oracle.kv_append(lat, rope, req, pos, w.page_table, ref, w.pool_pages, w.kv_format)
    d = upload(w)
    d.pool.zero_()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    smla.kv_append(t(lat), t(rope), t(req), t(pos), d.page_table, d.pool, kv_format=w.kv_format,
                   pool_pages=w.pool_pages)
    out, lse = smla.decode(d.q, d.pool, d.page_table, d.topk_idx, d.ctx_len, d.scale, kv_format=d.kv_format,
                           pool_pages=d.pool_pages)
    torch.cuda.synchronize()
    assert np.array_equal(d.pool.cpu().numpy(), ref)
    ref_o, ref_l = oracle.decode(w.q, w.kv_format, ref, w.pool_pages, w.page_table, w.topk_idx, w.ctx_len, w.scale)
    assert_parity(out, lse, ref_o, ref_l, "decode over appended rows")
