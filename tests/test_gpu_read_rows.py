"""smla_read_rows, the row-read measurement aid (needs an MI355X): every
thread's checksum word equals the XOR over the 16-byte pieces it reads, computed
on the CPU from the same pool bytes."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import sparse_mla_top_amd as smla
import workloads as W
from workloads.device import upload

pytestmark = pytest.mark.gpu

THREADS = 1024


def _say(msg):
    print(f"[gpu-test] {msg}", flush=True)


def _expected(pool: np.ndarray, slots: np.ndarray, per_group: int, n_groups: int, row_bytes: int) -> np.ndarray:
    pool_rows = pool.size // row_bytes
    rows = pool.reshape(pool_rows, row_bytes)
    out = np.zeros((n_groups, THREADS), np.uint32)
    for g in range(n_groups):
        sl = slots[g * per_group:(g + 1) * per_group]
        if sl.size == 0:
            continue
        ok = (sl >= 0) & (sl < pool_rows)
        data = np.zeros((sl.size, row_bytes), np.uint8)
        data[ok] = rows[sl[ok]]
        words = data.reshape(-1, 4, 4).view(np.uint8).reshape(-1, 16).view(np.uint32)   # pieces x 4 words
        piece = np.bitwise_xor.reduce(words, axis=1)
        pad = (-piece.size) % THREADS
        piece = np.concatenate([piece, np.zeros(pad, np.uint32)]).reshape(-1, THREADS)
        out[g] = np.bitwise_xor.reduce(piece, axis=0)
    return out


@pytest.mark.parametrize("fmt", [W.FMT_FP8, W.FMT_BF16])
@pytest.mark.parametrize("per_group", [512, 300])
def test_read_rows_checksums(fmt, per_group):
    w = W.build("read_rows", 970, 0, 4, [8192, 3000, 300, 20000], fmt, "uniform")
    d = upload(w)
    _, slots = smla.gather_rows(d.pool, d.page_table, d.topk_idx, d.ctx_len, kv_format=d.kv_format,
                                pool_pages=d.pool_pages)
    slots = slots.reshape(-1).contiguous()
    rb = w.row_bytes
    pool_rows = d.pool_pages * W.PAGE
    # one slot out of range: it must be skipped like a masked one
    slots_h = slots.cpu().numpy().copy()
    slots_h[7] = pool_rows + 5
    slots = torch.from_numpy(slots_h).cuda()
    n_groups = (slots_h.size + per_group - 1) // per_group
    sink = torch.zeros(n_groups * THREADS, dtype=torch.int32, device="cuda")
    _say(f"read_rows fmt={fmt} per_group={per_group} groups={n_groups}")
    assert smla.read_rows_raw(d.pool, pool_rows, slots, per_group, rb, n_groups, sink) == smla.OK
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32).reshape(n_groups, THREADS)
    exp = _expected(d.pool.cpu().numpy(), slots_h, per_group, n_groups, rb)
    assert np.array_equal(got, exp)
    assert (slots_h < 0).any()            # masked slots were part of the read
