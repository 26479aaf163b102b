"""Upload a seeded Workload to GPU memory (torch is plumbing here: allocation and copies)."""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

from . import Workload


@dataclasses.dataclass
class DeviceInputs:
    q: torch.Tensor            # bf16 [B, 64, 576]
    pool: torch.Tensor         # uint8 [pool_bytes]
    page_table: torch.Tensor   # int32 [B, max_pages]
    topk_idx: torch.Tensor     # int32 [B, 512]
    ctx_len: torch.Tensor      # int32 [B]
    kv_format: int
    pool_pages: int
    scale: float


def upload(w: Workload, device="cuda", pool: torch.Tensor | None = None) -> DeviceInputs:
    """Copy w to `device`.  The pool is zero-filled and only the written rows are
    scattered in; pass `pool` to scatter into an existing (shared) pool."""
    dev = torch.device(device)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    if pool is None:
        pool = torch.zeros(w.pool_bytes, dtype=torch.uint8, device=dev)
    if len(w.row_slots):
        rows = pool.view(-1, w.row_bytes)
        rows[t(w.row_slots)] = t(w.row_data)
    return DeviceInputs(q=t(w.q).view(torch.bfloat16), pool=pool, page_table=t(w.page_table),
                        topk_idx=t(w.topk_idx), ctx_len=t(w.ctx_len), kv_format=w.kv_format,
                        pool_pages=w.pool_pages, scale=float(w.scale))


def request_slice(d: DeviceInputs, lo: int, hi: int) -> DeviceInputs:
    """Requests lo .. hi-1 of `d` as their own batch (views of the same memory,
    same pool): several disjoint batches can be cut from one input set."""
    return dataclasses.replace(d, q=d.q[lo:hi], page_table=d.page_table[lo:hi], topk_idx=d.topk_idx[lo:hi],
                               ctx_len=d.ctx_len[lo:hi])
