"""Seeded synthetic inputs for sparse-MLA decode attention.

This module is shared by the GPU path's tests and benchmark and by the oracle's
tests.  It draws random numbers and lays out bytes; it holds none of the
attention arithmetic (no dequantisation, no dot products, no softmax).

Inputs follow the workloads of the DeepSeek-V4-Flash decode deployment that the
pages study ("Inside the Decode Performance Investigation ...", section "The
Setup": 64 query heads, index_topk = 512, 512K context, graph buckets up to 96):

* Q ~ N(0, 1), rounded to bf16 (round-to-nearest-even).
* Latent KV ~ N(0, 1) in fp32, quantised per (token, 128-dim block) with
  scale = amax / 448 to OCP e4m3fn (round-to-nearest-even); rope ~ N(0, 1) in bf16.
* Top-k indices drawn without replacement, in random order, padded with -1 when
  a request has fewer than 512 tokens.
* Each request's logical 64-token pages map to distinct physical pages drawn
  from a random permutation of one shared pool.

Only the rows that some top-k index selects are generated and written; every
other row of the pool stays zero and is never read ("row-sparse pool").
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

H = 64            # query heads
D_LATENT = 512    # latent dims = V dims
D_ROPE = 64       # rope dims
D_QK = D_LATENT + D_ROPE
TOPK = 512
PAGE = 64         # tokens per page
BLOCK = 128       # latent dims per fp8 scale

FMT_BF16 = 0      # row = 576 bf16 (latent then rope)            -> 1152 B
FMT_FP8 = 1       # row = 512 e4m3 | 4 fp32 scales | 64 bf16 rope -> 656 B
ROW_BYTES = {FMT_BF16: 2 * D_QK, FMT_FP8: D_LATENT + 4 * (D_LATENT // BLOCK) + 2 * D_ROPE}

SCALE = np.float32(1.0 / math.sqrt(D_QK))   # fp32 1/24, bits 0x3D2AAAAB
SEED_BASE = 0x5317A

# workload ids used in the seed tuple, and their descriptive names
WORKLOADS = {
    1: "b1_ctx4k_bf16",
    2: "b32_ctx64k_fp8",
    3: "b80_ctx128k_fp8_local",
    4: "b96_ragged_fp8",
    5: "sweep_ctx512k_fp8",
}
SWEEP_B = (1, 8, 16, 32, 48, 64, 80, 88, 96)
SWEEP_LAYERS = 42


# --------------------------------------------------------------------------- encoders
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round-to-nearest-even (torch's cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def e4m3_codes(x: np.ndarray) -> np.ndarray:
    """fp32 -> OCP e4m3fn codes (uint8), round-to-nearest-even (torch's cast).

    Callers keep |x| <= 448, so no value saturates or turns into NaN.
    """
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def quantise_latent(latent: np.ndarray):
    """Per (token, 128-dim block) scale = amax / 448 (fp32); an all-zero block uses 1.0.

    Returns (codes uint8 [n, 512], scales fp32 [n, 4]).
    """
    n = latent.shape[0]
    blocks = latent.reshape(n, D_LATENT // BLOCK, BLOCK).astype(np.float32)
    amax = np.abs(blocks).max(axis=2)
    scales = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    scaled = (blocks / scales[:, :, None]).astype(np.float32)
    codes = e4m3_codes(scaled.reshape(n, D_LATENT))
    return codes, scales


def pack_rows(fmt: int, latent: np.ndarray, rope: np.ndarray) -> np.ndarray:
    """Lay out n cache rows (uint8 [n, row_bytes]) from fp32 latent [n,512] and rope [n,64]."""
    n = latent.shape[0]
    rows = np.zeros((n, ROW_BYTES[fmt]), dtype=np.uint8)
    if fmt == FMT_FP8:
        codes, scales = quantise_latent(latent)
        rows[:, 0:512] = codes
        rows[:, 512:528] = scales.astype("<f4").view(np.uint8).reshape(n, 16)
        rows[:, 528:656] = bf16_bits(rope).astype("<u2").view(np.uint8).reshape(n, 128)
    elif fmt == FMT_BF16:
        rows[:, 0:1024] = bf16_bits(latent).astype("<u2").view(np.uint8).reshape(n, 1024)
        rows[:, 1024:1152] = bf16_bits(rope).astype("<u2").view(np.uint8).reshape(n, 128)
    else:
        raise ValueError(f"unknown kv format {fmt}")
    return rows


def lazy_zeros(nbytes: int) -> np.ndarray:
    """uint8 zeros whose pages are only materialised when written."""
    import mmap
    m = mmap.mmap(-1, max(int(nbytes), 1), flags=mmap.MAP_PRIVATE | mmap.MAP_ANONYMOUS)
    if hasattr(mmap, "MADV_NOHUGEPAGE"):
        m.madvise(mmap.MADV_NOHUGEPAGE)
    return np.frombuffer(m, dtype=np.uint8)[:int(nbytes)]


# --------------------------------------------------------------------------- workload
@dataclasses.dataclass
class Workload:
    name: str
    kv_format: int
    q: np.ndarray            # uint16 bf16 bits [B, H, 576], or [B, q_len, H, 576]
    page_table: np.ndarray   # int32 [B, max_pages]
    topk_idx: np.ndarray     # int32 [B, TOPK]
    ctx_len: np.ndarray      # int32 [B]
    pool_pages: int          # physical pages in the pool
    row_slots: np.ndarray    # int64 [n] physical slots written (page * 64 + row)
    row_data: np.ndarray     # uint8 [n, row_bytes]
    scale: np.float32 = SCALE

    @property
    def B(self) -> int:
        return int(self.q.shape[0])

    @property
    def q_len(self) -> int:
        return int(self.q.shape[1]) if self.q.ndim == 4 else 1

    @property
    def row_bytes(self) -> int:
        return ROW_BYTES[self.kv_format]

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def pool_bytes(self) -> int:
        return self.pool_pages * PAGE * self.row_bytes

    def host_pool(self) -> np.ndarray:
        """The pool as uint8 [pool_pages * 64 * row_bytes].

        Backed by an anonymous mapping with 4 KiB pages (no huge pages), so a
        large pool only costs resident memory for the rows written here.
        """
        pool = lazy_zeros(self.pool_bytes)
        if len(self.row_slots):
            pool.reshape(-1, self.row_bytes)[self.row_slots] = self.row_data
        return pool

    def subset(self, b: int) -> "Workload":
        """The first b requests (same pool)."""
        return dataclasses.replace(
            self, name=f"{self.name}[:{b}]", q=self.q[:b].copy(),
            page_table=self.page_table[:b].copy(), topk_idx=self.topk_idx[:b].copy(),
            ctx_len=self.ctx_len[:b].copy())

    def n_valid(self) -> np.ndarray:
        """Selected, in-range slots per request (what the kernels must read)."""
        i = self.topk_idx.astype(np.int64)
        return ((i >= 0) & (i < self.ctx_len[:, None])).sum(axis=1)


def _streams(workload_id: int, layer: int):
    ss = np.random.SeedSequence([SEED_BASE, workload_id, layer])
    return [np.random.default_rng(s) for s in ss.spawn(5)]   # q, kv, idx, page table, ctx


def with_query_tokens(w: "Workload", q_len: int, seed_tag: int = 0x4D5450) -> "Workload":
    """A copy of `w` with q_len query tokens per request sharing its selection:
    q becomes [B, q_len, H, 576]; token 0 is w's own Q, tokens 1.. are N(0,1)
    draws (bf16 RNE) from the stream SeedSequence([SEED_BASE, seed_tag, name
    hash, q_len]).  The selection, page table and rows are w's."""
    assert w.q.ndim == 3 and q_len >= 1
    B = w.q.shape[0]
    tag = int.from_bytes(w.name.encode()[:8].ljust(8, b"\0"), "little") & 0x7FFFFFFF
    rng = np.random.default_rng(np.random.SeedSequence([SEED_BASE, seed_tag, tag, q_len]))
    q = np.empty((B, q_len, H, D_QK), dtype=np.uint16)
    q[:, 0] = w.q
    if q_len > 1:
        q[:, 1:] = bf16_bits(rng.standard_normal((B, q_len - 1, H, D_QK), dtype=np.float32))
    return dataclasses.replace(w, q=q, name=f"{w.name}_q{q_len}")


def _uniform_idx(rng, ctx: int) -> np.ndarray:
    if ctx >= TOPK:
        return rng.choice(ctx, TOPK, replace=False).astype(np.int32)
    out = np.full(TOPK, -1, dtype=np.int32)
    out[:ctx] = rng.permutation(ctx).astype(np.int32)
    return out


def _local_idx(rng, ctx: int, recent: int = 8192, n_recent: int = 358) -> np.ndarray:
    """358 indices from the last 8192 tokens, 154 from the rest, shuffled."""
    a = rng.choice(np.arange(ctx - recent, ctx), n_recent, replace=False)
    b = rng.choice(ctx - recent, TOPK - n_recent, replace=False)
    return rng.permutation(np.concatenate([a, b])).astype(np.int32)


def build(name: str, workload_id: int, layer: int, B: int, ctx_len, kv_format: int,
          idx_mode: str = "uniform", compact: bool = False, page_base: int = 0,
          max_pages: int | None = None, topk_idx: np.ndarray | None = None,
          q_zero: bool = False) -> Workload:
    """Draw one seeded input set.

    idx_mode: "uniform" | "local" | "given" (topk_idx supplied).
    compact:  False -> every logical page of every request gets a physical page
              (pool = sum ceil(ctx/64)); True -> only pages that hold a selected
              token get one ("row-sparse pool"), the rest map to page_base.
    page_base: first physical page of this set (several sets can share a pool).
    """
    rq, rkv, ridx, rpt, _ = _streams(workload_id, layer)
    ctx = np.asarray(ctx_len, dtype=np.int64).reshape(B)
    npages = (ctx + PAGE - 1) // PAGE
    if max_pages is None:
        max_pages = int(max(1, npages.max()))

    # indices
    if idx_mode == "given":
        idx = np.asarray(topk_idx, dtype=np.int32).reshape(B, TOPK).copy()
    else:
        idx = np.empty((B, TOPK), dtype=np.int32)
        for b in range(B):
            idx[b] = _local_idx(ridx, int(ctx[b])) if idx_mode == "local" else _uniform_idx(ridx, int(ctx[b]))

    # page table
    pt = np.full((B, max_pages), page_base, dtype=np.int32)
    valid = (idx >= 0) & (idx < ctx[:, None])
    if not compact:
        pool_pages = int(npages.sum())
        perm = rpt.permutation(pool_pages) + page_base
        off = 0
        for b in range(B):
            pt[b, :npages[b]] = perm[off:off + npages[b]]
            off += int(npages[b])
    else:
        ref = [np.unique(idx[b][valid[b]] // PAGE) for b in range(B)]
        pool_pages = int(sum(len(r) for r in ref))
        perm = rpt.permutation(pool_pages) + page_base
        off = 0
        for b in range(B):
            pt[b, ref[b]] = perm[off:off + len(ref[b])]
            off += len(ref[b])
    pool_pages = max(pool_pages, 1)

    # Q
    qf = rq.standard_normal((B, H, D_QK), dtype=np.float32)
    if q_zero:
        qf[:] = 0
    q = bf16_bits(qf)

    # rows, drawn per request in top-k order (first b requests are prefix-stable)
    slots_all, data_all = [], []
    for b in range(B):
        sel = idx[b][valid[b]].astype(np.int64)
        if len(sel) == 0:
            continue
        slots = pt[b, sel // PAGE].astype(np.int64) * PAGE + sel % PAGE
        lat = rkv.standard_normal((len(sel), D_LATENT), dtype=np.float32)
        rope = rkv.standard_normal((len(sel), D_ROPE), dtype=np.float32)
        slots_all.append(slots)
        data_all.append(pack_rows(kv_format, lat, rope))
    rb = ROW_BYTES[kv_format]
    row_slots = np.concatenate(slots_all) if slots_all else np.zeros(0, np.int64)
    row_data = np.concatenate(data_all) if data_all else np.zeros((0, rb), np.uint8)
    # a slot selected twice keeps its first row, so every copy of the pool agrees
    row_slots, first = np.unique(row_slots, return_index=True)
    row_data = row_data[first]
    return Workload(name=name, kv_format=kv_format, q=q, page_table=pt, topk_idx=idx,
                    ctx_len=ctx.astype(np.int32), pool_pages=pool_pages + page_base,
                    row_slots=row_slots, row_data=row_data)


def make(workload_id: int, layer: int = 0, compact: bool | None = None, page_base: int = 0,
         kv_format: int | None = None) -> Workload:
    """The five standard workloads (ids 1..5); `layer` selects an independent draw."""
    name = WORKLOADS[workload_id]
    if workload_id == 1:
        fmt = FMT_BF16 if kv_format is None else kv_format
        return build(name, 1, layer, 1, [4096], fmt, "uniform", bool(compact), page_base)
    if workload_id == 2:
        return build(name, 2, layer, 32, [65536] * 32, FMT_FP8 if kv_format is None else kv_format,
                     "uniform", bool(compact), page_base)
    if workload_id == 3:
        return build(name, 3, layer, 80, [131072] * 80, FMT_FP8 if kv_format is None else kv_format,
                     "local", bool(compact), page_base)
    if workload_id == 4:
        rctx = _streams(4, layer)[4]
        u = rctx.uniform(math.log(128.0), math.log(524288.0), size=96)
        ctx = np.clip(np.floor(np.exp(u)), 128, 524288).astype(np.int64)
        return build(name, 4, layer, 96, ctx, FMT_FP8 if kv_format is None else kv_format,
                     "uniform", bool(compact), page_base)
    if workload_id == 5:
        return build(name, 5, layer, 96, [524288] * 96, FMT_FP8 if kv_format is None else kv_format,
                     "uniform", True if compact is None else compact, page_base)
    raise ValueError(workload_id)

# --------------------------------------------------------------------------- indexer inputs
INDEXER_HEADS = 64
INDEXER_DIM = 128


@dataclasses.dataclass
class IndexerInputs:
    q: np.ndarray            # uint16 bf16 bits [B, HI, DI]
    w: np.ndarray            # float32 [B, HI]
    keys: np.ndarray         # uint16 bf16 bits [pool_pages * 64, DI]
    page_table: np.ndarray   # int32 [B, max_pages]
    ctx_len: np.ndarray      # int32 [B]
    pool_pages: int


def indexer_inputs(B: int, ctx_len, seed: int, heads: int = INDEXER_HEADS, dim: int = INDEXER_DIM,
                   max_pages: int | None = None) -> IndexerInputs:
    """Seeded inputs of the top-k indexer: q ~ N(0,1) and keys ~ N(0,1) rounded to bf16,
    head weights ~ U(-0.25, 1) (mostly positive), every logical page of every request on a
    distinct physical page (a random permutation of the pool).  Stream:
    SeedSequence([SEED_BASE, 0x1D3, seed])."""
    rng = np.random.default_rng(np.random.SeedSequence([SEED_BASE, 0x1D3, seed]))
    ctx = np.asarray(ctx_len, dtype=np.int64).reshape(B)
    npages = (ctx + PAGE - 1) // PAGE
    mp = int(max(1, npages.max())) if max_pages is None else max_pages
    pool_pages = int(max(1, npages.sum()))
    perm = rng.permutation(pool_pages)
    pt = np.zeros((B, mp), dtype=np.int32)
    off = 0
    for b in range(B):
        pt[b, :npages[b]] = perm[off:off + npages[b]]
        off += int(npages[b])
    q = bf16_bits(rng.standard_normal((B, heads, dim), dtype=np.float32))
    w = rng.uniform(-0.25, 1.0, (B, heads)).astype(np.float32)
    keys = bf16_bits(rng.standard_normal((pool_pages * PAGE, dim), dtype=np.float32))
    return IndexerInputs(q=q, w=w, keys=keys, page_table=pt, ctx_len=ctx.astype(np.int32), pool_pages=pool_pages)
