"""sparse_mla_top_amd -- sparse-MLA decode attention on MI355X (gfx950).

A thin ctypes binding over the C ABI of `libsparse_mla.so` (declared in
include/sparse_mla.h).  Every step of the decode runs in the library's HIP
kernels; this module only marshals torch device tensors into pointers and the
current HIP stream.  There is no CPU fallback: a missing library raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads torch's HIP runtime first; the library then binds to the same one

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsparse_mla.so")

NUM_HEADS = 64
D_QK = 576
D_V = 512
TOPK = 512
PAGE_SIZE = 64
KV_BF16 = 0
KV_FP8 = 1
ROW_BYTES = {KV_BF16: 1152, KV_FP8: 656}

OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED_SHAPE = -2
ERR_WORKSPACE = -3
ERR_PLAN = -4
ERR_HIP = -5
ERR_INDEX = -6       # validate mode (environment SMLA_VALIDATE=1): an index or page id out of range
ERR_MERGE = -7       # validate mode: an in-kernel split merge gave up waiting (smla_workspace_init needed)
NOALLOC_SCRATCH_BYTES = 32 << 20   # the workspace that sparse_mla_decode_noalloc brings, per GPU

MERGE_AUTO = 0
MERGE_IN_KERNEL = 1
MERGE_SEPARATE = 2
MERGE_SPREAD = 3     # same launch, every split merges a share (grids of at most one workgroup per CU)


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("d_qk", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("topk", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("max_pages_per_req", ctypes.c_int32), ("kv_format", ctypes.c_int32),
                ("pool_pages", ctypes.c_int64), ("q_len", ctypes.c_int32)]


class Plan(ctypes.Structure):
    _fields_ = [("nsplit", ctypes.c_int32), ("tile_tokens", ctypes.c_int32),
                ("heads_per_wg", ctypes.c_int32), ("wg_per_cu", ctypes.c_int32), ("merge", ctypes.c_int32)]

    def as_dict(self) -> dict:
        return {f: int(getattr(self, f)) for f, _ in self._fields_}


class SmlaError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {strerror(code)} ({code})")
        self.code = code


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32p, i64p = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
        L.smla_plan_for.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Plan), ctypes.POINTER(Plan),
                                    ctypes.POINTER(ctypes.c_size_t)]
        L.smla_plan_for.restype = ctypes.c_int
        L.smla_plan_for_cus.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Plan), ctypes.c_int,
                                        ctypes.POINTER(Plan), ctypes.POINTER(ctypes.c_size_t)]
        L.smla_plan_for_cus.restype = ctypes.c_int
        L.sparse_mla_decode.argtypes = [vp, vp, i32p, i32p, i32p, ctypes.c_float, vp, vp,
                                        ctypes.POINTER(Shape), ctypes.POINTER(Plan), vp, ctypes.c_size_t, vp]
        L.sparse_mla_decode.restype = ctypes.c_int
        L.sparse_mla_decode_noalloc.argtypes = [vp, vp, i32p, i32p, i32p, ctypes.c_float, vp, vp,
                                                ctypes.POINTER(Shape), ctypes.POINTER(Plan), vp]
        L.sparse_mla_decode_noalloc.restype = ctypes.c_int
        L.smla_decode_split.argtypes = L.sparse_mla_decode.argtypes
        L.smla_decode_split.restype = ctypes.c_int
        L.smla_decode_combine.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Plan), vp, ctypes.c_size_t, vp, vp, vp]
        L.smla_decode_combine.restype = ctypes.c_int
        L.smla_workspace_init.argtypes = [vp, ctypes.c_size_t, vp]
        L.smla_workspace_init.restype = ctypes.c_int
        L.smla_gather_rows.argtypes = [vp, i32p, i32p, i32p, ctypes.POINTER(Shape), vp, i64p, vp]
        L.smla_gather_rows.restype = ctypes.c_int
        L.smla_read_rows.argtypes = [vp, ctypes.c_int64, i64p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32, vp, vp]
        L.smla_read_rows.restype = ctypes.c_int
        L.smla_kv_append.argtypes = [vp, vp, i32p, i32p, i32p, vp, ctypes.c_int32, ctypes.POINTER(Shape), vp]
        L.smla_kv_append.restype = ctypes.c_int
        L.smla_indexer_topk.argtypes = [vp, vp, vp, i32p, i32p, vp, i32p, ctypes.POINTER(Shape), vp]
        L.smla_indexer_topk.restype = ctypes.c_int
        L.smla_row_bytes.argtypes = [ctypes.c_int]
        L.smla_row_bytes.restype = ctypes.c_int
        L.smla_strerror.argtypes = [ctypes.c_int]
        L.smla_strerror.restype = ctypes.c_char_p
        L.smla_version.argtypes = []
        L.smla_version.restype = ctypes.c_int
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().smla_strerror(int(code)).decode()


def make_shape(batch: int, kv_format: int, max_pages_per_req: int, pool_pages: int, q_len: int = 1) -> Shape:
    return Shape(int(batch), NUM_HEADS, D_QK, D_V, TOPK, PAGE_SIZE, int(max_pages_per_req),
                 int(kv_format), int(pool_pages), int(q_len))


def _plan_arg(plan):
    if plan is None:
        return None
    if isinstance(plan, Plan):
        return ctypes.byref(plan)
    if isinstance(plan, dict):
        return ctypes.byref(Plan(int(plan.get("nsplit", 0)), int(plan.get("tile_tokens", 0)),
                                 int(plan.get("heads_per_wg", 0)), int(plan.get("wg_per_cu", 0)),
                                 int(plan.get("merge", 0))))
    return ctypes.byref(Plan(int(plan), 0, 0, 0, 0))     # an int = forced nsplit


def plan_for(shape: Shape, plan=None):
    """(Plan, workspace bytes) on the current device."""
    out, ws = Plan(), ctypes.c_size_t(0)
    rc = lib().smla_plan_for(ctypes.byref(shape), _plan_arg(plan), ctypes.byref(out), ctypes.byref(ws))
    if rc != OK:
        raise SmlaError(rc, "smla_plan_for")
    return out, int(ws.value)


def plan_for_cus(shape: Shape, num_cus: int, plan=None):
    """(Plan, workspace bytes) for a device with `num_cus` compute units (host only)."""
    out, ws = Plan(), ctypes.c_size_t(0)
    rc = lib().smla_plan_for_cus(ctypes.byref(shape), _plan_arg(plan), int(num_cus), ctypes.byref(out),
                                 ctypes.byref(ws))
    if rc != OK:
        raise SmlaError(rc, "smla_plan_for_cus")
    return out, int(ws.value)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check_tensors(shape: Shape, q, kv_pool, page_table, topk_idx, ctx_len, out, lse):
    """Raise if a tensor is smaller than `shape` says (the kernels trust the shape)."""
    B = int(shape.batch)
    if B <= 0:
        return
    Q = B * max(int(shape.q_len), 1)          # query sets (request, query token)
    rb = ROW_BYTES.get(int(shape.kv_format))
    need = [(q, Q * NUM_HEADS * D_QK * 2, "q"), (page_table, B * int(shape.max_pages_per_req) * 4, "page_table"),
            (topk_idx, B * TOPK * 4, "topk_idx"), (ctx_len, B * 4, "ctx_len"),
            (out, Q * NUM_HEADS * D_V * 2, "out"), (lse, Q * NUM_HEADS * 4, "lse")]
    if rb is not None:
        need.append((kv_pool, int(shape.pool_pages) * PAGE_SIZE * rb, "kv_pool"))
    for t, nbytes, name in need:
        if t is None:
            continue
        have = t.numel() * t.element_size()
        if have < nbytes or not t.is_contiguous():
            raise ValueError(f"{name}: {have} bytes (contiguous={t.is_contiguous()}) but the shape needs {nbytes}")


def decode_raw(q, kv_pool, page_table, topk_idx, ctx_len, scale, out, lse, shape: Shape, plan=None,
               workspace=None, stream=None) -> int:
    """sparse_mla_decode on torch tensors; returns the library's status code."""
    _check_tensors(shape, q, kv_pool, page_table, topk_idx, ctx_len, out, lse)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return lib().sparse_mla_decode(_ptr(q), _ptr(kv_pool), _ptr(page_table), _ptr(topk_idx), _ptr(ctx_len),
                                   float(scale), _ptr(out), _ptr(lse), ctypes.byref(shape), _plan_arg(plan),
                                   _ptr(workspace), ctypes.c_size_t(ws_bytes), _stream(stream))


def decode_noalloc_raw(q, kv_pool, page_table, topk_idx, ctx_len, scale, out, lse, shape: Shape, plan=None,
                       stream=None) -> int:
    """sparse_mla_decode_noalloc on torch tensors (the workspace is the library's
    own device array); returns the library's status code."""
    _check_tensors(shape, q, kv_pool, page_table, topk_idx, ctx_len, out, lse)
    return lib().sparse_mla_decode_noalloc(_ptr(q), _ptr(kv_pool), _ptr(page_table), _ptr(topk_idx), _ptr(ctx_len),
                                           float(scale), _ptr(out), _ptr(lse), ctypes.byref(shape), _plan_arg(plan),
                                           _stream(stream))


def split_raw(q, kv_pool, page_table, topk_idx, ctx_len, scale, out, lse, shape: Shape, plan=None,
              workspace=None, stream=None) -> int:
    """smla_decode_split on torch tensors; returns the status code."""
    _check_tensors(shape, q, kv_pool, page_table, topk_idx, ctx_len, out, lse)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return lib().smla_decode_split(_ptr(q), _ptr(kv_pool), _ptr(page_table), _ptr(topk_idx), _ptr(ctx_len),
                                   float(scale), _ptr(out), _ptr(lse), ctypes.byref(shape), _plan_arg(plan),
                                   _ptr(workspace), ctypes.c_size_t(ws_bytes), _stream(stream))


def combine_raw(shape: Shape, plan, workspace, out, lse, stream=None) -> int:
    """smla_decode_combine on torch tensors; returns the status code."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return lib().smla_decode_combine(ctypes.byref(shape), _plan_arg(plan), _ptr(workspace),
                                     ctypes.c_size_t(ws_bytes), _ptr(out), _ptr(lse), _stream(stream))


def new_workspace(nbytes: int, device=None, stream=None):
    """A zero-initialised workspace of `nbytes` (at least 256) for sparse_mla_decode."""
    ws = torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device or "cuda")
    return ws


def workspace_init(workspace, stream=None) -> None:
    """Zero a workspace's arrival counters on the stream (fill kernel)."""
    rc = lib().smla_workspace_init(_ptr(workspace), ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                                   _stream(stream))
    if rc != OK:
        raise SmlaError(rc, "smla_workspace_init")


def decode(q, kv_pool, page_table, topk_idx, ctx_len, scale, *, kv_format: int, pool_pages: int,
           out=None, lse=None, plan=None, workspace=None, stream=None):
    """Sparse-MLA decode attention.  Returns (out bf16 [B,64,512], lse fp32 [B,64]).

    q bf16 [B,64,576], or [B,q_len,64,576] for q_len query tokens per request
    sharing its selection (out [B,q_len,64,512], lse [B,q_len,64]);
    kv_pool uint8 [pool bytes]; page_table int32 [B,max_pages];
    topk_idx int32 [B,512]; ctx_len int32 [B] -- all on the current GPU.
    """
    B = q.shape[0]
    q_len = q.shape[1] if q.dim() == 4 else 1
    lead = (B, q_len) if q.dim() == 4 else (B,)
    shape = make_shape(B, kv_format, page_table.shape[1], pool_pages, q_len)
    if out is None:
        out = torch.empty(lead + (NUM_HEADS, D_V), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty(lead + (NUM_HEADS,), dtype=torch.float32, device=q.device)
    if workspace is None:
        _, ws = plan_for(shape, plan)
        workspace = new_workspace(ws, q.device)
    rc = decode_raw(q, kv_pool, page_table, topk_idx, ctx_len, scale, out, lse, shape, plan, workspace, stream)
    if rc != OK:
        raise SmlaError(rc, "sparse_mla_decode")
    return out, lse


def gather_rows(kv_pool, page_table, topk_idx, ctx_len, *, kv_format: int, pool_pages: int, stream=None):
    """Test hook: (rows uint8 [B,512,row_bytes], slots int64 [B,512]) from the gather stage."""
    B = topk_idx.shape[0]
    shape = make_shape(B, kv_format, page_table.shape[1], pool_pages)
    _check_tensors(shape, None, kv_pool, page_table, topk_idx, ctx_len, None, None)
    rows = torch.empty((B, TOPK, ROW_BYTES[kv_format]), dtype=torch.uint8, device=topk_idx.device)
    slots = torch.empty((B, TOPK), dtype=torch.int64, device=topk_idx.device)
    rc = lib().smla_gather_rows(_ptr(kv_pool), _ptr(page_table), _ptr(topk_idx), _ptr(ctx_len),
                                ctypes.byref(shape), _ptr(rows), _ptr(slots), _stream(stream))
    if rc != OK:
        raise SmlaError(rc, "smla_gather_rows")
    return rows, slots


def read_rows_raw(kv_pool, pool_rows: int, slots, per_group: int, row_bytes: int, n_groups: int, sink,
                  stream=None) -> int:
    """smla_read_rows on torch tensors (slots int64, sink uint32-sized int32); returns the status code."""
    n = int(slots.numel())
    for t, nbytes, name in ((slots, n * 8, "slots"), (sink, int(n_groups) * 1024 * 4, "sink"),
                            (kv_pool, int(pool_rows) * int(row_bytes), "kv_pool")):
        if t.numel() * t.element_size() < nbytes or not t.is_contiguous():
            raise ValueError(f"{name}: smaller than the call needs ({nbytes} bytes) or not contiguous")
    return lib().smla_read_rows(_ptr(kv_pool), int(pool_rows), _ptr(slots), n, int(per_group), int(row_bytes),
                                int(n_groups), _ptr(sink), _stream(stream))


def kv_append_raw(latent, rope, req, pos, page_table, kv_pool, shape: Shape, stream=None) -> int:
    """smla_kv_append on torch tensors; returns the library's status code."""
    n = int(latent.shape[0]) if latent is not None else 0
    if n > 0:
        for t, nbytes, name in ((latent, n * 512 * 4, "latent"), (rope, n * 64 * 4, "rope"), (req, n * 4, "req"),
                                (pos, n * 4, "pos"),
                                (page_table, int(shape.batch) * int(shape.max_pages_per_req) * 4, "page_table")):
            have = t.numel() * t.element_size()
            if have < nbytes or not t.is_contiguous():
                raise ValueError(f"{name}: {have} bytes (contiguous={t.is_contiguous()}) but {nbytes} are needed")
        rb = ROW_BYTES.get(int(shape.kv_format))
        if rb is not None and kv_pool.numel() * kv_pool.element_size() < int(shape.pool_pages) * PAGE_SIZE * rb:
            raise ValueError("kv_pool is smaller than shape.pool_pages pages")
    return lib().smla_kv_append(_ptr(latent), _ptr(rope), _ptr(req), _ptr(pos), _ptr(page_table), _ptr(kv_pool),
                                n, ctypes.byref(shape), _stream(stream))


def kv_append(latent, rope, req, pos, page_table, kv_pool, *, kv_format: int, pool_pages: int, stream=None) -> None:
    """Quantise new tokens' rows (latent fp32 [n,512], rope fp32 [n,64]) and write them into
    kv_pool at page_table[req][pos // 64] * 64 + pos % 64 (all on the current GPU)."""
    shape = make_shape(page_table.shape[0], kv_format, page_table.shape[1], pool_pages)
    rc = kv_append_raw(latent, rope, req, pos, page_table, kv_pool, shape, stream)
    if rc != OK:
        raise SmlaError(rc, "smla_kv_append")


INDEXER_HEADS = 64
INDEXER_DIM = 128


def indexer_topk_raw(q_idx, head_w, key_pool, page_table, ctx_len, scores, topk_idx, shape: Shape,
                     stream=None) -> int:
    """smla_indexer_topk on torch tensors; returns the library's status code."""
    B = int(shape.batch)
    if B > 0:
        npos = int(shape.max_pages_per_req) * PAGE_SIZE
        for t, nbytes, name in ((q_idx, B * INDEXER_HEADS * INDEXER_DIM * 2, "q_idx"),
                                (head_w, B * INDEXER_HEADS * 4, "head_w"),
                                (key_pool, int(shape.pool_pages) * PAGE_SIZE * INDEXER_DIM * 2, "key_pool"),
                                (page_table, B * int(shape.max_pages_per_req) * 4, "page_table"),
                                (ctx_len, B * 4, "ctx_len"), (scores, B * npos * 4, "scores"),
                                (topk_idx, B * TOPK * 4, "topk_idx")):
            have = t.numel() * t.element_size()
            if have < nbytes or not t.is_contiguous():
                raise ValueError(f"{name}: {have} bytes (contiguous={t.is_contiguous()}) but {nbytes} are needed")
    return lib().smla_indexer_topk(_ptr(q_idx), _ptr(head_w), _ptr(key_pool), _ptr(page_table), _ptr(ctx_len),
                                   _ptr(scores), _ptr(topk_idx), ctypes.byref(shape), _stream(stream))


def indexer_topk(q_idx, head_w, key_pool, page_table, ctx_len, *, pool_pages: int, stream=None):
    """Top-k indexer: returns (topk_idx int32 [B,512], scores fp32 [B,max_pages*64]).
    q_idx bf16 [B,64,128]; head_w fp32 [B,64]; key_pool bf16 [pool_pages*64,128]."""
    B, mp = page_table.shape
    shape = make_shape(B, KV_FP8, mp, pool_pages)
    scores = torch.empty((B, mp * PAGE_SIZE), dtype=torch.float32, device=q_idx.device)
    idx = torch.empty((B, TOPK), dtype=torch.int32, device=q_idx.device)
    rc = indexer_topk_raw(q_idx, head_w, key_pool, page_table, ctx_len, scores, idx, shape, stream)
    if rc != OK:
        raise SmlaError(rc, "smla_indexer_topk")
    return idx, scores
