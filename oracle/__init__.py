"""fp64 CPU oracle for sparse-MLA decode attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It wraps `oracle.c` (plain C, fp64, OpenMP) through ctypes and
shares no code with the HIP library it checks.  What it computes, and the
readings it takes where the pages are silent, are stated in `oracle.c`.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

FMT_BF16 = 0
FMT_FP8 = 1


def build(out_path: str = _LIB_PATH, defines: tuple[str, ...] = ()) -> str:
    """Compile oracle.c with gcc (-O2, IEEE semantics, OpenMP) into a shared library."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
           "-ffp-contract=off", *[f"-D{d}" for d in defines], _SRC, "-o", out_path, "-lm"]
    subprocess.run(cmd, check=True)
    return out_path


def _bind(lib):
    c = ctypes
    p = c.c_void_p
    lib.oracle_e4m3_to_f64.restype = c.c_double
    lib.oracle_e4m3_to_f64.argtypes = [c.c_uint8]
    lib.oracle_bf16_to_f64.restype = c.c_double
    lib.oracle_bf16_to_f64.argtypes = [c.c_uint16]
    lib.oracle_row_bytes.restype = c.c_int
    lib.oracle_row_bytes.argtypes = [c.c_int]
    lib.oracle_decode_row.restype = None
    lib.oracle_decode_row.argtypes = [c.c_int, p, p]
    lib.oracle_gather.restype = c.c_int
    lib.oracle_gather.argtypes = [c.c_int, c.c_int, c.c_int, c.c_int64, c.c_int, p, p, p, p, p, p]
    lib.oracle_decode.restype = c.c_int
    lib.oracle_decode.argtypes = [c.c_int, c.c_int, c.c_int, c.c_int, c.c_int64, c.c_int,
                                  p, p, p, p, p, c.c_float, p, p, c.c_int]
    lib.oracle_max_threads.restype = c.c_int
    lib.oracle_e4m3_encode.argtypes = [c.c_float]
    lib.oracle_e4m3_encode.restype = c.c_uint8
    lib.oracle_f32_to_bf16.argtypes = [c.c_float]
    lib.oracle_f32_to_bf16.restype = c.c_uint16
    lib.oracle_kv_append.argtypes = [c.c_int, c.c_int, c.c_int, c.c_int64, c.c_int, p, p, p, p, p, p]
    lib.oracle_kv_append.restype = c.c_int
    lib.oracle_topk_select.argtypes = [c.c_int, c.c_int, c.c_int, c.c_int64, p, p, p, p]
    lib.oracle_topk_select.restype = c.c_int
    lib.oracle_indexer.argtypes = [c.c_int, c.c_int, c.c_int, c.c_int, c.c_int, c.c_int64, p, p, p, p, p, p, p,
                                   c.c_int]
    lib.oracle_indexer.restype = c.c_int
    lib.oracle_max_threads.argtypes = []
    return lib


def load(path: str | None = None):
    """Load the built oracle (building it first if absent).  A path loads a variant."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def e4m3_to_f64(code: int, lib=None) -> float:
    return (lib or load()).oracle_e4m3_to_f64(int(code))


def bf16_to_f64(bits: int, lib=None) -> float:
    return (lib or load()).oracle_bf16_to_f64(int(bits))


def decode_row(kv_format: int, row: np.ndarray, lib=None) -> np.ndarray:
    row = np.ascontiguousarray(row, dtype=np.uint8)
    x = np.zeros(576, dtype=np.float64)
    (lib or load()).oracle_decode_row(int(kv_format), _ptr(row), _ptr(x))
    return x


def gather(q_shape_B: int, topk: int, kv_format: int, kv_pool: np.ndarray, pool_pages: int,
           page_table: np.ndarray, topk_idx: np.ndarray, ctx_len: np.ndarray,
           with_rows: bool = True, lib=None):
    """Index translation + row gather: (slots int64 [B, topk], rows uint8 [B, topk, row_bytes])."""
    lib = lib or load()
    B = int(q_shape_B)
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx_len, dtype=np.int32)
    rb = lib.oracle_row_bytes(int(kv_format))
    slots = np.empty((B, topk), dtype=np.int64)
    rows = np.empty((B, topk, rb), dtype=np.uint8) if with_rows else None
    rc = lib.oracle_gather(B, topk, pt.shape[1], int(pool_pages), int(kv_format), _ptr(kv_pool),
                           _ptr(pt), _ptr(idx), _ptr(ctx), _ptr(slots),
                           _ptr(rows) if with_rows else None)
    if rc != 0:
        raise ValueError(f"oracle_gather failed ({rc})")
    return slots, rows


def decode(q: np.ndarray, kv_format: int, kv_pool: np.ndarray, pool_pages: int,
           page_table: np.ndarray, topk_idx: np.ndarray, ctx_len: np.ndarray, scale,
           nthreads: int = 0, lib=None):
    """Attention over the selected rows: (out float64 [B, H, 512], lse float64 [B, H]).

    q may also be [B, q_len, H, 576]: q_len query tokens per request sharing its
    selection, each (token, head) row attending over the same selected rows;
    then out is [B, q_len, H, 512] and lse [B, q_len, H].
    """
    lib = lib or load()
    q = np.ascontiguousarray(q, dtype=np.uint16)
    if q.ndim == 4:
        B4, T4, H4, _ = q.shape
        o, l = decode(q.reshape(B4, T4 * H4, q.shape[3]), kv_format, kv_pool, pool_pages, page_table,
                      topk_idx, ctx_len, scale, nthreads=nthreads, lib=lib)
        return o.reshape(B4, T4, H4, o.shape[-1]), l.reshape(B4, T4, H4)
    B, H, dqk = q.shape
    assert dqk == 576
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx_len, dtype=np.int32)
    out = np.zeros((B, H, 512), dtype=np.float64)
    lse = np.zeros((B, H), dtype=np.float64)
    rc = lib.oracle_decode(B, H, idx.shape[1], pt.shape[1], int(pool_pages), int(kv_format),
                           _ptr(q), _ptr(kv_pool), _ptr(pt), _ptr(idx), _ptr(ctx),
                           float(np.float32(scale)), _ptr(out), _ptr(lse), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_decode failed ({rc})")
    return out, lse


def decode_workload(w, nthreads: int = 0, lib=None, pool: np.ndarray | None = None):
    """Convenience: run `decode` on a workloads.Workload."""
    if pool is None:
        pool = w.host_pool()
    return decode(w.q, w.kv_format, pool, w.pool_pages, w.page_table, w.topk_idx, w.ctx_len,
                  w.scale, nthreads=nthreads, lib=lib)


def gather_workload(w, with_rows: bool = True, lib=None, pool: np.ndarray | None = None):
    if pool is None:
        pool = w.host_pool()
    return gather(w.B, w.topk_idx.shape[1], w.kv_format, pool, w.pool_pages, w.page_table,
                  w.topk_idx, w.ctx_len, with_rows=with_rows, lib=lib)


def e4m3_encode(v: float, lib=None) -> int:
    return int((lib or load()).oracle_e4m3_encode(float(v)))


def f32_to_bf16(v: float, lib=None) -> int:
    return int((lib or load()).oracle_f32_to_bf16(float(v)))


def kv_append(latent: np.ndarray, rope: np.ndarray, req: np.ndarray, pos: np.ndarray, page_table: np.ndarray,
              kv_pool: np.ndarray, pool_pages: int, kv_format: int, lib=None) -> int:
    """Quantise and write each token's row into kv_pool (uint8, modified in place) at the slot
    page_table[req][pos // 64] * 64 + pos % 64; out-of-range destinations are skipped.
    latent float32 [n, 512], rope float32 [n, 64].  Returns the number of rows written."""
    lib = lib or load()
    lat = np.ascontiguousarray(latent, dtype=np.float32)
    rp = np.ascontiguousarray(rope, dtype=np.float32)
    rq = np.ascontiguousarray(req, dtype=np.int32)
    ps = np.ascontiguousarray(pos, dtype=np.int32)
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    assert kv_pool.dtype == np.uint8 and kv_pool.flags.c_contiguous
    n = lat.shape[0]
    assert lat.shape == (n, 512) and rp.shape == (n, 64) and rq.shape == (n,) and ps.shape == (n,)
    rc = lib.oracle_kv_append(n, pt.shape[0], pt.shape[1], int(pool_pages), int(kv_format), _ptr(lat), _ptr(rp),
                              _ptr(rq), _ptr(ps), _ptr(pt), _ptr(kv_pool))
    if rc < 0:
        raise ValueError(f"oracle_kv_append failed ({rc})")
    return rc


def indexer(q: np.ndarray, w: np.ndarray, kpool: np.ndarray, pool_pages: int, page_table: np.ndarray,
            ctx_len: np.ndarray, topk: int = 512, nthreads: int = 0, lib=None):
    """Indexer scores and selection: (scores float64 [B, max_pages*64] (NaN where excluded),
    topk_idx int32 [B, topk]).  q bf16 bits [B, HI, DI], w float32 [B, HI],
    kpool bf16 bits [pool_pages*64, DI]."""
    lib = lib or load()
    q = np.ascontiguousarray(q, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.float32)
    kp = np.ascontiguousarray(kpool, dtype=np.uint16)
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx_len, dtype=np.int32)
    B, HI, DI = q.shape
    scores = np.empty((B, pt.shape[1] * 64), dtype=np.float64)
    idx = np.empty((B, topk), dtype=np.int32)
    rc = lib.oracle_indexer(B, HI, DI, topk, pt.shape[1], int(pool_pages), _ptr(q), _ptr(w), _ptr(kp), _ptr(pt),
                            _ptr(ctx), _ptr(scores), _ptr(idx), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_indexer failed ({rc})")
    return scores, idx


def topk_select(scores: np.ndarray, pool_pages: int, page_table: np.ndarray, ctx_len: np.ndarray, topk: int = 512,
                lib=None) -> np.ndarray:
    """The selection rule alone, on given scores [B, max_pages*64] (e.g. a kernel's fp32 scores)."""
    lib = lib or load()
    sc = np.ascontiguousarray(scores, dtype=np.float64)
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx_len, dtype=np.int32)
    idx = np.empty((pt.shape[0], topk), dtype=np.int32)
    rc = lib.oracle_topk_select(pt.shape[0], topk, pt.shape[1], int(pool_pages), _ptr(pt), _ptr(ctx), _ptr(sc),
                                _ptr(idx))
    if rc != 0:
        raise ValueError(f"oracle_topk_select failed ({rc})")
    return idx


def max_threads(lib=None) -> int:
    return (lib or load()).oracle_max_threads()
