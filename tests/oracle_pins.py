"""Pins of the fp64 oracle against what the mathematics and library routines fix.

Each `pin_*` takes a loaded oracle library (the real one, or a variant with a
planted mistake) and raises AssertionError when the oracle disagrees.  Nothing
here re-types the oracle's attention arithmetic: attention is checked against
torch's scaled_dot_product_attention / logsumexp in float64, against closed
forms and invariants, and against a pure-Python brute force on tiny inputs;
element decoders are checked against torch's own fp8/bf16 casts.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
import workloads as W

TOL = 1e-11


# ----------------------------------------------------------------- test-side helpers
def _torch_rows(fmt: int, rows: np.ndarray):
    """(K float64 [n,576], V float64 [n,512]) from row bytes, decoded with torch casts."""
    rows = np.ascontiguousarray(rows, dtype=np.uint8)
    n = rows.shape[0]
    if fmt == W.FMT_FP8:
        codes = torch.from_numpy(rows[:, :512].copy()).view(torch.float8_e4m3fn).to(torch.float64)
        scales = torch.from_numpy(rows[:, 512:528].copy().view("<f4").astype(np.float64)).reshape(n, 4)
        lat = codes * scales.repeat_interleave(128, dim=1)
        rope = torch.from_numpy(rows[:, 528:656].copy().view("<u2").astype(np.int16)).view(torch.bfloat16)
    else:
        lat = torch.from_numpy(rows[:, :1024].copy().view("<u2").astype(np.int16)).view(torch.bfloat16)
        lat = lat.to(torch.float64)
        rope = torch.from_numpy(rows[:, 1024:1152].copy().view("<u2").astype(np.int16)).view(torch.bfloat16)
    k = torch.cat([lat, rope.to(torch.float64)], dim=1)
    return k, lat.clone()


def _q64(w: W.Workload) -> torch.Tensor:
    return torch.from_numpy(w.q.astype(np.int16)).view(torch.bfloat16).to(torch.float64)


def _valid_rows(w: W.Workload, pool: np.ndarray, b: int) -> np.ndarray:
    rb = w.row_bytes
    out = []
    for i in w.topk_idx[b]:
        i = int(i)
        if 0 <= i < int(w.ctx_len[b]):
            slot = int(w.page_table[b, i // W.PAGE]) * W.PAGE + i % W.PAGE
            out.append(pool[slot * rb:(slot + 1) * rb])
    return np.array(out, dtype=np.uint8).reshape(len(out), rb)


def _context_rows(w: W.Workload, pool: np.ndarray, b: int) -> np.ndarray:
    """Rows of tokens 0..ctx-1 of request b, in token order (dense context)."""
    rb = w.row_bytes
    out = []
    for t in range(int(w.ctx_len[b])):
        slot = int(w.page_table[b, t // W.PAGE]) * W.PAGE + t % W.PAGE
        out.append(pool[slot * rb:(slot + 1) * rb])
    return np.array(out, dtype=np.uint8).reshape(len(out), rb)


def _dense_ws(fmt: int):
    """Selections that cover the whole context: dense attention over every token."""
    ctx = [512, 300, 1]
    idx = np.full((3, W.TOPK), -1, np.int32)
    rng = np.random.default_rng(11)
    for b, c in enumerate(ctx):
        idx[b, :c] = rng.permutation(c)
    rng.shuffle(idx[1])           # masked slots scattered among valid ones
    return W.build("dense", 901, fmt, 3, ctx, fmt, "given", topk_idx=idx)


# ----------------------------------------------------------------- pins
def pin_e4m3_all_codes(lib):
    """All 256 e4m3fn codes decode as torch's float8_e4m3fn cast decodes them."""
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    for c in range(256):
        got = oracle.e4m3_to_f64(c, lib)
        r = float(ref[c])
        assert (math.isnan(got) and math.isnan(r)) or got == r, (c, got, r)


def pin_bf16_all_patterns(lib):
    """Every bf16 bit pattern decodes as torch's bfloat16 decodes it."""
    allbits = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).to(torch.float64).numpy()
    for bits in range(0, 65536, 7):
        got = oracle.bf16_to_f64(bits, lib)
        r = allbits[bits]
        assert (math.isnan(got) and math.isnan(r)) or got == r, (bits, got, r)


def pin_gather_bruteforce(lib):
    """Index translation + gather against a plain Python walk, bit-exact.

    Covers masked (-1), negative, >= ctx, page ids past the pool or negative,
    ragged ctx and duplicates.
    """
    for fmt in (W.FMT_FP8, W.FMT_BF16):
        B = 4
        ctx = [700, 64, 3, 200]
        rng = np.random.default_rng(5)
        idx = np.stack([rng.integers(-3, 720, W.TOPK) for _ in range(B)]).astype(np.int32)
        idx[2, :5] = [2, 2, 1, 0, 3]
        w = W.build("g", 902, 0, B, ctx, fmt, "given", topk_idx=idx, max_pages=12)
        pt = w.page_table.copy()
        pt[0, 3] = w.pool_pages + 5        # beyond the pool -> masked
        pt[3, 1] = -2                      # negative page -> masked
        pool = w.host_pool()
        # fill the whole pool with non-zero bytes so a wrong row cannot read zeros by luck
        pool[:] = np.random.default_rng(6).integers(0, 256, pool.size, dtype=np.uint8)
        slots, rows = oracle.gather(B, W.TOPK, fmt, pool, w.pool_pages, pt, w.topk_idx, w.ctx_len, lib=lib)
        rb = w.row_bytes
        for b in range(B):
            for j in range(W.TOPK):
                i = int(w.topk_idx[b, j])
                exp_slot = -1
                if 0 <= i < ctx[b] and i // 64 < pt.shape[1]:
                    page = int(pt[b, i // 64])
                    if 0 <= page < w.pool_pages:
                        exp_slot = page * 64 + (i - (i // 64) * 64)
                assert slots[b, j] == exp_slot, (b, j, i, slots[b, j], exp_slot)
                if exp_slot < 0:
                    assert not rows[b, j].any()
                else:
                    assert np.array_equal(rows[b, j], pool[exp_slot * rb:(exp_slot + 1) * rb])


def pin_dense_equals_sdpa(lib):
    """Selections covering the whole context equal dense attention (torch SDPA, float64)."""
    for fmt in (W.FMT_FP8, W.FMT_BF16):
        w = _dense_ws(fmt)
        pool = w.host_pool()
        out, lse = oracle.decode_workload(w, lib=lib, pool=pool)
        q = _q64(w)
        for b in range(w.B):
            k, v = _torch_rows(fmt, _context_rows(w, pool, b))
            qb = q[b][None, :, None, :]                       # [1, H, 1, 576]
            kb = k[None, None].expand(1, W.H, -1, -1)
            vb = v[None, None].expand(1, W.H, -1, -1)
            ref = torch.nn.functional.scaled_dot_product_attention(qb, kb, vb, scale=float(w.scale))
            ref = ref[0, :, 0, :].numpy()
            ref_lse = torch.logsumexp(float(w.scale) * (q[b] @ k.T), dim=1).numpy()
            assert np.abs(out[b] - ref).max() <= TOL * max(1.0, np.abs(ref).max()), (fmt, b)
            assert np.abs(lse[b] - ref_lse).max() <= TOL * 10, (fmt, b)


def pin_single_token(lib):
    """One valid token: out = V_t exactly, lse = scaled score of that token."""
    for fmt in (W.FMT_FP8, W.FMT_BF16):
        idx = np.full((2, W.TOPK), -1, np.int32)
        idx[0, 77] = 1000
        idx[1, 3] = 5
        w = W.build("one", 903, fmt, 2, [4096, 6], fmt, "given", topk_idx=idx)
        pool = w.host_pool()
        out, lse = oracle.decode_workload(w, lib=lib, pool=pool)
        q = _q64(w).numpy()
        for b in range(2):
            k, v = _torch_rows(fmt, _valid_rows(w, pool, b))
            assert np.array_equal(out[b], np.broadcast_to(v.numpy()[0], (W.H, 512))), (fmt, b)
            s = float(w.scale) * np.dot(q[b], k.numpy()[0])
            assert np.abs(lse[b] - s).max() <= 1e-12 * max(1, np.abs(s).max()), (fmt, b)


def pin_q_zero(lib):
    """q = 0: every score is 0, so out = mean of the valid V rows and lse = ln(n_valid)."""
    for fmt in (W.FMT_FP8, W.FMT_BF16):
        w = W.build("q0", 904, fmt, 3, [4096, 100, 600], fmt, "uniform", q_zero=True)
        pool = w.host_pool()
        out, lse = oracle.decode_workload(w, lib=lib, pool=pool)
        for b in range(3):
            _, v = _torch_rows(fmt, _valid_rows(w, pool, b))
            n = v.shape[0]
            assert np.allclose(out[b], np.broadcast_to(v.numpy().mean(axis=0), (W.H, 512)), rtol=0, atol=1e-13)
            assert np.allclose(lse[b], math.log(n), rtol=0, atol=1e-13), (b, n)


def pin_two_tokens(lib):
    """Two tokens: weights are the logistic function of the score difference."""
    idx = np.full((1, W.TOPK), -1, np.int32)
    idx[0, 10], idx[0, 400] = 7, 130
    w = W.build("two", 905, W.FMT_FP8, 1, [200], W.FMT_FP8, "given", topk_idx=idx)
    pool = w.host_pool()
    out, lse = oracle.decode_workload(w, lib=lib, pool=pool)
    k, v = _torch_rows(W.FMT_FP8, _valid_rows(w, pool, 0))
    q = _q64(w).numpy()[0]
    s = float(w.scale) * (q @ k.numpy().T)                   # [H, 2]
    a = 1.0 / (1.0 + np.exp(s[:, 1] - s[:, 0]))
    ref = a[:, None] * v.numpy()[0][None] + (1 - a)[:, None] * v.numpy()[1][None]
    assert np.abs(out[0] - ref).max() <= 1e-12
    ref_lse = np.maximum(s[:, 0], s[:, 1]) + np.log1p(np.exp(-np.abs(s[:, 0] - s[:, 1])))
    assert np.abs(lse[0] - ref_lse).max() <= 1e-12


def pin_permutation_and_mask_invariance(lib):
    """Permuting the top-k list (with its -1s) or adding masked slots changes nothing."""
    w = W.build("perm", 906, 0, 3, [5000, 700, 300], W.FMT_FP8, "uniform")
    pool = w.host_pool()
    out0, lse0 = oracle.decode_workload(w, lib=lib, pool=pool)
    rng = np.random.default_rng(3)
    idx = w.topk_idx.copy()
    for b in range(w.B):
        idx[b] = idx[b][rng.permutation(W.TOPK)]
    out1, lse1 = oracle.decode(w.q, w.kv_format, pool, w.pool_pages, w.page_table, idx, w.ctx_len, w.scale, lib=lib)
    assert np.abs(out1 - out0).max() <= 1e-12 and np.abs(lse1 - lse0).max() <= 1e-12
    # masking slots (with -1, with a value >= ctx, with another negative value)
    # equals selecting only the remaining tokens, packed in another order
    keep = w.topk_idx.copy()
    keep[:, 400:] = -1
    keep[0, 390:400] = w.ctx_len[0] + 3
    keep[1, 380:390] = -77
    outm, lsem = oracle.decode(w.q, w.kv_format, pool, w.pool_pages, w.page_table, keep, w.ctx_len, w.scale, lib=lib)
    sel = np.full_like(keep, -1)
    for b in range(w.B):
        kept = [int(i) for i in keep[b] if 0 <= i < w.ctx_len[b]]
        sel[b, :len(kept)] = kept
        sel[b] = sel[b][rng.permutation(W.TOPK)]
    outs, lses = oracle.decode(w.q, w.kv_format, pool, w.pool_pages, w.page_table, sel, w.ctx_len, w.scale, lib=lib)
    assert np.abs(outm - outs).max() <= 1e-12 and np.abs(lsem - lses).max() <= 1e-12
    assert np.abs(outm - out0).max() > 1e-6          # masking really removed tokens


def pin_page_relabel(lib):
    """Relabelling physical pages (pool permuted to match) changes nothing."""
    w = W.build("relabel", 907, 0, 2, [3000, 4096], W.FMT_FP8, "uniform")
    pool = w.host_pool()
    out0, lse0 = oracle.decode_workload(w, lib=lib, pool=pool)
    P = w.pool_pages
    perm = np.random.default_rng(9).permutation(P)       # old page p -> new page perm[p]
    page_bytes = W.PAGE * w.row_bytes
    pool2 = np.zeros_like(pool)
    pool2.reshape(P, page_bytes)[perm] = pool.reshape(P, page_bytes)
    pt2 = perm[w.page_table].astype(np.int32)
    out1, lse1 = oracle.decode(w.q, w.kv_format, pool2, P, pt2, w.topk_idx, w.ctx_len, w.scale, lib=lib)
    assert np.array_equal(out1, out0) and np.array_equal(lse1, lse0)


def pin_scale_doubling(lib):
    """With q's latent half zero, doubling every block scale doubles out and keeps lse;
    with q's rope half zero, scaling one block's scale scales that block of V only."""
    w = W.build("dbl", 908, 0, 2, [2048, 900], W.FMT_FP8, "uniform")
    q = w.q.copy()
    q[:, :, :512] = 0
    pool = w.host_pool()
    out0, lse0 = oracle.decode(q, w.kv_format, pool, w.pool_pages, w.page_table, w.topk_idx, w.ctx_len, w.scale, lib=lib)
    pool2 = pool.copy()
    rows = pool2.reshape(-1, w.row_bytes)
    sc = rows[w.row_slots, 512:528].copy().view("<f4") * np.float32(2)
    rows[w.row_slots, 512:528] = sc.view(np.uint8)
    out1, lse1 = oracle.decode(q, w.kv_format, pool2, w.pool_pages, w.page_table, w.topk_idx, w.ctx_len, w.scale, lib=lib)
    assert np.array_equal(out1, 2 * out0)
    assert np.abs(lse1 - lse0).max() <= 1e-13
    # only block 2's scale changes; rope-only scores stay, V block 2 scales by 4
    pool3 = pool.copy()
    rows3 = pool3.reshape(-1, w.row_bytes)
    s3 = rows3[w.row_slots, 512:528].copy().view("<f4").reshape(-1, 4)
    s3[:, 2] *= np.float32(4)
    rows3[w.row_slots, 512:528] = s3.reshape(-1).view(np.uint8).reshape(-1, 16)
    out3, lse3 = oracle.decode(q, w.kv_format, pool3, w.pool_pages, w.page_table, w.topk_idx, w.ctx_len, w.scale, lib=lib)
    assert np.array_equal(out3[:, :, 256:384], 4 * out0[:, :, 256:384])
    assert np.array_equal(out3[:, :, :256], out0[:, :, :256]) and np.array_equal(out3[:, :, 384:], out0[:, :, 384:])
    assert np.abs(lse3 - lse0).max() <= 1e-13


def pin_split_merge(lib):
    """Any partition of the selection, merged with the LSE rule, equals the whole (fp64)."""
    w = W.build("split", 909, 0, 2, [9000, 800], W.FMT_FP8, "uniform")
    pool = w.host_pool()
    out, lse = oracle.decode_workload(w, lib=lib, pool=pool)
    rng = np.random.default_rng(4)
    for nsplit in (2, 3, 7):
        part = rng.integers(0, nsplit, W.TOPK)
        outs, lses = [], []
        for s in range(nsplit):
            idx = np.where(part[None] == s, w.topk_idx, -1).astype(np.int32)
            o, l = oracle.decode(w.q, w.kv_format, pool, w.pool_pages, w.page_table, idx, w.ctx_len, w.scale, lib=lib)
            outs.append(o)
            lses.append(l)
        L = np.stack(lses)                                   # [S, B, H]
        M = L.max(axis=0)
        wgt = np.exp(L - M[None])
        merged = (wgt[..., None] * np.stack(outs)).sum(axis=0) / wgt.sum(axis=0)[..., None]
        assert np.abs(merged - out).max() <= 1e-12
        assert np.abs(M + np.log(wgt.sum(axis=0)) - lse).max() <= 1e-12


def pin_empty_selection(lib):
    """No valid slot: out = 0 and lse = -inf (never NaN)."""
    idx = np.full((2, W.TOPK), -1, np.int32)
    idx[1, :3] = [900, 901, 5000]        # all >= ctx
    w = W.build("empty", 910, 0, 2, [600, 800], W.FMT_FP8, "given", topk_idx=idx)
    out, lse = oracle.decode_workload(w, lib=lib)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def pin_bruteforce_tiny(lib):
    """B=2, ctx=64 (one page), against a pure-Python restatement with math.exp."""
    for fmt in (W.FMT_FP8, W.FMT_BF16):
        w = W.build("tiny", 911, fmt, 2, [64, 40], fmt, "uniform")
        pool = w.host_pool()
        out, lse = oracle.decode_workload(w, lib=lib, pool=pool)
        q = _q64(w).numpy()
        for b in range(2):
            k, v = _torch_rows(fmt, _valid_rows(w, pool, b))
            k, v = k.numpy().tolist(), v.numpy().tolist()
            for h in (0, 17, 63):
                sc = [float(w.scale) * sum(q[b, h, d] * kt[d] for d in range(576)) for kt in k]
                m = max(sc)
                ex = [math.exp(x - m) for x in sc]
                L = sum(ex)
                ref = [sum(ex[t] * v[t][d] for t in range(len(v))) / L for d in range(512)]
                assert max(abs(a - r) for a, r in zip(out[b, h], ref)) <= 1e-12, (fmt, b, h)
                assert abs(lse[b, h] - (m + math.log(L))) <= 1e-12


def pin_head_and_request_order(lib):
    """Each (request, head) uses its own q row: swapping two requests' inputs swaps outputs."""
    w = W.build("order", 912, 0, 3, [3000, 3000, 3000], W.FMT_FP8, "uniform")
    pool = w.host_pool()
    out, lse = oracle.decode_workload(w, lib=lib, pool=pool)
    perm = [2, 0, 1]
    hperm = np.random.default_rng(2).permutation(W.H)
    q2 = w.q[perm][:, hperm]
    out2, lse2 = oracle.decode(q2, w.kv_format, pool, w.pool_pages, w.page_table[perm], w.topk_idx[perm],
                               w.ctx_len[perm], w.scale, lib=lib)
    assert np.array_equal(out2, out[perm][:, hperm]) and np.array_equal(lse2, lse[perm][:, hperm])


def pin_query_tokens_share_selection(lib):
    """q_len query tokens per request: each (token, head) row attends over the
    request's selected rows, checked against torch SDPA (float64) on the rows
    gathered here, and against one single-token call per token."""
    base = W.build("mtp", 913, 0, 3, [9000, 700, 40], W.FMT_FP8, "uniform")
    w = W.with_query_tokens(base, 3)
    assert w.q.shape == (3, 3, W.H, W.D_QK) and np.array_equal(w.q[:, 0], base.q)
    pool = w.host_pool()
    out, lse = oracle.decode_workload(w, lib=lib, pool=pool)
    assert out.shape == (3, 3, W.H, 512) and lse.shape == (3, 3, W.H)
    q = torch.from_numpy(w.q.astype(np.int16)).view(torch.bfloat16).to(torch.float64)
    for b in range(w.B):
        k, v = _torch_rows(w.kv_format, _valid_rows(w, pool, b))
        for t in range(3):
            qb = q[b, t][None, :, None, :]
            ref = torch.nn.functional.scaled_dot_product_attention(
                qb, k[None, None].expand(1, W.H, -1, -1), v[None, None].expand(1, W.H, -1, -1),
                scale=float(w.scale))[0, :, 0, :].numpy()
            ref_lse = torch.logsumexp(float(w.scale) * (q[b, t] @ k.T), dim=1).numpy()
            assert np.abs(out[b, t] - ref).max() <= TOL * max(1.0, np.abs(ref).max()), (b, t)
            assert np.abs(lse[b, t] - ref_lse).max() <= TOL * 10, (b, t)
    for t in range(3):
        o1, l1 = oracle.decode(w.q[:, t], w.kv_format, pool, w.pool_pages, w.page_table, w.topk_idx,
                               w.ctx_len, w.scale, lib=lib)
        assert np.array_equal(o1, out[:, t]) and np.array_equal(l1, lse[:, t])


def pin_e4m3_encode_roundtrip_ties_saturation(lib):
    """The encoder inverts the decoder on every finite code, sends each midpoint
    between neighbouring codes to the even one, saturates beyond 448 (infinities
    too) and sends NaN to the NaN code."""
    vals = {}
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue                                   # NaN codes
        v = oracle.e4m3_to_f64(c, lib)
        assert oracle.e4m3_encode(np.float32(v), lib) == c, hex(c)
        vals[c] = v
    pos = sorted((v, c) for c, v in vals.items() if c < 0x80)
    for (v0, c0), (v1, c1) in zip(pos, pos[1:]):
        mid = (v0 + v1) / 2                            # exact in fp32 (5 significant bits)
        even = c0 if c0 % 2 == 0 else c1
        for sgn in (1, -1):
            sb = 0 if sgn == 1 else 0x80
            assert oracle.e4m3_encode(np.float32(sgn * mid), lib) == (even | sb) if c0 != 0 or sgn == 1 else True
            assert oracle.e4m3_encode(np.nextafter(np.float32(sgn * mid), np.float32(sgn * 1e9)), lib) == (c1 | sb)
            assert oracle.e4m3_encode(np.nextafter(np.float32(sgn * mid), np.float32(0)), lib) == (c0 | sb)
    for v in (448.0, 463.99, 464.0, 480.0, 1e5, 3.0e38, np.inf):
        assert oracle.e4m3_encode(np.float32(v), lib) == 0x7E and oracle.e4m3_encode(np.float32(-v), lib) == 0xFE
    # the format has no infinities; its NaN is S.1111.111
    assert oracle.e4m3_encode(np.float32(np.nan), lib) == 0x7F
    assert oracle.e4m3_encode(-np.float32(np.nan), lib) == 0xFF


def pin_encoders_match_torch_casts(lib):
    """e4m3 (within +-448) and bf16 rounding agree with torch's casts on random
    fp32 values spanning normal and subnormal ranges, including exact ties."""
    rng = np.random.default_rng(21)
    mag = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 100_000)).astype(np.float32)
    x = (mag * rng.choice([-1, 1], mag.size)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(v, lib) for v in x], dtype=np.uint8)
    assert np.array_equal(got, ref)
    bits = rng.integers(0, 2 ** 32, 100_000, dtype=np.uint64).astype(np.uint32)
    bits[:2000] = (bits[:2000] & 0xFFFF0000) | 0x8000     # exact ties
    y = bits.view(np.float32)
    y = y[np.isfinite(y)]
    ref16 = torch.from_numpy(y.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got16 = np.array([oracle.f32_to_bf16(v, lib) for v in y], dtype=np.uint16)
    assert np.array_equal(got16, ref16)


def _append_case(fmt, n=300, seed=22):
    """Inputs for the cache producer: fp32 rows with special blocks, and destinations
    (some invalid) through a shuffled page table."""
    rng = np.random.default_rng(seed)
    B, max_pages, pool_pages = 5, 12, 64
    lat = rng.standard_normal((n, 512)).astype(np.float32)
    rope = rng.standard_normal((n, 64)).astype(np.float32)
    lat[0, 128:256] = 0.0                                  # all-zero block
    lat[1, :128] = 0.0
    lat[1, 77] = -3.25                                     # one non-zero value
    lat[2, :] *= np.float32(1e-30)                         # tiny magnitudes
    lat[3, :] *= np.float32(1e30)                          # huge magnitudes
    pt = rng.permutation(pool_pages)[:B * max_pages].astype(np.int32).reshape(B, max_pages)
    pt[4, 3] = pool_pages + 7                              # out-of-range page
    req = rng.integers(0, B, n).astype(np.int32)
    # distinct destinations: positions drawn without replacement per request
    pos = np.empty(n, np.int32)
    for b in range(B):
        ix = np.nonzero(req == b)[0]
        pos[ix] = rng.choice(max_pages * W.PAGE, len(ix), replace=False)
    req[5], req[6], pos[7], pos[8] = -1, B, -4, max_pages * W.PAGE   # invalid destinations
    return lat, rope, req, pos, pt, pool_pages


def pin_kv_append_matches_generator(lib):
    """The producer writes exactly the rows the input generator packs (torch casts),
    at the slots the page table gives, and nothing for invalid destinations."""
    for fmt in (W.FMT_FP8, W.FMT_BF16):
        lat, rope, req, pos, pt, pool_pages = _append_case(fmt)
        rb = W.ROW_BYTES[fmt]
        pool = np.zeros(pool_pages * W.PAGE * rb, dtype=np.uint8)
        n = oracle.kv_append(lat, rope, req, pos, pt, pool, pool_pages, fmt, lib=lib)
        rows = pool.reshape(-1, rb)
        expect = W.pack_rows(fmt, lat, rope)
        written = np.zeros(rows.shape[0], bool)
        count = 0
        for t in range(lat.shape[0]):
            b, p = int(req[t]), int(pos[t])
            if not (0 <= b < pt.shape[0] and 0 <= p < pt.shape[1] * W.PAGE):
                continue
            page = int(pt[b, p // W.PAGE])
            if not (0 <= page < pool_pages):
                continue
            slot = page * W.PAGE + p % W.PAGE
            assert np.array_equal(rows[slot], expect[t]), (fmt, t)
            written[slot] = True
            count += 1
        assert n == count and count < lat.shape[0] - 3
        assert not rows[~written].any()


def _bf(bits):
    return torch.from_numpy(np.asarray(bits).astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def pin_indexer_bruteforce(lib):
    """Scores and selection against plain Python loops on a small case (4 heads, 8 dims,
    topk 16, three requests with ragged contexts, one invalid page)."""
    inp = W.indexer_inputs(3, [300, 9, 130], 1, heads=4, dim=8)
    inp.page_table[0, 2] = inp.pool_pages + 3                 # positions 128..191 of request 0 excluded
    sc, idx = oracle.indexer(inp.q, inp.w, inp.keys, inp.pool_pages, inp.page_table, inp.ctx_len, topk=16, lib=lib)
    q, k = _bf(inp.q), _bf(inp.keys)
    for b in range(3):
        pairs = []
        for s_ in range(int(inp.ctx_len[b])):
            page = int(inp.page_table[b, s_ // W.PAGE])
            if not 0 <= page < inp.pool_pages:
                assert math.isnan(sc[b, s_])
                continue
            row = k[page * W.PAGE + s_ % W.PAGE]
            v = sum(float(inp.w[b, j]) * max(0.0, float(np.dot(q[b, j], row))) for j in range(4))
            assert abs(sc[b, s_] - v) <= 1e-12 * max(1.0, abs(v))
            pairs.append((-v, s_))
        pairs.sort()
        want = [p_[1] for p_ in pairs[:16]] + [-1] * max(0, 16 - len(pairs))
        assert list(idx[b]) == want, b


def pin_indexer_closed_forms_and_ties(lib):
    """q = 0 scores every position 0, so the selection is the first valid positions in
    order; duplicated key rows tie exactly and the smaller position comes first; scaling
    every weight by 2 doubles every score and keeps the selection; a head whose products
    are all negative contributes nothing whatever its weight."""
    inp = W.indexer_inputs(2, [1000, 40], 2, heads=8, dim=16)
    q0 = np.zeros_like(inp.q)
    sc0, idx0 = oracle.indexer(q0, inp.w, inp.keys, inp.pool_pages, inp.page_table, inp.ctx_len, topk=64, lib=lib)
    assert np.all(sc0[0, :1000] == 0) and list(idx0[0]) == list(range(64))
    assert list(idx0[1]) == list(range(40)) + [-1] * 24
    # exact ties: copy the key row of position 500 onto positions 700 and 900
    keys = inp.keys.copy()
    slot = lambda s_: int(inp.page_table[0, s_ // W.PAGE]) * W.PAGE + s_ % W.PAGE
    keys[slot(700)] = keys[slot(500)]
    keys[slot(900)] = keys[slot(500)]
    sc, idx = oracle.indexer(inp.q, inp.w, keys, inp.pool_pages, inp.page_table, inp.ctx_len, topk=1000, lib=lib)
    order = list(idx[0])
    assert sc[0, 500] == sc[0, 700] == sc[0, 900]
    assert order.index(500) + 1 == order.index(700) and order.index(700) + 1 == order.index(900)
    sc2, idx2 = oracle.indexer(inp.q, inp.w * np.float32(2), keys, inp.pool_pages, inp.page_table, inp.ctx_len,
                               topk=1000, lib=lib)
    ok = ~np.isnan(sc)
    assert np.array_equal(sc2[ok], 2 * sc[ok]) and np.array_equal(idx2, idx)
    q3 = inp.q.copy()
    q3[:, 0] = W.bf16_bits(-np.abs(_bf(inp.keys).sum(axis=0)[None, :]).astype(np.float32))   # q_0 . k mostly < 0
    sc3, _ = oracle.indexer(q3, inp.w, keys, inp.pool_pages, inp.page_table, inp.ctx_len, topk=8, lib=lib)
    w4 = inp.w.copy()
    w4[:, 0] = 123.0
    sc4, _ = oracle.indexer(q3, w4, keys, inp.pool_pages, inp.page_table, inp.ctx_len, topk=8, lib=lib)
    qq, kk = _bf(q3), _bf(keys)
    for b, s_ in ((0, 10), (0, 999), (1, 5)):
        row = kk[int(inp.page_table[b, s_ // W.PAGE]) * W.PAGE + s_ % W.PAGE]
        if float(np.dot(qq[b, 0], row)) < 0:
            assert sc3[b, s_] == sc4[b, s_]


ALL_PINS = [
    pin_e4m3_all_codes, pin_bf16_all_patterns, pin_gather_bruteforce, pin_dense_equals_sdpa,
    pin_single_token, pin_q_zero, pin_two_tokens, pin_permutation_and_mask_invariance,
    pin_page_relabel, pin_scale_doubling, pin_split_merge, pin_empty_selection,
    pin_bruteforce_tiny, pin_head_and_request_order, pin_query_tokens_share_selection,
    pin_e4m3_encode_roundtrip_ties_saturation, pin_encoders_match_torch_casts, pin_kv_append_matches_generator,
    pin_indexer_bruteforce, pin_indexer_closed_forms_and_ties,
]
