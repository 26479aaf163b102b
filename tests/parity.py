"""The parity gate between the HIP path and the oracle.

Readings (where the pages give only the number 6.7e-3 for their built-in
relative-error check): per (request, head), the largest absolute error over the
512 output dims divided by the largest magnitude of the oracle's output row
must be <= 6.7e-3; lse must agree to 6.7e-3 in absolute terms (an lse error d
is a relative error exp(d) - 1 ~ d of the softmax normaliser).  A row whose
oracle output is exactly zero (no selected token) must be exactly zero with
lse = -inf.
"""
from __future__ import annotations

import json
import os

import numpy as np

TOL = 6.7e-3


def compare(out, lse, ref_o, ref_l):
    """(max row-relative error of out, max |lse - ref|, n rows checked)."""
    o = out.detach().float().cpu().numpy().astype(np.float64) if hasattr(out, "detach") else np.asarray(out, np.float64)
    l = lse.detach().float().cpu().numpy().astype(np.float64) if hasattr(lse, "detach") else np.asarray(lse, np.float64)
    assert np.all(np.isfinite(o)), "non-finite output"
    denom = np.abs(ref_o).max(axis=-1)
    err = np.abs(o - ref_o).max(axis=-1)
    empty = denom == 0
    assert np.all(err[empty] == 0), "masked-out row is not exactly zero"
    rel = np.where(empty, 0.0, err / np.where(empty, 1.0, denom))
    fin = np.isfinite(ref_l)
    assert np.all(np.isneginf(l[~fin])), "empty row lse is not -inf"
    assert np.all(np.isfinite(l[fin])), "non-finite lse"
    dl = np.abs(l[fin] - ref_l[fin]).max() if fin.any() else 0.0
    return float(rel.max()) if rel.size else 0.0, float(dl), int(rel.size)


def assert_parity(out, lse, ref_o, ref_l, what=""):
    rel, dl, n = compare(out, lse, ref_o, ref_l)
    print(f"[parity] {what}: rows={n} max_rel={rel:.3e} max_dlse={dl:.3e}", flush=True)
    log = os.environ.get("SMLA_PARITY_LOG")
    if log:
        with open(log, "a") as f:
            f.write(json.dumps({"case": what, "rows": n, "max_rel": rel, "max_dlse": dl}) + "\n")
    assert rel <= TOL, f"{what}: relative error {rel:.3e} > {TOL}"
    assert dl <= TOL, f"{what}: lse error {dl:.3e} > {TOL}"
    return rel, dl
