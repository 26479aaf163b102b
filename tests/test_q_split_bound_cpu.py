"""The fp8 hi + lo split of Q, as the decode kernel forms it, against the bound
its documentation states (CPU only; torch's float8_e4m3fn cast rounds to
nearest-even like the hardware conversion).

Per head, Q is scaled by 2^e, the largest power of two with max|q| * 2^e <= 448,
so the scaled maximum lies in (224, 448].  hi = e4m3(x), lo = e4m3(x - hi).
hi + lo reproduces x exactly whenever the residual x - hi is itself an e4m3
value; a residual below the normal range (2^-6) is rounded to the 2^-9 step of
the subnormals, so the error is at most 2^-10 in the scaled domain, i.e. less
than 2^-10 / 224 = 4.36e-6 of the head's largest |q|."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch


def _exponent(amax: float) -> int:
    m, E = math.frexp(amax)          # amax = m * 2^E, m in [0.5, 1)
    return (9 - E) if m <= 0.875 else (8 - E)


def _split(x: torch.Tensor):
    hi = x.to(torch.float8_e4m3fn).to(torch.float32)
    lo = (x - hi).to(torch.float8_e4m3fn).to(torch.float32)
    return hi, lo


@pytest.mark.parametrize("amax", [1.0, 3.71875, 0.0009765625, 200.0, 447.0, 0.875, 0.87890625])
def test_hi_lo_split_error_bound(amax):
    # every non-negative bf16 value up to amax (the sign is symmetric)
    bits = np.arange(0, 0x7F80, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    v = v[v <= np.float32(amax)]
    ex = _exponent(float(np.float32(torch.tensor(amax).to(torch.bfloat16).float())))
    x = torch.from_numpy(v.copy()) * (2.0 ** ex)
    top = float(torch.tensor(amax).to(torch.bfloat16).float()) * 2.0 ** ex
    assert 224.0 < top <= 448.0
    hi, lo = _split(x)
    err = (hi + lo - x).abs()
    assert err.max().item() <= 2.0 ** -10
    assert (err / top).max().item() < 4.36e-6
    # exact wherever the residual is an e4m3 value (normal, or on the subnormal grid)
    r = x - hi
    representable = r == r.to(torch.float8_e4m3fn).to(torch.float32)
    assert torch.equal(err[representable], torch.zeros_like(err[representable]))
    # and the inexact ones are exactly the residuals off the 2^-9 subnormal grid
    assert bool(((r[~representable].abs() < 2.0 ** -6)).all())
