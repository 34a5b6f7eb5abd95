"""The oracle's reading of fp8 storage, pinned to the formats' definitions.

The oracle takes every input as the exact fp64 value of its stored code (oracle._f64).  For
the two OCP 8-bit formats of the experimental fp8 precision mode (page "Entangled State
Attention v2.1", section "3. Precision") that value is fixed by the format's fields: sign,
exponent bias 7 (E4M3) or 15 (E5M2), subnormals at the smallest exponent, no infinities and
a single NaN mantissa (all ones) in E4M3, IEEE-style infinities and NaNs in E5M2.  Each of the
256 codes is decoded here from those fields and compared with the oracle's conversion.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from helpers import FLOOR, TOL, err

FORMATS = {
    # name: (torch dtype, exponent bits, mantissa bits, bias, has infinities)
    "e4m3": (torch.float8_e4m3fn, 4, 3, 7, False),
    "e5m2": (torch.float8_e5m2, 5, 2, 15, True),
}


def decode(code: int, ebits: int, mbits: int, bias: int, ieee: bool) -> float:
    sign = -1.0 if code >> 7 else 1.0
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    emax = (1 << ebits) - 1
    if ieee and e == emax:
        return sign * math.inf if m == 0 else math.nan
    if not ieee and e == emax and m == (1 << mbits) - 1:
        return math.nan
    if e == 0:
        return sign * m * 2.0 ** (1 - bias - mbits)
    return sign * (1 + m / 2.0 ** mbits) * 2.0 ** (e - bias)


@pytest.mark.parametrize("name", list(FORMATS))
def test_every_code_decodes_by_definition(name):
    dt, eb, mb, bias, ieee = FORMATS[name]
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    got = oracle._f64(codes.view(dt))
    ref = np.array([decode(c, eb, mb, bias, ieee) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_format_extremes():
    e4 = [decode(c, 4, 3, 7, False) for c in range(128)]
    e5 = [decode(c, 5, 2, 15, True) for c in range(128)]
    assert max(x for x in e4 if not math.isnan(x)) == 448.0
    assert max(x for x in e5 if math.isfinite(x)) == 57344.0
    assert min(x for x in e4 if x > 0) == 2.0 ** -9
    assert min(x for x in e5 if x > 0) == 2.0 ** -16


@pytest.mark.parametrize("dt", [torch.float8_e4m3fn, torch.float8_e5m2])
def test_bar_covers_one_rounding_and_not_two_steps(dt):
    """The parity bar for fp8 outputs admits exactly one round-to-nearest of the true value:
    rounding N(0, 1) draws passes it, and an error of one whole step (as from a truncation or
    an off-by-one code) fails it."""
    g = torch.Generator().manual_seed(5)
    x = torch.randn(200000, generator=g, dtype=torch.float64)
    r = x.to(dt)
    assert err(r, x) <= TOL[dt]
    # one code up from the rounded value, on the elements where that is a full step
    up = (r.view(torch.uint8).to(torch.int32) + torch.where(r.double() >= 0, 1, -1))
    up = up.clamp(0, 255).to(torch.uint8).view(dt)
    fin = torch.isfinite(up.double())
    assert err(up.double()[fin], x[fin]) > TOL[dt]


@pytest.mark.parametrize("dt", [torch.float8_e4m3fn, torch.float8_e5m2])
def test_bar_covers_subnormal_rounding_and_not_a_subnormal_step(dt):
    """Below the smallest normal number the formats round to a fixed absolute step; with the
    scale floor of the fp8 bar (the smallest normal), one correct rounding of values that are
    all subnormal passes and an error of one subnormal step fails."""
    g = torch.Generator().manual_seed(6)
    tiny = FLOOR[dt] / 4  # draws mostly below the smallest normal
    x = torch.randn(200000, generator=g, dtype=torch.float64) * tiny
    r = x.to(dt)
    assert err(r, x, FLOOR[dt]) <= TOL[dt]
    assert err(r, x) > TOL[dt]  # the unfloored metric rejects correct rounding here
    up = (r.view(torch.uint8).to(torch.int32) + torch.where(r.double() >= 0, 1, -1))
    up = up.clamp(0, 255).to(torch.uint8).view(dt)
    fin = torch.isfinite(up.double())
    assert err(up.double()[fin], x[fin], FLOOR[dt]) > TOL[dt]
