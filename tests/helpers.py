"""Shared test helpers: the parity error metric and tolerances.

The error of a result x against the oracle's r is

    err = max_i |x_i - r_i| / max(|r_i|, rms(r))

an elementwise relative error wherever |r_i| >= rms(r), and an absolute error scaled by
rms(r) below it.  A pure elementwise ratio is undefined where r_i = 0 and unbounded near
it, and the states and gradients here are signed sums that cancel.  The bar is 1e-5 for
fp32 inputs, 5e-3 for fp16 / bf16 inputs and the format's rounding bound for fp8 inputs.
"""
import numpy as np
import torch

# fp8 storage: the outputs are rounded once to the 8-bit format, whose relative rounding
# error is at most 2^-4 (E4M3, 3 stored mantissa bits) or 2^-3 (E5M2, 2 bits) in the normal
# range; below it the rounding is absolute, at most half the subnormal step: 2^-10 for E4M3,
# 2^-17 for E5M2.  The fp32 arithmetic adds ~1e-6 on top.
TOL = {torch.float32: 1e-5, torch.float16: 5e-3, torch.bfloat16: 5e-3,
       torch.float8_e4m3fn: 2.0 ** -4 + 1e-4, torch.float8_e5m2: 2.0 ** -3 + 1e-4}
# The scale floor that makes the fp8 bar cover that absolute half step: the smallest normal
# number, 2^-6 (E4M3) and 2^-14 (E5M2), times the relative bar is the half step.  Without it
# an output whose every value is subnormal (a gate gradient s (1 - s) dE E of a retentive
# gate, say) fails on correct rounding alone.
FLOOR = {torch.float8_e4m3fn: 2.0 ** -6, torch.float8_e5m2: 2.0 ** -14}


def f64(x):
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def err(x, r, floor: float = 0.0) -> float:
    """The error above; `floor` (default 0) bounds the scale from below, for references whose
    every element is numerically zero (e.g. the gate gradient of a saturated gate: exactly 0
    in fp32, about 1e-44 in fp64)."""
    x = f64(x)
    r = f64(r)
    assert x.shape == r.shape, (x.shape, r.shape)
    if r.size == 0:
        return 0.0
    if not np.all(np.isfinite(x)):
        return float("inf")
    rms = float(np.sqrt(np.mean(r * r)))
    scale = np.maximum(np.maximum(np.abs(r), rms), floor)
    scale = np.where(scale > 0, scale, 1.0)
    return float(np.max(np.abs(x - r) / scale))


def assert_close(name, x, r, dtype, floor: float = 0.0):
    e = err(x, r, max(floor, FLOOR.get(dtype, 0.0)))
    tol = TOL[dtype]
    print(f"  {name}: err {e:.3e} (bar {tol:.0e})", flush=True)
    assert e <= tol, f"{name}: err {e:.3e} > tol {tol:.0e}"
    return e
