"""Non-finite inputs propagate as the recurrence's definition makes them, through tiles,
the slot scan and the look-back.

Under E_t = s_t E_{t-1} + B_t (page "entangled-state-attention 0.1.0", "Core idea") a NaN
gate or value at step t0 makes its lane NaN from t0 on (0 * NaN is NaN); a NaN query
poisons only that readout, and in the backward every gradient of its head at and before
t0.  A logit of +inf gives the gate 1 exactly and -inf the gate 0 exactly (the complement
1 / (1 + e^a) is 0 and 1).  The oracle follows the same definition in fp64, so NaN positions must agree
exactly and the finite values within the parity bar.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from gated_linear_recurrence_chunked_amd import binding, synth
from helpers import FLOOR, TOL, err, f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MODES = {"direct": 0, "controlled": 1}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def same_nan_then_close(name, got, ref, dtype):
    g, r = f64(got), f64(ref)
    gn, rn = np.isnan(g), np.isnan(r)
    assert np.array_equal(gn, rn), f"{name}: NaN pattern differs ({gn.sum()} vs {rn.sum()})"
    fin = ~rn
    assert np.array_equal(np.isinf(g[fin]), np.isinf(r[fin])), f"{name}: inf pattern differs"
    ok = fin & np.isfinite(r)
    e = err(g[ok], r[ok], FLOOR.get(dtype, 0.0))
    print(f"  {name}: {rn.sum()} NaN, err {e:.3e} on the rest", flush=True)
    assert e <= TOL[dtype], f"{name}: err {e:.3e}"


CASES = {
    # tensor, value, positions (b, t, h, d)
    "nan_gate": ("a", float("nan"), [(0, 700, 1, 5), (1, 40, 0, 63)]),
    "nan_value": ("v", float("nan"), [(1, 1999, 1, 0), (0, 3, 0, 17)]),
    "nan_query": ("q", float("nan"), [(0, 1234, 1, 9)]),
    "inf_gates": ("a", float("inf"), [(0, 100, 0, 1), (0, 101, 0, 1), (1, 900, 1, 30)]),
    "neg_inf_gates": ("a", float("-inf"), [(0, 600, 1, 2), (1, 1500, 0, 40)]),
}


@pytest.mark.parametrize("case", list(CASES))
# One-byte storage takes its gates from a table of the 256 codes, whose NaN (and E5M2
# infinity) codes must give what the gate gives in place.  E4M3 has no infinity: an infinite
# logit is stored as NaN, and the oracle reads the same stored codes.
@pytest.mark.parametrize("dt,mode", [(torch.float16, "controlled"), (torch.float32, "direct"),
                                     (torch.float8_e4m3fn, "controlled"),
                                     (torch.float8_e5m2, "direct")])
def test_nonfinite_inputs_follow_the_definition(case, dt, mode):
    B, T, H, Dh = 2, 2000, 2, 64  # 8 forward and 16 backward tiles per channel block
    say(f"non-finite {case} {dt} {mode}")
    shp = (B, T, H, Dh)
    x = {k: synth.normal(shp, 50 + i, 0.5 if k == "a" else 0.0, 1.0, dt)
         for i, k in enumerate(("a", "v", "q", "dy"))}
    name, val, pos = CASES[case]
    for p in pos:
        x[name][p] = val
    e0 = synth.random_state(B, H, Dh, 59)
    g = {k: t.to(DEV) for k, t in x.items()}
    y, eT, ck = binding.scan_fwd(g["a"], g["v"], g["q"], e0.to(DEV), mode=mode, return_ckpt=True)
    da, dv, dq, de0 = binding.scan_bwd(g["a"], g["v"], g["q"], g["dy"], e0.to(DEV), None,
                                       ckpt=ck, mode=mode)
    torch.cuda.synchronize()
    m = MODES[mode]
    ry, reT = oracle.scan_fwd(x["a"], x["v"], x["q"], e0, mode=m, threads=2)
    rda, rdv, rdq, rde0 = oracle.scan_bwd(x["a"], x["v"], x["q"], x["dy"], e0, None, mode=m,
                                          threads=2)
    state_dt = torch.float32  # the fp32 outputs of every storage meet the fp32 bar
    same_nan_then_close("y", y, ry, dt)
    same_nan_then_close("final_state", eT, reT, state_dt)
    same_nan_then_close("d_logit", da, rda, dt)
    same_nan_then_close("d_value", dv, rdv, dt)
    same_nan_then_close("d_query", dq, rdq, dt)
    same_nan_then_close("d_init", de0, rde0, state_dt)
    for ws in binding._workspaces.values():
        assert int(ws[12:16].view(torch.int32).item()) == 0, "look-back wait timed out"
