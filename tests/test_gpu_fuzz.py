"""Seeded random cases over every argument the scans take, against the oracle.

Each case draws B, T, H, Dh, the storage dtype, the mode, the deterministic flag, whether an
initial state and an upstream state gradient are given, and the logit distribution, then
runs the forward (with checkpoint) and the backward through the library and compares every
output with the oracle.  The cases are fixed by their seeds, so a failure names its case.
"""
import random
import sys

import pytest
import torch

import oracle
from gated_linear_recurrence_chunked_amd import binding, synth
from helpers import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
DTYPES = [torch.float32, torch.float16, torch.bfloat16, torch.float8_e4m3fn, torch.float8_e5m2]
FP8 = (torch.float8_e4m3fn, torch.float8_e5m2)


def case_of(seed):
    r = random.Random(seed)
    Dh = r.choice([16, 32, 64, 128])
    H = r.choice([1, 2, 3, 4])
    B = r.choice([1, 2, 3, 5, 8])
    T = r.choice([1, 2, 63, 64, 65, r.randint(3, 700), r.randint(700, 2600)])
    while B * T * H * Dh > 3_000_000:
        T = max(1, T // 2)
    return dict(B=B, T=T, H=H, Dh=Dh, dtype=r.choice(DTYPES), mode=r.choice(["direct", "controlled"]),
                det=r.random() < 0.3, e0=r.random() < 0.5, dET=r.random() < 0.5,
                a_mean=r.choice([-2.0, 0.0, 0.5, 2.0, 4.0]), a_std=r.choice([0.5, 1.0, 3.0]))


def retentive_case_of(seed):
    """Long-memory gates, mean logit 6 or 8 (about 400 or 3000 steps of memory), for every
    storage dtype, fp32 included."""
    c = case_of(10_000 + seed)
    c["a_mean"] = random.Random(seed).choice([6.0, 8.0])
    c["a_std"] = random.Random(seed + 1).choice([0.5, 1.0, 2.0])
    return c


@pytest.mark.parametrize("seed", range(160))
def test_random_case(seed):
    run_case(seed, case_of(seed))


# fp16, Dh = 64 sizes in the forward's tile table (256-thread workgroups), with random draws
TABLE_CASES = [(1, 700, 8), (4, 512, 8), (4, 333, 8), (1, 2000, 8), (16, 1024, 32), (2, 900, 16)]


@pytest.mark.parametrize("k", range(len(TABLE_CASES)))
def test_random_case_tile_table(k):
    B, T, H = TABLE_CASES[k]
    c = case_of(20_000 + k)
    c.update(B=B, T=T, H=H, Dh=64, dtype=torch.float16)
    run_case(20_000 + k, c)


@pytest.mark.parametrize("seed", range(48))
def test_random_case_retentive(seed):
    run_case(10_000 + seed, retentive_case_of(seed))


def run_case(seed, c):
    print(f"fuzz {seed}: {c}", flush=True)
    sys.stdout.flush()
    dt = c["dtype"]
    shp = (c["B"], c["T"], c["H"], c["Dh"])
    x = {k: synth.normal(shp, 7000 + 10 * seed + i, c["a_mean"] if k == "a" else 0.0,
                         c["a_std"] if k == "a" else 1.0, dt)
         for i, k in enumerate(("a", "v", "q", "dy"))}
    e0 = synth.random_state(c["B"], c["H"], c["Dh"], 7900 + seed) if c["e0"] else None
    dET = synth.random_state(c["B"], c["H"], c["Dh"], 7950 + seed) if c["dET"] else None
    g = {k: t.to(DEV) for k, t in x.items()}
    ge0 = None if e0 is None else e0.to(DEV)
    gdET = None if dET is None else dET.to(DEV)
    y, eT, ck = binding.scan_fwd(g["a"], g["v"], g["q"], ge0, mode=c["mode"], return_ckpt=True,
                                 deterministic=c["det"])
    da, dv, dq, de0 = binding.scan_bwd(g["a"], g["v"], g["q"], g["dy"], ge0, gdET, ckpt=ck,
                                       mode=c["mode"], deterministic=c["det"])
    torch.cuda.synchronize()
    m = 0 if c["mode"] == "direct" else 1
    ry, reT = oracle.scan_fwd(x["a"], x["v"], x["q"], e0, mode=m, threads=4)
    rda, rdv, rdq, rde0 = oracle.scan_bwd(x["a"], x["v"], x["q"], x["dy"], e0, dET, mode=m,
                                          threads=4)
    sbar = torch.float32  # fp32 outputs carry fp32 arithmetic alone, whatever the storage
    # saturated gates (|a| large) make some gradients numerically zero: compare those at an
    # absolute 1e-30 (the scale floor), as the look-back stress tests do
    floor = 1e-30
    assert_close("y", y, ry, dt, floor=floor)
    assert_close("final_state", eT, reT, sbar, floor=floor)
    assert_close("d_logit", da, rda, dt, floor=floor)
    assert_close("d_value", dv, rdv, dt, floor=floor)
    assert_close("d_query", dq, rdq, dt, floor=floor)
    assert_close("d_init", de0, rde0, sbar, floor=floor)
    for ws in binding._workspaces.values():
        assert int(ws[12:16].view(torch.int32).item()) == 0, "look-back wait timed out"
