"""The scan over a sequence cut into segments (one per device, say), on one GPU, against the
oracle's scan of the whole sequence.

Forward: each segment's aggregate from a zero state (its final state and gate product),
the aggregates composed in order into each segment's entering state, then each segment's
forward with that state.  Backward: each segment's gradient reaching its start with none
arriving at its end, composed from the last segment into each segment's incoming gradient,
then each segment's backward with it.  The composition is the associative pair combine of
page "Entangled State Attention", "[ ARCHITECTURE ]".
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from gated_linear_recurrence_chunked_amd import binding, synth
from helpers import TOL, assert_close, f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
      "f8e4m3": torch.float8_e4m3fn}
MODES = {"direct": 0, "controlled": 1}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def state_bar(dtype):
    """fp32 outputs carry fp32 arithmetic alone, whatever the storage: the fp32 bar."""
    return torch.float32


CASES = [
    # (B, H, Dh, segment lengths)
    (2, 2, 64, [300, 1, 450, 249]),
    (3, 1, 16, [64, 64, 64]),
    (1, 4, 128, [1000, 0, 777]),
    (8, 1, 64, [513, 1024, 300, 7, 200, 96, 100, 50]),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}-{len(c[3])}seg")
@pytest.mark.parametrize("dt,mode", [("f32", "direct"), ("f16", "controlled"),
                                     ("bf16", "direct"), ("f8e4m3", "controlled")])
def test_segmented_scan_equals_whole_sequence(case, dt, mode):
    B, H, Dh, lens = case
    dtype = DT[dt]
    T = sum(lens)
    say(f"segments {case} {dt} {mode}")
    shp = (B, T, H, Dh)
    x = {k: synth.normal(shp, 70 + i, 0.7 if k == "a" else 0.0, 1.5 if k == "a" else 1.0, dtype)
         for i, k in enumerate(("a", "v", "q", "dy"))}
    e0 = synth.random_state(B, H, Dh, 75)
    dET = synth.random_state(B, H, Dh, 76)
    g = {k: t.to(DEV) for k, t in x.items()}
    bounds = np.cumsum([0] + lens)
    seg = [{k: g[k][:, bounds[i]:bounds[i + 1]].contiguous() for k in g} for i in range(len(lens))]

    # forward, pass 1: every segment's aggregate (independent: one per device)
    aggs = [binding.segment_fwd(s["a"], s["v"], mode=mode) for s in seg]
    E_seg = torch.stack([e for e, _ in aggs])
    P_seg = torch.stack([p for _, p in aggs])
    # pass 2: compose, then each segment's forward from its entering state
    carry, total = binding.segment_compose(P_seg, E_seg, e0.to(DEV))
    outs = [binding.scan_fwd(s["a"], s["v"], s["q"], carry[i], mode=mode, return_ckpt=True)
            for i, s in enumerate(seg)]
    y = torch.cat([o[0] for o in outs], 1)
    # backward, pass 1: every segment's gradient reaching its start (none at its end)
    lam = torch.stack([binding.segment_bwd(s["a"], s["v"], s["q"], s["dy"], carry[i],
                                           ckpt=outs[i][2], mode=mode)
                       for i, s in enumerate(seg)])
    # pass 2: compose from the last segment, then each segment's backward
    dcarry, dtotal = binding.segment_compose(P_seg, lam, dET.to(DEV), reverse=True)
    grads = [binding.scan_bwd(s["a"], s["v"], s["q"], s["dy"], carry[i], dcarry[i],
                              ckpt=outs[i][2], mode=mode) for i, s in enumerate(seg)]
    torch.cuda.synchronize()

    m = MODES[mode]
    ry, reT, rE = oracle.scan_fwd(x["a"], x["v"], x["q"], e0, mode=m, states=True, threads=8)
    rda, rdv, rdq, rde0 = oracle.scan_bwd(x["a"], x["v"], x["q"], x["dy"], e0, dET, mode=m,
                                          threads=8)
    assert_close("y", y, ry, dtype)
    assert_close("final state (composed)", total, reT, state_bar(dtype))
    assert_close("final state (last segment)", outs[-1][1], reT, state_bar(dtype))
    for i in range(1, len(lens)):  # the state entering segment i is E at its start - 1
        if bounds[i] > 0:
            assert_close(f"carry {i}", carry[i], rE[:, bounds[i] - 1], state_bar(dtype))
    assert_close("d_logit", torch.cat([gr[0] for gr in grads], 1), rda, dtype)
    assert_close("d_value", torch.cat([gr[1] for gr in grads], 1), rdv, dtype)
    assert_close("d_query", torch.cat([gr[2] for gr in grads], 1), rdq, dtype)
    assert_close("d_init (composed)", dtotal, rde0, state_bar(dtype))
    assert_close("d_init (first segment)", grads[0][3], rde0, state_bar(dtype))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_segment_aggregate_against_its_definition(dt):
    """The aggregate pair of one segment: E from a zero state (the oracle's scan) and the
    product of the gates (the oracle's gates, multiplied out)."""
    dtype = DT[dt]
    B, T, H, Dh = 3, 2500, 2, 32
    say(f"segment aggregate {dt}")
    # long memory (mean gate ~0.996): the product over 2500 steps stays near 1e-5, inside the
    # fp32 range
    a = synth.normal((B, T, H, Dh), 81, 6.0, 1.0, dtype)
    v = synth.normal((B, T, H, Dh), 82, 0.0, 1.0, dtype)
    for mode in ("direct", "controlled"):
        E, P = binding.segment_fwd(a.to(DEV), v.to(DEV), mode=mode)
        torch.cuda.synchronize()
        _, rE = oracle.scan_fwd(a, v, v, mode=MODES[mode])
        A, _ = oracle.gates(a, v, MODES[mode])
        rP = np.prod(A, axis=1)
        assert_close("seg_state", E, rE, torch.float32 if dtype == torch.float32 else torch.float16)
        # each step's gate carries a few fp32 ulps and each product one more: the relative
        # error of the product stays below T * 2^-20
        assert (rP > 1e-30).all()
        assert np.max(np.abs(f64(P) - rP) / np.abs(rP)) < T * 2.0 ** -20


def test_empty_segment_is_the_identity():
    say("empty segment")
    z = torch.empty((2, 0, 2, 16), dtype=torch.float16, device=DEV)
    E, P = binding.segment_fwd(z, z.clone())
    lam = binding.segment_bwd(z, z.clone(), z.clone(), z.clone())
    torch.cuda.synchronize()
    assert (E == 0).all() and (P == 1).all() and (lam == 0).all()
