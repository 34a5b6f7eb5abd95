"""Every one-byte logit code through the scans, against the oracle.

With one-byte storage the kernels take each step's gate from a table of the 256 codes
(filled per workgroup) instead of evaluating it in place, so the codes that random N(mu,
sigma) draws rarely or never produce (the extremes 448 and 57344, subnormals, zeros of both
signs, E5M2's infinities) are driven here on purpose: every lane cycles through all codes but
NaN's (a NaN gate would turn its lane NaN for the rest of the sequence; the NaN codes are
covered by test_gpu_nonfinite.py).  The gate is sigma(a) of the decoded code (page
"entangled-state-attention 0.1.0", "Core idea"); the oracle decodes the same codes in fp64.
"""
import sys

import pytest
import torch

import oracle
from gated_linear_recurrence_chunked_amd import binding, synth
from helpers import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MODES = {"direct": 0, "controlled": 1}
NAN_CODES = {torch.float8_e4m3fn: (0x7F, 0xFF),
             torch.float8_e5m2: (0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF)}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def all_codes(B, T, H, Dh, dt):
    """Logits whose codes cycle over every non-NaN code, shifted per lane so that neighbouring
    lanes and steps hold different codes."""
    codes = torch.tensor([c for c in range(256) if c not in NAN_CODES[dt]], dtype=torch.int64)
    t = torch.arange(T).view(1, T, 1, 1)
    lane = torch.arange(B * H * Dh).view(B, 1, H, Dh)
    idx = (t * 37 + lane * 11) % codes.numel()
    return codes[idx].to(torch.uint8).view(dt)


@pytest.mark.parametrize("dt", [torch.float8_e4m3fn, torch.float8_e5m2])
@pytest.mark.parametrize("mode", ["direct", "controlled"])
def test_every_logit_code(dt, mode):
    B, T, H, Dh = 2, 1500, 2, 64  # ragged last tile; 12 forward and 24 backward tiles
    say(f"fp8 codes {dt} {mode}")
    shp = (B, T, H, Dh)
    x = {"a": all_codes(B, T, H, Dh, dt)}
    for i, k in enumerate(("v", "q", "dy")):
        x[k] = synth.normal(shp, 90 + i, 0.0, 1.0, dt)
    e0 = synth.random_state(B, H, Dh, 97)
    g = {k: t.to(DEV) for k, t in x.items()}
    y, eT, ck = binding.scan_fwd(g["a"], g["v"], g["q"], e0.to(DEV), mode=mode, return_ckpt=True)
    da, dv, dq, de0 = binding.scan_bwd(g["a"], g["v"], g["q"], g["dy"], e0.to(DEV), None,
                                       ckpt=ck, mode=mode)
    torch.cuda.synchronize()
    m = MODES[mode]
    ry, reT = oracle.scan_fwd(x["a"], x["v"], x["q"], e0, mode=m, threads=2)
    rda, rdv, rdq, rde0 = oracle.scan_bwd(x["a"], x["v"], x["q"], x["dy"], e0, None, mode=m,
                                          threads=2)
    assert_close("y", y, ry, dt)  # the fp8 bars carry their subnormal floor (helpers.FLOOR)
    assert_close("final_state", eT, reT, torch.float32)
    assert_close("d_logit", da, rda, dt)
    assert_close("d_value", dv, rdv, dt)
    assert_close("d_query", dq, rdq, dt)
    assert_close("d_init", de0, rde0, torch.float32)
