"""The look-back statistics instance (ESA_LOOKBACK_STATS): its results are those of the
default look-back (checked against the oracle), and its counters, read with
esa_workspace_status, account for every lane of every tile that has an earlier tile in its
chain: each one either found its neighbour's inclusive value published or walked back."""
import sys

import pytest
import torch

import oracle
from gated_linear_recurrence_chunked_amd import binding, synth
from helpers import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("dt", [torch.float16, torch.float8_e4m3fn])
def test_stats_instance_counts_every_lane(dt):
    B, T, H, Dh = 3, 5000, 2, 64
    mode = "controlled"
    say(f"look-back statistics {dt}")
    shp = (B, T, H, Dh)
    x = {k: synth.normal(shp, 5100 + i, 1.0 if k == "a" else 0.0, 1.0, dt)
         for i, k in enumerate(("a", "v", "q", "dy"))}
    g = {k: t.to(DEV) for k, t in x.items()}
    ws = torch.zeros(binding.workspace_bytes(B, T, H, Dh, dt), dtype=torch.uint8, device=DEV)
    m = binding.MODES[mode] | binding.LOOKBACK_STATS
    y, eT, ck = binding.scan_fwd(g["a"], g["v"], g["q"], mode=m, return_ckpt=True, workspace=ws)
    f = binding.workspace_status(ws)
    say(f"  forward {f}")
    ws.zero_()
    da, dv, dq, de0 = binding.scan_bwd(g["a"], g["v"], g["q"], g["dy"], ckpt=ck, mode=m,
                                       workspace=ws)
    b = binding.workspace_status(ws)
    say(f"  backward {b}")
    torch.cuda.synchronize()
    lanes = B * H * Dh
    tt_f = 256 if dt == torch.float16 else 128  # forward tile lengths at Dh = 64
    tt_b = 128 if dt == torch.float16 else 64
    for st, tt in ((f, tt_f), (b, tt_b)):
        n_tiles = -(-T // tt)
        assert st["timeout_tag"] == 0
        assert st["took_published"] + st["walked"] == (n_tiles - 1) * lanes
        assert st["tiles_folded"] >= 0
        assert (st["longest_walk"] >= 1) == (st["walked"] > 0)
        assert st["tiles_folded"] <= st["walked"] * (n_tiles - 1)
    ry, reT = oracle.scan_fwd(x["a"], x["v"], x["q"], mode=1, threads=8)
    rda, rdv, rdq, rde0 = oracle.scan_bwd(x["a"], x["v"], x["q"], x["dy"], mode=1, threads=8)
    assert_close("y", y, ry, dt)
    assert_close("final_state", eT, reT, torch.float32)
    assert_close("d_logit", da, rda, dt)
    assert_close("d_value", dv, rdv, dt)
    assert_close("d_query", dq, rdq, dt)
