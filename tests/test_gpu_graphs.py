"""Scan calls recorded into a HIP graph (stream capture) and replayed.

A recorded scan launch cannot reuse the host's per-call look-back tag: every replay would
find the previous replay's finished words under the same tag and take stale carries.  The
library records a one-thread kernel that advances a device tag in the workspace before each
recorded scan launch.  Here the graph is replayed several times with new inputs written
between replays, with eager calls on the same workspace in between, and every replay is
checked against the eager result and the oracle.
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


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("det", [False, True], ids=["default", "deterministic"])
@pytest.mark.parametrize("dt,mode", [(torch.float16, "controlled"), (torch.bfloat16, "direct")])
def test_recorded_scans_replay_correctly(dt, mode, det):
    """With ESA_DETERMINISTIC (blocks of 8 tiles on these 8 chains) every replay also gives
    the eager call's bits."""
    B, T, H, Dh = 4, 3000, 2, 64  # 12 forward and 24 backward tiles per channel block
    say(f"graph replay {dt} {mode} det={det}")
    shp = (B, T, H, Dh)
    x = {k: torch.empty(shp, dtype=dt, device=DEV) for k in ("a", "v", "q", "dy")}
    e0 = synth.random_state(B, H, Dh, 41).to(DEV)

    def fill(r):
        for i, k in enumerate(x):
            x[k].copy_(synth.normal(shp, 4000 + 10 * r + i, 0.5 if k == "a" else 0.0, 1.0, dt))

    fill(0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm up: the workspace for stream s exists before capture
        binding.scan_fwd(x["a"], x["v"], x["q"], e0, mode=mode, return_ckpt=True,
                         deterministic=det)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        y, eT, ck = binding.scan_fwd(x["a"], x["v"], x["q"], e0, mode=mode, return_ckpt=True,
                                     deterministic=det)
        da, dv, dq, de0 = binding.scan_bwd(x["a"], x["v"], x["q"], x["dy"], e0, None, ckpt=ck,
                                           mode=mode, deterministic=det)
        seg_e, seg_p = binding.segment_fwd(x["a"], x["v"], mode=mode, deterministic=det)

    for r in range(1, 5):
        fill(r)  # new inputs, written eagerly between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"  replay {r}")
        # eager calls on the same stream and workspace, between replays
        with torch.cuda.stream(s):
            ey, eeT, eck = binding.scan_fwd(x["a"], x["v"], x["q"], e0, mode=mode,
                                            return_ckpt=True, deterministic=det)
            eda, edv, edq, ede0 = binding.scan_bwd(x["a"], x["v"], x["q"], x["dy"], e0, None,
                                                   ckpt=eck, mode=mode, deterministic=det)
            es_e, es_p = binding.segment_fwd(x["a"], x["v"], mode=mode, deterministic=det)
        torch.cuda.synchronize()
        if det:
            for got, ref in ((y, ey), (eT, eeT), (ck, eck), (da, eda), (dv, edv), (dq, edq),
                             (de0, ede0), (seg_e, es_e), (seg_p, es_p)):
                assert torch.equal(got, ref), "a deterministic replay differs from eager"
        for name, got, ref in (("y", y, ey), ("d_logit", da, eda), ("d_value", dv, edv),
                               ("d_query", dq, edq)):
            assert_close(f"{name} replay {r} vs eager", got, ref, dt)
        for name, got, ref in (("final", eT, eeT), ("d_init", de0, ede0)):
            assert_close(f"{name} replay {r} vs eager", got, ref, torch.float32)
        c = {k: t.cpu() for k, t in x.items()}
        ry, reT = oracle.scan_fwd(c["a"], c["v"], c["q"], e0.cpu(), mode=MODES[mode], threads=8)
        rda, rdv, rdq, rde0 = oracle.scan_bwd(c["a"], c["v"], c["q"], c["dy"], e0.cpu(), None,
                                              mode=MODES[mode], threads=8)
        _, rse = oracle.scan_fwd(c["a"], c["v"], c["v"], None, mode=MODES[mode])
        assert_close(f"y replay {r}", y, ry, dt)
        assert_close(f"d_logit replay {r}", da, rda, dt)
        assert_close(f"d_value replay {r}", dv, rdv, dt)
        assert_close(f"d_query replay {r}", dq, rdq, dt)
        assert_close(f"d_init replay {r}", de0, rde0, torch.float32)
        assert_close(f"final replay {r}", eT, reT, torch.float32)
        assert_close(f"segment state replay {r}", seg_e, rse, torch.float32)
    for ws in binding._workspaces.values():
        assert int(ws[12:16].view(torch.int32).item()) == 0, "look-back wait timed out"
    del g


def test_replay_after_the_stream_workspace_grew():
    """A recorded scan keeps the raw address of the workspace it ran on.  An eager call on
    the capture stream that needs more workspace makes the binding cache a larger one; the
    superseded workspace must stay alive, since every replay still writes its look-back words
    there.  Memory allocated after the growth (where a freed workspace would be reused) keeps
    its contents through the replays, and every replay matches the oracle."""
    dt, mode = torch.float16, "controlled"
    B, T, H, Dh = 2, 2000, 2, 64
    say("graph replay after the workspace grew")
    shp = (B, T, H, Dh)
    x = {k: synth.normal(shp, 4500 + i, 0.5 if k == "a" else 0.0, 1.0, dt).to(DEV)
         for i, k in enumerate(("a", "v", "q", "dy"))}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        binding.scan_fwd(x["a"], x["v"], x["q"], mode=mode, return_ckpt=True)
        ws_before = binding.get_workspace(0, DEV)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        y, eT, ck = binding.scan_fwd(x["a"], x["v"], x["q"], mode=mode, return_ckpt=True)
        da, dv, dq, _ = binding.scan_bwd(x["a"], x["v"], x["q"], x["dy"], ckpt=ck, mode=mode)
    c = {k: t.cpu() for k, t in x.items()}
    ry, _ = oracle.scan_fwd(c["a"], c["v"], c["q"], mode=1, threads=8)
    rda, rdv, rdq, _ = oracle.scan_bwd(c["a"], c["v"], c["q"], c["dy"], mode=1, threads=8)
    # a problem 16 times larger, eagerly on the capture stream: the cached workspace grows
    big = {k: synth.normal((B, 16 * T, H, Dh), 4600 + i, 0.0, 1.0, dt).to(DEV)
           for i, k in enumerate("avq")}
    with torch.cuda.stream(s):
        binding.scan_fwd(big["a"], big["v"], big["q"], mode=mode)
        ws_after = binding.get_workspace(0, DEV)
    torch.cuda.synchronize()
    assert ws_after.data_ptr() != ws_before.data_ptr()
    nb = ws_before.numel()
    del ws_before
    junk = torch.full((nb,), 0x5A, dtype=torch.uint8, device=DEV)
    for r in range(3):
        with torch.cuda.stream(s):
            g.replay()
            binding.scan_fwd(big["a"], big["v"], big["q"], mode=mode)  # eager, between replays
        torch.cuda.synchronize()
        say(f"  replay {r}")
        assert bool((junk == 0x5A).all()), "a replay wrote into memory it does not own"
        assert_close(f"y replay {r}", y, ry, dt)
        assert_close(f"d_logit replay {r}", da, rda, dt)
        assert_close(f"d_value replay {r}", dv, rdv, dt)
        assert_close(f"d_query replay {r}", dq, rdq, dt)
    del g
