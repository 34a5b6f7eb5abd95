"""The generation workload end to end: prefill B=256 prompts of 512 tokens (H=8, Dh=64,
fp16, controlled), then 1024 one-token steps with fresh inputs, two ways:

  - eagerly, one esa_state_step launch per step through binding.StepPlan;
  - as binding.DecodeGraph, the 1024 steps recorded once into a HIP graph, replayed twice
    from the prefill state.

Every step's readout and the state after steps 1, 256 and 1024 are compared with the
oracle's chain of one-token updates on sampled batch rows (page "Entangled State
Attention", "[ GENERATION / MEMORY ]": prompt lengths and one-token updates; page
"Entangled State Attention v2.1", sections 5 and 6).  The step kernel has no cross-workgroup
combine, so the eager chain and every replay also agree bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from gated_linear_recurrence_chunked_amd import binding, synth
from helpers import TOL, assert_close, err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SAMPLE = [0, 131, 255]
CHECK_AFTER = (1, 256, 1024)  # state checks, after this many steps


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_prefill_then_1024_steps_eager_and_graph():
    wl = synth.WORKLOADS["decode_f16"]
    B, H, Dh, n = wl.B, wl.H, wl.Dh, wl.steps
    T = wl.prompts[0]
    dt = torch.float16
    assert n == 1024
    say(f"decode workload: prefill B={B} T={T}, then {n} steps")
    g = synth.make_inputs(wl, device=DEV, T=T)
    y0, st0 = binding.scan_fwd(g["a"], g["v"], g["q"], mode=wl.mode)
    steps = [synth.decode_step_inputs(wl, k, device=DEV) for k in range(n)]
    A = torch.stack([s["a"] for s in steps])
    V = torch.stack([s["v"] for s in steps])
    Q = torch.stack([s["q"] for s in steps])
    del steps
    torch.cuda.synchronize()

    # the oracle: prefill of the sampled rows, then the chain of one-token updates
    rows = {k: g[k][SAMPLE].cpu() for k in ("a", "v", "q")}
    ry0, rst = oracle.scan_fwd(rows["a"], rows["v"], rows["q"], mode=1, threads=3)
    assert_close("prefill y", y0[SAMPLE].cpu(), ry0, dt)
    assert_close("prefill state", st0[SAMPLE].cpu(), rst, torch.float32)
    As, Vs, Qs = (X[:, SAMPLE].cpu() for X in (A, V, Q))
    ref_y = np.empty((n, len(SAMPLE), H, Dh))
    ref_state = {}
    for k in range(n):
        ref_y[k], rst = oracle.state_step(As[k], Vs[k], Qs[k], rst, mode=1)
        if k + 1 in CHECK_AFTER:
            ref_state[k + 1] = rst
    say("  oracle chain done")

    # eager: one launch per step through a StepPlan
    st = st0.clone()
    plan = binding.StepPlan(st, dt, wl.mode)
    ye = torch.empty((n, B, H, Dh), dtype=dt, device=DEV)
    eager_state = {}
    for k in range(n):
        plan(A[k], V[k], Q[k], ye[k])
        if k + 1 in CHECK_AFTER:
            eager_state[k + 1] = st.clone()
    torch.cuda.synchronize()
    assert_close("eager y, all steps", ye[:, SAMPLE].cpu(), ref_y, dt)
    for k in CHECK_AFTER:
        assert_close(f"eager state after {k}", eager_state[k][SAMPLE].cpu(), ref_state[k],
                     torch.float32)

    # the same chain recorded once into a graph, replayed twice from the prefill state
    dg = binding.DecodeGraph(B, H, Dh, n, dtype=dt, mode=wl.mode, device=DEV,
                             snapshot_steps=CHECK_AFTER[:-1])
    dg.a.copy_(A)
    dg.v.copy_(V)
    dg.q.copy_(Q)
    for r in range(2):
        dg.state.copy_(st0)
        dg.y.fill_(float("nan"))
        dg.replay()
        torch.cuda.synchronize()
        say(f"  replay {r}")
        assert_close(f"graph y, all steps, replay {r}", dg.y[:, SAMPLE].cpu(), ref_y, dt)
        got = {k: dg.snapshots[i] for i, k in enumerate(CHECK_AFTER[:-1])}
        got[n] = dg.state
        for k in CHECK_AFTER:
            assert_close(f"graph state after {k}, replay {r}", got[k][SAMPLE].cpu(),
                         ref_state[k], torch.float32)
            assert torch.equal(got[k], eager_state[k]), "replay differs from the eager chain"
        assert torch.equal(dg.y, ye), "replay readouts differ from the eager chain"
    # prefill + 1024 steps equals one scan over the 1536 tokens (whole batch, fp32 state)
    Ac, Vc, Qc = (torch.cat([g[k], X.transpose(0, 1)], 1).contiguous()
                  for k, X in (("a", A), ("v", V), ("q", Q)))
    yl, stl = binding.scan_fwd(Ac, Vc, Qc, mode=wl.mode)
    torch.cuda.synchronize()
    assert err(dg.state, stl) <= TOL[torch.float32]
    assert err(dg.y.transpose(0, 1), yl[:, T:]) <= TOL[dt]


def test_decode_graph_one_token_per_replay():
    """steps = 1: the per-token graph of a generation loop, inputs written between replays
    (here fp8 E4M3 storage, direct mode, snapshots refused outside 1..steps)."""
    B, H, Dh, n = 5, 3, 128, 40
    dt = torch.float8_e4m3fn
    say("decode graph, one token per replay")
    with pytest.raises(ValueError):
        binding.DecodeGraph(B, H, Dh, 1, dtype=dt, snapshot_steps=(2,))
    st0 = synth.random_state(B, H, Dh, 611)
    dg = binding.DecodeGraph(B, H, Dh, 1, dtype=dt, mode="direct", device=DEV)
    dg.state.copy_(st0)
    rst = st0
    for k in range(n):
        x = {c: synth.normal((B, H, Dh), 620 + 3 * k + i, 0.0, 1.0, dt)
             for i, c in enumerate("avq")}
        dg.a[0].copy_(x["a"])
        dg.v[0].copy_(x["v"])
        dg.q[0].copy_(x["q"])
        dg.replay()
        torch.cuda.synchronize()
        ry, rst = oracle.state_step(x["a"], x["v"], x["q"], rst, mode=0)
        assert_close(f"y step {k}", dg.y[0], ry, dt)
        assert_close(f"state step {k}", dg.state, rst, torch.float32)
