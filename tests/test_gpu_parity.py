"""Parity of the HIP path (through the C ABI) against the fp64 oracle, element by element.

Sizes are ones the oracle finishes in seconds while still spanning several tiles and a
ragged tail; every dtype, mode and head size the library supports appears.  The
workloads (tests/../gated_linear_recurrence_chunked_amd/synth.py) also run at full size in
the launch configuration the benchmark times, compared on whole sampled batch rows (every
row is an independent problem the oracle solves exactly).
"""
import sys
import zlib

import numpy as np
import pytest
import torch

import oracle
from gated_linear_recurrence_chunked_amd import binding, synth
from helpers import TOL, assert_close, err, f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
      "f8e4m3": torch.float8_e4m3fn, "f8e5m2": torch.float8_e5m2}
FP8 = (torch.float8_e4m3fn, torch.float8_e5m2)


def state_bar(dtype):
    """The bar for fp32 outputs (final states, checkpoints, initial-state gradients): the
    storage dtype rounds only the sequence tensors, so the fp32 outputs of every storage dtype
    carry fp32 arithmetic alone and are held to the fp32 bar."""
    return torch.float32
MODES = {"direct": 0, "controlled": 1}


def seed_of(*parts) -> int:
    """A seed that depends only on the case (not on Python's per-process string hashing)."""
    return zlib.crc32(repr(parts).encode()) % 100000


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def inputs_cpu(B, T, H, Dh, dtype, seed, a_mean=0.0, a_std=1.5, dy=False):
    shp = (B, T, H, Dh)
    out = {
        "a": synth.normal(shp, seed, a_mean, a_std, dtype),
        "v": synth.normal(shp, seed + 1, 0.0, 1.0, dtype),
        "q": synth.normal(shp, seed + 2, 0.0, 1.0, dtype),
    }
    if dy:
        out["dy"] = synth.normal(shp, seed + 3, 0.0, 1.0, dtype)
    return out


def check_abort_clear():
    for ws in binding._workspaces.values():
        torch.cuda.synchronize()
        assert int(ws[12:16].view(torch.int32).item()) == 0, "look-back wait timed out"


# (B, T, H, Dh): single tile, ragged tails, many tiles, channel blocks that do not fill
SHAPES = [
    (1, 1, 1, 16),
    (2, 63, 2, 16),
    (1, 65, 1, 128),
    (3, 129, 3, 32),
    (2, 1000, 2, 64),
    (1, 4097, 1, 64),
    (5, 300, 1, 16),
    (2, 777, 2, 128),
    (1, 256, 2, 16),
    # channel-block counts divisible by 8: the XCD-aware tile order
    (8, 300, 1, 64),
    (4, 130, 4, 32),
    (2, 200, 8, 128),
    (16, 257, 2, 16),
    # fp16, Dh = 64 sizes that the forward's tile table gives 256-thread workgroups (128-step
    # tiles): 8 channel blocks at T = 1024, and a ragged T = 1000 of 8 blocks
    (1, 1024, 8, 64),
    (2, 1000, 4, 64),
]
DTYPE_MODE = [("f32", "direct"), ("f32", "controlled"), ("f16", "controlled"), ("f16", "direct"),
              ("bf16", "direct"), ("bf16", "controlled"), ("f8e4m3", "controlled"),
              ("f8e4m3", "direct"), ("f8e5m2", "direct"), ("f8e5m2", "controlled")]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dt,mode", DTYPE_MODE)
def test_fwd_parity(shape, dt, mode):
    B, T, H, Dh = shape
    dtype = DT[dt]
    say(f"fwd {shape} {dt} {mode}")
    x = inputs_cpu(B, T, H, Dh, dtype, seed=seed_of(shape, dt, mode))
    e0 = synth.random_state(B, H, Dh, seed=7) if T % 2 else None
    g = {k: t.to(DEV) for k, t in x.items()}
    y, eT, ck = binding.scan_fwd(g["a"], g["v"], g["q"], None if e0 is None else e0.to(DEV),
                                 mode=mode, return_ckpt=True)
    torch.cuda.synchronize()
    ry, reT, rE = oracle.scan_fwd(x["a"], x["v"], x["q"], e0, mode=MODES[mode], states=True,
                                  threads=8)
    assert_close("y", y, ry, dtype)
    assert_close("final_state", eT, reT, state_bar(dtype))
    nck = -(-T // 64)
    ckv = ck[: B * nck * H * Dh].view(B, nck, H, Dh)
    idx = [min(T, 64 * (k + 1)) - 1 for k in range(nck)]
    assert_close("ckpt", ckv, rE[:, idx], state_bar(dtype))
    check_abort_clear()


@pytest.mark.parametrize("shape", SHAPES[1:], ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dt,mode", DTYPE_MODE)
def test_bwd_parity(shape, dt, mode):
    B, T, H, Dh = shape
    dtype = DT[dt]
    say(f"bwd {shape} {dt} {mode}")
    x = inputs_cpu(B, T, H, Dh, dtype, seed=seed_of(shape, dt, mode, 1), a_mean=0.5,
                   dy=True)
    e0 = synth.random_state(B, H, Dh, seed=8) if T % 2 else None
    dET = synth.random_state(B, H, Dh, seed=9) if T % 3 else None
    g = {k: t.to(DEV) for k, t in x.items()}
    ge0 = None if e0 is None else e0.to(DEV)
    gdET = None if dET is None else dET.to(DEV)
    _, _, ck = binding.scan_fwd(g["a"], g["v"], g["q"], ge0, mode=mode, return_ckpt=True)
    da, dv, dq, de0 = binding.scan_bwd(g["a"], g["v"], g["q"], g["dy"], ge0, gdET, ckpt=ck,
                                       mode=mode)
    # the same without a checkpoint (the library recomputes it)
    da2, dv2, dq2, de02 = binding.scan_bwd(g["a"], g["v"], g["q"], g["dy"], ge0, gdET, ckpt=None,
                                           mode=mode)
    torch.cuda.synchronize()
    r = oracle.scan_bwd(x["a"], x["v"], x["q"], x["dy"], e0, dET, mode=MODES[mode], threads=8)
    for name, got, got2, ref in zip(("d_logit", "d_value", "d_query", "d_init"),
                                    (da, dv, dq, de0), (da2, dv2, dq2, de02), r):
        bar = state_bar(dtype) if name == "d_init" else dtype
        assert_close(name, got, ref, bar)
        assert_close(name + " (no ckpt)", got2, ref, bar)
    check_abort_clear()


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16", "f8e4m3", "f8e5m2"])
@pytest.mark.parametrize("Dh", [16, 32, 64, 128])
@pytest.mark.parametrize("mode", ["direct", "controlled"])
def test_step_parity(dt, Dh, mode):
    dtype = DT[dt]
    B, H = 7, 3
    say(f"step B={B} H={H} Dh={Dh} {dt} {mode}")
    x = inputs_cpu(B, 1, H, Dh, dtype, seed=Dh * 31 + len(dt))
    st0 = synth.random_state(B, H, Dh, seed=11)
    st = st0.to(DEV)
    y = binding.state_step(x["a"][:, 0].contiguous().to(DEV), x["v"][:, 0].contiguous().to(DEV),
                           x["q"][:, 0].contiguous().to(DEV), st, mode=mode)
    torch.cuda.synchronize()
    ry, rst = oracle.state_step(x["a"][:, 0], x["v"][:, 0], x["q"][:, 0], st0, mode=MODES[mode])
    assert_close("y", y, ry, dtype)
    assert_close("state", st, rst, state_bar(dtype))


@pytest.mark.parametrize("a_mean", [6.0, 8.0, 10.0])
def test_fp32_gate_near_one_is_correctly_rounded(a_mean):
    """With fp32 storage the gate s = sigma(a) of a retentive logit is s rounded correctly
    from the exact value (read back through one direct-mode step from state 1 with v = 0,
    which returns s itself): a long chain sums any bias of s relative to 1 - s over its
    ~1 / (1 - s) steps of memory.  Against the oracle's fp64 sigma: at most one unit in the
    last place off, off at all in at most 2 % of draws, and a mean error relative to 1 - s
    below 2e-6 (a reciprocal-based s is off in half the draws, with a mean of -1.5e-5 at
    a ~ N(8, 1))."""
    say(f"fp32 gate rounding a~N({a_mean},1)")
    B, H, Dh = 1024, 4, 64
    a = synth.normal((B, H, Dh), 990 + int(a_mean), a_mean, 1.0, torch.float32)
    st = torch.ones((B, H, Dh), device=DEV)
    z = torch.zeros((B, H, Dh), device=DEV)
    binding.state_step(a.to(DEV), z, z, st, mode="direct")
    torch.cuda.synchronize()
    s_gpu = st.cpu().double().numpy()
    s_true, _ = oracle.gates(a, torch.zeros_like(a), 0)
    s_true = np.asarray(s_true, dtype=np.float64).reshape(s_gpu.shape)
    s_rn = s_true.astype(np.float32).astype(np.float64)
    ulp = 2.0 ** -24  # spacing of fp32 in [0.5, 1)
    assert np.all(s_true > 0.5)
    assert np.max(np.abs(s_gpu - s_rn)) <= ulp
    assert np.mean(s_gpu != s_rn) <= 0.02
    assert abs(np.mean((s_gpu - s_true) / (1.0 - s_true))) < 2e-6


@pytest.mark.parametrize("mode", ["direct", "controlled"])
def test_fp32_retentive_gates_do_not_drift(mode):
    """fp32 storage with very retentive gates (a ~ N(10, 1): 1 - s ~ 5e-5, ~20000 steps of
    memory) over 15000 steps, the whole sequence one chain of 118 forward tiles.  Gate
    products are carried as complements and the fp32 kernels accumulate the state and its
    reverse-time gradient in fp64, so every output meets the fp32 bar (1e-5).  (A sequential
    fp32 loop on the host, with correctly rounded gates, is off by up to 3.5e-5 in y and
    1.5e-4 in the gate gradient on these inputs; with plain products and fp32 accumulation
    the kernels drifted to 1.3e-4 in y and 4.9e-4 in the gate gradient.)"""
    say(f"fp32 retentive gates {mode}")
    B, T, H, Dh = 2, 15000, 2, 64
    m = 0 if mode == "direct" else 1
    x = {k: synth.normal((B, T, H, Dh), 700 + i, 10.0 if k == "a" else 0.0, 1.0, torch.float32)
         for i, k in enumerate("avqd")}
    e0 = synth.random_state(B, H, Dh, 777)
    g = {k: t.to(DEV) for k, t in x.items()}
    y, eT, ck = binding.scan_fwd(g["a"], g["v"], g["q"], e0.to(DEV), mode=mode, return_ckpt=True)
    da, dv, dq, de0 = binding.scan_bwd(g["a"], g["v"], g["q"], g["d"], e0.to(DEV), None, ckpt=ck,
                                       mode=mode)
    torch.cuda.synchronize()
    ry, reT = oracle.scan_fwd(x["a"], x["v"], x["q"], e0, mode=m)
    rda, rdv, rdq, rde0 = oracle.scan_bwd(x["a"], x["v"], x["q"], x["d"], e0, None, mode=m)
    for name, got, ref in (("y", y, ry), ("final_state", eT, reT), ("d_init", de0, rde0),
                           ("d_logit", da, rda), ("d_value", dv, rdv), ("d_query", dq, rdq)):
        assert_close(name, got, ref, torch.float32)


def test_step_plan_matches_oracle_and_checks_its_tensors():
    """binding.StepPlan: the decode loop's fixed arguments validated once; steps through it
    equal the oracle's state_step chain, and a mismatched step tensor is refused."""
    say("step plan")
    B, H, Dh = 6, 2, 64
    st0 = synth.random_state(B, H, Dh, seed=21)
    st = st0.to(DEV)
    plan = binding.StepPlan(st, torch.float16, "controlled")
    rst = st0
    for k in range(5):
        x = inputs_cpu(B, 1, H, Dh, torch.float16, seed=300 + k)
        a, v, q = (x[n][:, 0].contiguous() for n in ("a", "v", "q"))
        y = torch.empty((B, H, Dh), dtype=torch.float16, device=DEV)
        plan(a.to(DEV), v.to(DEV), q.to(DEV), y)
        torch.cuda.synchronize()
        ry, rst = oracle.state_step(a, v, q, rst, mode=1)
        assert_close(f"y step {k}", y, ry, torch.float16)
        assert_close(f"state step {k}", st, rst, torch.float16)
    good = torch.empty((B, H, Dh), dtype=torch.float16, device=DEV)
    for bad in (torch.empty((B, H, Dh), dtype=torch.bfloat16, device=DEV),
                torch.empty((B, H, Dh + 1), dtype=torch.float16, device=DEV),
                torch.empty((B, H, 2 * Dh), dtype=torch.float16, device=DEV)[..., ::2]):
        with pytest.raises(ValueError):
            plan(good, good, good, bad)


def test_empty_sequence():
    say("empty sequence")
    B, H, Dh = 2, 2, 32
    z = torch.zeros((B, 0, H, Dh), dtype=torch.float16, device=DEV)
    e0 = synth.random_state(B, H, Dh, seed=3).to(DEV)
    y, eT = binding.scan_fwd(z, z.clone(), z.clone(), e0, mode="controlled")
    assert y.shape == z.shape
    torch.testing.assert_close(eT, e0, rtol=0, atol=0)
    y, eT = binding.scan_fwd(z, z.clone(), z.clone(), None, mode="controlled")
    torch.testing.assert_close(eT, torch.zeros_like(eT), rtol=0, atol=0)
    dET = synth.random_state(B, H, Dh, seed=4).to(DEV)
    _, _, _, dI = binding.scan_bwd(z, z.clone(), z.clone(), z.clone(), e0, dET, mode="controlled")
    torch.testing.assert_close(dI, dET, rtol=0, atol=0)


def test_in_place_final_state():
    say("in-place final state")
    B, T, H, Dh = 2, 700, 2, 64
    x = inputs_cpu(B, T, H, Dh, torch.float16, seed=123)
    e0 = synth.random_state(B, H, Dh, seed=5)
    g = {k: t.to(DEV) for k, t in x.items()}
    st = e0.to(DEV)
    y, eT = binding.scan_fwd(g["a"], g["v"], g["q"], st, mode="controlled", final_state=st)
    torch.cuda.synchronize()
    ry, reT = oracle.scan_fwd(x["a"], x["v"], x["q"], e0, mode=1)
    assert eT.data_ptr() == st.data_ptr()
    assert_close("y", y, ry, torch.float16)
    assert_close("state", st, reT, torch.float32)


def test_binding_rejects_mismatched_outputs():
    """Caller-provided outputs are written in place: a wrong shape, dtype or layout is an
    error, never a silent write past the tensor."""
    say("binding output validation")
    B, T, H, Dh = 2, 64, 2, 64
    x = {k: t.to(DEV) for k, t in inputs_cpu(B, T, H, Dh, torch.float16, seed=77).items()}
    bad_y = [torch.empty(B, T, H, Dh, device=DEV, dtype=torch.float32),
             torch.empty(B, T - 1, H, Dh, device=DEV, dtype=torch.float16),
             torch.empty(B, H, T, Dh, device=DEV, dtype=torch.float16).transpose(1, 2)]
    for y in bad_y:
        with pytest.raises(ValueError):
            binding.scan_fwd(x["a"], x["v"], x["q"], y=y)
    for eT in (torch.empty(B, H, Dh, device=DEV, dtype=torch.float16),
               torch.empty(B, H, Dh + 1, device=DEV)[..., :Dh]):
        with pytest.raises(ValueError):
            binding.scan_fwd(x["a"], x["v"], x["q"], final_state=eT)
    a1, v1, q1 = (x[k][:, 0].contiguous() for k in "avq")
    st = torch.zeros(B, H, Dh, device=DEV)
    for y in (torch.empty(B, H, Dh, device=DEV), torch.empty(B, H, 2 * Dh, device=DEV,
                                                               dtype=torch.float16)[..., ::2]):
        with pytest.raises(ValueError):
            binding.state_step(a1, v1, q1, st, y=y)
    with pytest.raises(ValueError):
        binding.state_step(a1, v1, q1, st.to(torch.float16))
    with pytest.raises(ValueError):
        binding.state_step(a1, v1, q1, st.cpu())
    # backward outputs: wrong ones are rejected; right ones are written in place
    dy = x["a"].flip(1).contiguous()
    _, _, ck = binding.scan_fwd(x["a"], x["v"], x["q"], return_ckpt=True)
    for kw in ({"d_logit": bad_y[0]}, {"d_value": bad_y[1]}, {"d_query": bad_y[2]},
               {"d_init": torch.empty(B, H, Dh, device=DEV, dtype=torch.float16)}):
        with pytest.raises(ValueError):
            binding.scan_bwd(x["a"], x["v"], x["q"], dy, ckpt=ck, deterministic=True, **kw)
    ref = binding.scan_bwd(x["a"], x["v"], x["q"], dy, ckpt=ck, deterministic=True)
    outs = [torch.full_like(x["a"], float("nan")) for _ in range(3)]
    outs.append(torch.full((B, H, Dh), float("nan"), device=DEV))
    got = binding.scan_bwd(x["a"], x["v"], x["q"], dy, ckpt=ck, deterministic=True,
                           d_logit=outs[0], d_value=outs[1], d_query=outs[2], d_init=outs[3])
    torch.cuda.synchronize()
    for g_, o_, r_ in zip(got, outs, ref):
        assert g_ is o_
        assert torch.equal(g_, r_)
    # mismatched sequence inputs are refused; non-contiguous ones are taken as their values
    with pytest.raises(TypeError):
        binding.scan_fwd(x["a"], x["v"].cpu(), x["q"])
    with pytest.raises(ValueError):
        binding.scan_fwd(x["a"], x["v"][:, :-1], x["q"][:, :-1])
    with pytest.raises(ValueError):
        binding.scan_fwd(x["a"], x["v"].float(), x["q"])
    with pytest.raises(ValueError):
        binding.scan_bwd(x["a"], x["v"], x["q"], dy, ckpt=ck.half())
    with pytest.raises(ValueError):
        binding.scan_fwd(x["a"], x["v"], x["q"], init_state=torch.zeros(B, H, Dh + 1, device=DEV))
    # host memory where device memory is needed is refused before any launch
    host_ws = torch.zeros(1 << 20, dtype=torch.uint8)
    with pytest.raises(ValueError):
        binding.scan_fwd(x["a"], x["v"], x["q"], workspace=host_ws)
    with pytest.raises(ValueError):
        binding.scan_bwd(x["a"], x["v"], x["q"], dy, ckpt=ck, workspace=host_ws)
    with pytest.raises(ValueError):
        binding.scan_bwd(x["a"], x["v"], x["q"], dy, ckpt=ck.cpu())
    with pytest.raises(ValueError):
        binding.segment_fwd(x["a"], x["v"], workspace=host_ws)
    with pytest.raises(ValueError):
        binding.segment_bwd(x["a"], x["v"], x["q"], dy, ckpt=ck.cpu())
    vt = x["v"].transpose(1, 2).contiguous().transpose(1, 2)  # same values, strided
    assert not vt.is_contiguous()
    y1, e1 = binding.scan_fwd(x["a"], x["v"], x["q"], deterministic=True)
    y2, e2 = binding.scan_fwd(x["a"], vt, x["q"], deterministic=True)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(e1, e2)


def test_saturated_gates_reach_special_cases():
    """a = +100 gives A = 1 exactly (a prefix sum over t); a = -100 gives A ~ 0 (E = v)."""
    say("saturated gates")
    B, T, H, Dh = 2, 256, 2, 16
    v = synth.normal((B, T, H, Dh), 31, 0, 1, torch.float32)
    q = synth.normal((B, T, H, Dh), 32, 0, 1, torch.float32)
    for val, ref_E in ((100.0, np.cumsum(f64(v), axis=1)), (-100.0, f64(v))):
        a = torch.full_like(v, val)
        y, eT, ck = binding.scan_fwd(a.to(DEV), v.to(DEV), q.to(DEV), mode="direct",
                                     return_ckpt=True)
        torch.cuda.synchronize()
        assert err(eT, ref_E[:, -1]) <= 1e-5
        ckv = ck.view(B, T // 64, H, Dh)
        assert err(ckv, ref_E[:, 63::64]) <= 1e-5
        ry, _ = oracle.scan_fwd(a, v, q, mode=0)
        assert_close("y", y, ry, torch.float32)


def test_workspace_reuse_across_shapes():
    """One cached workspace serves problems of different shapes in turn (the epoch tags keep
    stale look-back words of earlier calls from matching)."""
    say("workspace reuse")
    cases = [(2, 3000, 2, 64, torch.float16), (1, 500, 4, 32, torch.bfloat16),
             (2, 3000, 2, 64, torch.float16), (3, 129, 1, 128, torch.float32)]
    for B, T, H, Dh, dtype in cases + cases:
        x = inputs_cpu(B, T, H, Dh, dtype, seed=B * 1000 + T)
        g = {k: t.to(DEV) for k, t in x.items()}
        y, eT = binding.scan_fwd(g["a"], g["v"], g["q"], mode="controlled")
        torch.cuda.synchronize()
        ry, reT = oracle.scan_fwd(x["a"], x["v"], x["q"], mode=1, threads=8)
        assert_close("y", y, ry, dtype)
        assert_close("eT", eT, reT, state_bar(dtype))
    check_abort_clear()


def test_resume_equals_unsplit():
    """scan(T1) then scan(T2, E0 = E_T1) equals scan(T1 + T2), within tolerance."""
    say("resume")
    B, T1, T2, H, Dh = 2, 1000, 600, 2, 64
    x = inputs_cpu(B, T1 + T2, H, Dh, torch.float16, seed=77)
    g = {k: t.to(DEV) for k, t in x.items()}
    y, eT = binding.scan_fwd(g["a"], g["v"], g["q"], mode="controlled")
    y1, e1 = binding.scan_fwd(g["a"][:, :T1], g["v"][:, :T1], g["q"][:, :T1], mode="controlled")
    y2, e2 = binding.scan_fwd(g["a"][:, T1:], g["v"][:, T1:], g["q"][:, T1:], e1, mode="controlled")
    torch.cuda.synchronize()
    assert err(torch.cat([y1, y2], 1), y) <= 5e-3
    assert err(e2, eT) <= 1e-5


@pytest.mark.parametrize("mode", ["direct", "controlled"])
def test_causality(mode):
    """The readout at t depends on no input after t, and the gradients at t on no upstream
    gradient before t (the pages' "causal behavior" test of page "entangled-state-attention
    0.1.0", on the GPU path).  Every input from a mid-tile step t0 on is redrawn: y before t0
    keeps its bits (deterministic look-back, so a changed carry would show).  Then every dy
    before t0 is redrawn: the gradients from t0 on keep their bits."""
    say(f"causality {mode}")
    B, T, H, Dh, t0 = 2, 3000, 2, 64, 1234
    x = {k: t.to(DEV) for k, t in inputs_cpu(B, T, H, Dh, torch.float16, seed=81, dy=True).items()}
    z = {k: t.to(DEV) for k, t in inputs_cpu(B, T, H, Dh, torch.float16, seed=82, dy=True).items()}
    x2 = {k: x[k].clone() for k in x}
    for k in ("a", "v", "q"):
        x2[k][:, t0:] = z[k][:, t0:]
    y1, e1, ck1 = binding.scan_fwd(x["a"], x["v"], x["q"], mode=mode, return_ckpt=True,
                                   deterministic=True)
    y2, e2, _ = binding.scan_fwd(x2["a"], x2["v"], x2["q"], mode=mode, return_ckpt=True,
                                 deterministic=True)
    torch.cuda.synchronize()
    assert torch.equal(y1[:, :t0], y2[:, :t0])
    assert not torch.equal(y1[:, t0:], y2[:, t0:])
    dy2 = x["dy"].clone()
    dy2[:, :t0] = z["dy"][:, :t0]
    g1 = binding.scan_bwd(x["a"], x["v"], x["q"], x["dy"], ckpt=ck1, mode=mode,
                          deterministic=True)
    g2 = binding.scan_bwd(x["a"], x["v"], x["q"], dy2, ckpt=ck1, mode=mode, deterministic=True)
    torch.cuda.synchronize()
    for a_, b_ in zip(g1[:3], g2[:3]):
        assert torch.equal(a_[:, t0:], b_[:, t0:])
        assert not torch.equal(a_[:, :t0], b_[:, :t0])


# ---------------------------------------------------------------------------------------
# The workloads at full size, compared on sampled batch rows.
# ---------------------------------------------------------------------------------------
def gpu_inputs(wl, T=None, dy=False):
    return synth.make_inputs(wl, device=DEV, T=T, with_dy=dy)


def rows(t, idx):
    return t[idx].to("cpu")


def test_workload_small_fwd_f32():
    wl = synth.WORKLOADS["small_fwd_f32"]
    say(f"workload {wl.name}")
    g = gpu_inputs(wl)
    y, eT = binding.scan_fwd(g["a"], g["v"], g["q"], mode=wl.mode)
    torch.cuda.synchronize()
    ry, reT = oracle.scan_fwd(g["a"].cpu(), g["v"].cpu(), g["q"].cpu(), mode=MODES[wl.mode])
    assert_close("y", y, ry, torch.float32)
    assert_close("eT", eT, reT, torch.float32)


def test_workload_layer_fwd_f16():
    wl = synth.WORKLOADS["layer_fwd_f16"]
    say(f"workload {wl.name}")
    g = gpu_inputs(wl)
    y, eT = binding.scan_fwd(g["a"], g["v"], g["q"], mode=wl.mode)
    torch.cuda.synchronize()
    ry, reT = oracle.scan_fwd(g["a"].cpu(), g["v"].cpu(), g["q"].cpu(), mode=MODES[wl.mode],
                              threads=8)
    assert_close("y", y, ry, torch.float16)
    assert_close("eT", eT, reT, state_bar(torch.float16))


def _fwd_bwd_rows(wl, sample):
    dtype = DT[wl.dtype]
    g = gpu_inputs(wl, dy=True)
    y, eT, ck = binding.scan_fwd(g["a"], g["v"], g["q"], mode=wl.mode, return_ckpt=True)
    da, dv, dq, de0 = binding.scan_bwd(g["a"], g["v"], g["q"], g["dy"], ckpt=ck, mode=wl.mode)
    torch.cuda.synchronize()
    check_abort_clear()
    for b in sample:
        say(f"  row {b}")
        xa, xv, xq, xd = (rows(g[k], [b]) for k in ("a", "v", "q", "dy"))
        ry, reT = oracle.scan_fwd(xa, xv, xq, mode=MODES[wl.mode])
        assert_close(f"y[{b}]", rows(y, [b]), ry, dtype)
        assert_close(f"eT[{b}]", rows(eT, [b]), reT, state_bar(dtype))
        r = oracle.scan_bwd(xa, xv, xq, xd, mode=MODES[wl.mode])
        for name, got, ref in zip(("d_logit", "d_value", "d_query", "d_init"),
                                  (da, dv, dq, de0), r):
            bar = state_bar(dtype) if name == "d_init" else dtype
            assert_close(f"{name}[{b}]", rows(got, [b]), ref, bar)
    del g, y, eT, ck, da, dv, dq, de0
    torch.cuda.empty_cache()


def test_workload_train8k_bf16():
    wl = synth.WORKLOADS["train8k_bf16"]
    say(f"workload {wl.name}")
    _fwd_bwd_rows(wl, [0, 9, 15])


def test_workload_long64k_f16():
    wl = synth.WORKLOADS["long64k_f16"]
    say(f"workload {wl.name}")
    _fwd_bwd_rows(wl, [0, 63])


def test_long64k_shapes_in_fp32_8gib_tensors():
    """The 64K workload's shapes and draws in fp32 storage: every sequence tensor is 8 GiB,
    so element and byte offsets pass 2^31 and 2^32 inside a call."""
    wl = synth.WORKLOADS["long64k_f16"]
    say("64K shapes in fp32 (8 GiB tensors)")
    g = synth.make_inputs(wl, device=DEV, with_dy=True, dtype="f32")
    assert g["a"].numel() * 4 == 8 << 30
    y, eT, ck = binding.scan_fwd(g["a"], g["v"], g["q"], mode=wl.mode, return_ckpt=True)
    da, dv, dq, de0 = binding.scan_bwd(g["a"], g["v"], g["q"], g["dy"], ckpt=ck, mode=wl.mode)
    torch.cuda.synchronize()
    check_abort_clear()
    for b in (0, 63):
        say(f"  row {b}")
        xa, xv, xq, xd = (rows(g[k], [b]) for k in ("a", "v", "q", "dy"))
        ry, reT = oracle.scan_fwd(xa, xv, xq, mode=MODES[wl.mode])
        assert_close(f"y[{b}]", rows(y, [b]), ry, torch.float32)
        assert_close(f"eT[{b}]", rows(eT, [b]), reT, torch.float32)
        r = oracle.scan_bwd(xa, xv, xq, xd, mode=MODES[wl.mode])
        for name, got, ref in zip(("d_logit", "d_value", "d_query", "d_init"),
                                  (da, dv, dq, de0), r):
            assert_close(f"{name}[{b}]", rows(got, [b]), ref, torch.float32)
    del g, y, eT, ck, da, dv, dq, de0
    torch.cuda.empty_cache()


def test_rows_wider_than_a_32_bit_tile_span():
    """C = 8M channels (H = 131072 heads of 64) in fp16: one tile's rows span 2^32 bytes in the
    forward and 2^31 in the backward, beyond the 32-bit lane offsets of the buffer-addressed
    path, so every tile takes the 64-bit-addressed path.  T = 300 leaves ragged last tiles.
    Sampled heads are compared with the oracle (heads are independent)."""
    B, T, H, Dh = 1, 300, 131072, 64
    dt, mode = torch.float16, "controlled"
    say(f"wide rows C={H * Dh}")
    shp = (B, T, H, Dh)
    g = {k: synth.normal(shp, 960 + i, 1.0 if k == "a" else 0.0, 1.0, dt, DEV)
         for i, k in enumerate(("a", "v", "q", "dy"))}
    e0 = synth.random_state(B, H, Dh, 965, DEV)
    dET = synth.random_state(B, H, Dh, 966, DEV)
    y, eT, ck = binding.scan_fwd(g["a"], g["v"], g["q"], e0, mode=mode, return_ckpt=True)
    da, dv, dq, de0 = binding.scan_bwd(g["a"], g["v"], g["q"], g["dy"], e0, dET, ckpt=ck,
                                       mode=mode)
    torch.cuda.synchronize()
    check_abort_clear()
    heads = [0, 1, 4097, H // 2, H - 1]
    c = {k: t[:, :, heads].cpu() for k, t in g.items()}
    ce0, cdET = e0[:, heads].cpu(), dET[:, heads].cpu()
    ry, reT = oracle.scan_fwd(c["a"], c["v"], c["q"], ce0, mode=MODES[mode])
    assert_close("y", y[:, :, heads].cpu(), ry, dt)
    assert_close("eT", eT[:, heads].cpu(), reT, state_bar(dt))
    r = oracle.scan_bwd(c["a"], c["v"], c["q"], c["dy"], ce0, cdET, mode=MODES[mode])
    for name, got, ref in zip(("d_logit", "d_value", "d_query"), (da, dv, dq), r):
        assert_close(name, got[:, :, heads].cpu(), ref, dt)
    assert_close("d_init", de0[:, heads].cpu(), r[3], state_bar(dt))
    del g, y, eT, ck, da, dv, dq, de0
    torch.cuda.empty_cache()


def test_workload_long64k_f8e4m3():
    wl = synth.WORKLOADS["long64k_f8e4m3"]
    say(f"workload {wl.name}")
    _fwd_bwd_rows(wl, [0, 37, 63])


def test_workload_decode_f16():
    """Prefill at every prompt length, then decode steps, against the oracle on sampled rows;
    prefill + steps also equals one longer scan of the same inputs."""
    wl = synth.WORKLOADS["decode_f16"]
    dtype = DT[wl.dtype]
    n_steps = 8
    sample = [0, 131, 255]
    for T in wl.prompts:
        say(f"workload {wl.name} prompt {T}")
        g = gpu_inputs(wl, T=T)
        y, st = binding.scan_fwd(g["a"], g["v"], g["q"], mode=wl.mode)
        torch.cuda.synchronize()
        ry, rst = oracle.scan_fwd(rows(g["a"], sample), rows(g["v"], sample), rows(g["q"], sample),
                                  mode=1, threads=3)
        assert_close("prefill y", rows(y, sample), ry, dtype)
        assert_close("prefill state", rows(st, sample), rst, state_bar(dtype))
        if T != wl.prompts[0]:
            continue
        # decode steps, chained from the prefill state
        seq_a, seq_v, seq_q, ys = [g["a"]], [g["v"]], [g["q"]], []
        for k in range(n_steps):
            s = synth.decode_step_inputs(wl, k, device=DEV)
            ys.append(binding.state_step(s["a"], s["v"], s["q"], st, mode=wl.mode))
            seq_a.append(s["a"][:, None])
            seq_v.append(s["v"][:, None])
            seq_q.append(s["q"][:, None])
            torch.cuda.synchronize()
            ryk, rst = oracle.state_step(rows(s["a"], sample), rows(s["v"], sample),
                                         rows(s["q"], sample), rst, mode=1)
            assert_close(f"step {k} y", rows(ys[-1], sample), ryk, dtype)
            assert_close(f"step {k} state", rows(st, sample), rst, state_bar(dtype))
        # prefill + steps == one scan over prompt + generated tokens
        A, V, Q = (torch.cat(s, 1).contiguous() for s in (seq_a, seq_v, seq_q))
        yl, stl = binding.scan_fwd(A, V, Q, mode=wl.mode)
        torch.cuda.synchronize()
        assert err(st, stl) <= 1e-5
        assert err(torch.stack(ys, 1), yl[:, T:]) <= TOL[dtype]
