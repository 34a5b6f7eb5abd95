"""A look-back failure forced from the host with the ESA_TEST_FORCE_TIMEOUT mode flag: the
first tile of every chain withholds its published values and the wait's poll limit is
small, so every wait on a withheld value ends by timing out.  The call still returns; the
workspace records the timeout (header word 3, read through esa_workspace_status, which then
returns ESA_ERR_TIMEOUT); the outputs of the first tile are exact and every output that
depends on the withheld values is NaN.  Later launches on the same workspace are not
affected, and esa_workspace_init clears the record.  The binding surfaces the record as an
EsaError, after every call in its debug mode or at check_timeouts()."""
import ctypes
import sys

import pytest
import torch

from gated_linear_recurrence_chunked_amd import binding, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def header(ws):
    return ws[:16].view(torch.int32)


def first_nan_step(t):
    """Index along T of the first step holding a NaN ([B, T, H, Dh] tensor), or T."""
    bad = torch.isnan(t.float()).flatten(2).any(-1).any(0)
    idx = torch.nonzero(bad)
    return int(idx[0]) if len(idx) else t.shape[1]


def last_nan_step(t):
    bad = torch.isnan(t.float()).flatten(2).any(-1).any(0)
    idx = torch.nonzero(bad)
    return int(idx[-1]) if len(idx) else -1


@pytest.mark.parametrize("det", [False, True])
def test_withheld_first_tile_times_out_to_nan(det):
    B, T, H, Dh = 2, 1000, 2, 64
    dt, mode = torch.float16, "controlled"
    say(f"forced look-back failure det={det}")
    shp = (B, T, H, Dh)
    x = {k: synth.normal(shp, 970 + i, 1.0 if k == "a" else 0.0, 1.0, dt).to(DEV)
         for i, k in enumerate(("a", "v", "q", "dy"))}
    y0, eT0, ck0 = binding.scan_fwd(x["a"], x["v"], x["q"], mode=mode, return_ckpt=True,
                                    deterministic=True)
    g0 = binding.scan_bwd(x["a"], x["v"], x["q"], x["dy"], ckpt=ck0, mode=mode,
                          deterministic=True)
    ws = torch.zeros(binding.workspace_bytes(B, T, H, Dh, dt), dtype=torch.uint8, device=DEV)

    forced = binding.MODES[mode] | binding.TEST_FORCE_TIMEOUT
    h = header(ws)
    # forward: the chain's first tile withholds; every later tile's carry is NaN
    y, eT, ck = binding.scan_fwd(x["a"], x["v"], x["q"], mode=forced, return_ckpt=True,
                                 workspace=ws, deterministic=det)
    torch.cuda.synchronize()
    assert int(h[3]) != 0, "the timeout is recorded"
    assert binding.workspace_status(ws)["timeout_tag"] == int(h[3]) & 0xffffffff
    k = first_nan_step(y)
    say(f"  forward: exact through step {k - 1}, NaN from step {k}")
    assert 0 < k < T and k % 64 == 0
    assert torch.equal(y[:, :k], y0[:, :k])
    assert torch.isnan(y[:, k:].float()).all()
    assert torch.isnan(eT).all()

    # backward (from the good checkpoint): the chain starts at the last tile
    h.zero_()
    da, dv, dq, de0 = binding.scan_bwd(x["a"], x["v"], x["q"], x["dy"], ckpt=ck0, mode=forced,
                                       workspace=ws, deterministic=det)
    torch.cuda.synchronize()
    assert int(h[3]) != 0
    j = last_nan_step(da)
    say(f"  backward: NaN through step {j}, exact from step {j + 1}")
    assert 0 <= j < T - 1 and (j + 1) % 64 == 0
    for got, ref in ((da, g0[0]), (dv, g0[1])):
        assert torch.equal(got[:, j + 1:], ref[:, j + 1:])
        assert torch.isnan(got[:, :j + 1].float()).all()
    assert torch.equal(dq, g0[2])  # the query gradient needs no carry
    assert torch.isnan(de0).all()

    # a normal launch on the same workspace is unaffected by the recorded timeout
    y2, eT2 = binding.scan_fwd(x["a"], x["v"], x["q"], mode=mode, workspace=ws,
                               deterministic=True)
    torch.cuda.synchronize()
    assert torch.equal(y2, y0) and torch.equal(eT2, eT0)
    assert int(h[3]) != 0
    # re-initialised through the library, the workspace's record is clear again
    lib = binding.load_library()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.esa_workspace_init(ctypes.c_void_p(ws.data_ptr()), ws.numel(), stream) == 0
    y1, eT1, ck1 = binding.scan_fwd(x["a"], x["v"], x["q"], mode=mode, return_ckpt=True,
                                    workspace=ws, deterministic=True)
    g1 = binding.scan_bwd(x["a"], x["v"], x["q"], x["dy"], ckpt=ck1, mode=mode, workspace=ws,
                          deterministic=True)
    torch.cuda.synchronize()
    assert int(h[3]) == 0
    assert torch.equal(y1, y0) and torch.equal(eT1, eT0)
    for a_, b_ in zip(g1, g0):
        assert torch.equal(a_, b_)


def test_binding_surfaces_a_timeout():
    """A timed-out wait reaches the caller as EsaError(ESA_ERR_TIMEOUT): after the call in the
    binding's debug mode, or from check_timeouts() for the binding's cached workspaces; each
    timeout is reported once."""
    B, T, H, Dh = 2, 1000, 2, 64
    dt = torch.float16
    say("timeout surfaced through the binding")
    shp = (B, T, H, Dh)
    x = {k: synth.normal(shp, 980 + i, 1.0 if k == "a" else 0.0, 1.0, dt).to(DEV)
         for i, k in enumerate(("a", "v", "q"))}
    forced = binding.MODES["controlled"] | binding.TEST_FORCE_TIMEOUT
    binding.check_timeouts()  # nothing recorded so far
    binding.set_timeout_checks(True)
    try:
        with pytest.raises(binding.EsaError) as ei:
            binding.scan_fwd(x["a"], x["v"], x["q"], mode=forced)
        assert ei.value.status == binding.ESA_ERR_TIMEOUT
        binding.scan_fwd(x["a"], x["v"], x["q"], mode="controlled")  # reported once: clean now
    finally:
        binding.set_timeout_checks(False)
    binding.scan_fwd(x["a"], x["v"], x["q"], mode=forced)
    with pytest.raises(binding.EsaError) as ei:
        binding.check_timeouts()
    assert ei.value.status == binding.ESA_ERR_TIMEOUT
    binding.check_timeouts()
