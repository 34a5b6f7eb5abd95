"""esa_scan_fwd_noalloc, the forward without a workspace, through the C ABI (ctypes): its
outputs against esa_scan_fwd's on the same inputs, on two calls in a row (the second one
smaller, so it reuses the static scratch array as the first left it), and a refusal of a
problem too large for the array.

With ESA_DETERMINISTIC both entry points fold every carry in the same fixed order, so their
outputs are compared bit for bit as well as against the parity bar; without it both are
compared with the oracle at the bar.
"""
import ctypes
import sys

import pytest
import torch

import oracle
from gated_linear_recurrence_chunked_amd import binding, synth
from helpers import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
P = ctypes.c_void_p


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def ptr(t):
    return P(t.data_ptr()) if t is not None else P(None)


def noalloc_fwd(lib, a, v, q, e0, mode_code, y, eT, ck):
    B, T, H, Dh = a.shape
    stream = P(torch.cuda.current_stream().cuda_stream)
    return lib.esa_scan_fwd_noalloc(B, T, H, Dh, binding.DTYPES[a.dtype], mode_code, ptr(a),
                                    ptr(v), ptr(q), ptr(e0), ptr(y), ptr(eT), ptr(ck), stream)


# the first case is the larger one: the second reuses the array the first left behind
CASES = [((4, 3000, 2, 64), torch.float16, "controlled"),
         ((2, 777, 3, 32), torch.bfloat16, "direct")]


@pytest.mark.parametrize("det", [True, False], ids=["deterministic", "default"])
def test_noalloc_forward_matches_workspace_forward(det):
    lib = binding.load_library()
    for k, (shape, dt, mode) in enumerate(CASES):
        B, T, H, Dh = shape
        say(f"noalloc forward call {k}: {shape} {dt} {mode} det={det}")
        x = {n: synth.normal(shape, 880 + 10 * k + i, 1.0 if n == "a" else 0.0, 1.0, dt)
             for i, n in enumerate("avq")}
        e0 = synth.random_state(B, H, Dh, 890 + k)
        g = {n: t.to(DEV) for n, t in x.items()}
        ge0 = e0.to(DEV)
        ref_y, ref_eT, ref_ck = binding.scan_fwd(g["a"], g["v"], g["q"], ge0, mode=mode,
                                                 return_ckpt=True, deterministic=det)
        y = torch.full_like(g["a"], float("nan"))
        eT = torch.full((B, H, Dh), float("nan"), device=DEV)
        ck = torch.full_like(ref_ck, float("nan"))
        code = binding.MODES[mode] | (binding.DETERMINISTIC if det else 0)
        assert noalloc_fwd(lib, g["a"], g["v"], g["q"], ge0, code, y, eT, ck) == 0
        torch.cuda.synchronize()
        assert_close("y vs esa_scan_fwd", y, ref_y, dt)
        assert_close("final_state vs esa_scan_fwd", eT, ref_eT, torch.float32)
        assert_close("ckpt vs esa_scan_fwd", ck, ref_ck, torch.float32)
        if det:
            assert torch.equal(y, ref_y) and torch.equal(eT, ref_eT) and torch.equal(ck, ref_ck)
        ry, reT = oracle.scan_fwd(x["a"], x["v"], x["q"], e0, mode=binding.MODES[mode],
                                  threads=8)
        assert_close("y vs oracle", y, ry, dt)
        assert_close("final_state vs oracle", eT, reT, torch.float16)


def test_noalloc_forward_refuses_what_does_not_fit():
    """A problem whose look-back words exceed the static array is refused before anything
    runs (its outputs keep their contents); the refused flag and a valid call after it."""
    lib = binding.load_library()
    B, T, H, Dh = 256, 8192, 8, 64  # 64 MiB + 256 B of look-back words: one header too many
    say("noalloc forward: too large")
    a = torch.zeros((B, T, H, Dh), dtype=torch.float16, device=DEV)
    y = torch.full_like(a, 7.0)
    eT = torch.full((B, H, Dh), 7.0, device=DEV)
    stream = P(torch.cuda.current_stream().cuda_stream)
    st = lib.esa_scan_fwd_noalloc(B, T, H, Dh, 1, 1, ptr(a), ptr(a), ptr(a), P(None), ptr(y),
                                  ptr(eT), P(None), stream)
    assert st == 5, st  # ESA_ERR_SCRATCH_LIMIT
    assert "SCRATCH" in lib.esa_status_string(st).decode()
    torch.cuda.synchronize()
    assert bool((eT == 7.0).all()) and bool((y[:, ::97] == 7.0).all())
    # the forced-timeout test flag has no no-allocation instance
    small = torch.zeros((1, 64, 1, 64), dtype=torch.float16, device=DEV)
    ys = torch.empty_like(small)
    assert lib.esa_scan_fwd_noalloc(1, 64, 1, 64, 1, 1 | binding.TEST_FORCE_TIMEOUT, ptr(small),
                                    ptr(small), ptr(small), P(None), ptr(ys), P(None), P(None),
                                    stream) == 1
    del a, y
    torch.cuda.empty_cache()
