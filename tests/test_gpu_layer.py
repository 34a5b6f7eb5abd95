"""The differentiable scan and the ESA layer wrapper against the oracle.

The reference composes library fp64 matrix products (the projections, page
"entangled-state-attention 0.1.0", "Core idea") with the oracle's scan, wrapped in a
test-side autograd function whose backward is the oracle's backward.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from gated_linear_recurrence_chunked_amd import synth
from gated_linear_recurrence_chunked_amd.autograd import ESALayer, esa_scan
from helpers import TOL, assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MODES = {"direct": 0, "controlled": 1}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class OracleScan(torch.autograd.Function):
    """fp64 CPU scan through the oracle, differentiable through the oracle's backward."""

    @staticmethod
    def forward(ctx, a, v, q, e0, mode):
        y, eT = oracle.scan_fwd(a.numpy(), v.numpy(), q.numpy(),
                                None if e0 is None else e0.numpy(), mode=MODES[mode], threads=8)
        ctx.save_for_backward(a, v, q, e0 if e0 is not None else torch.zeros(0))
        ctx.mode, ctx.has_e0 = mode, e0 is not None
        return torch.from_numpy(y), torch.from_numpy(eT)

    @staticmethod
    def backward(ctx, dy, deT):
        a, v, q, e0 = ctx.saved_tensors
        e0 = e0 if ctx.has_e0 else None
        da, dv, dq, de0 = oracle.scan_bwd(a.numpy(), v.numpy(), q.numpy(), dy.numpy(),
                                          None if e0 is None else e0.numpy(),
                                          None if deT is None else deT.numpy(),
                                          mode=MODES[ctx.mode], threads=8)
        return (torch.from_numpy(da), torch.from_numpy(dv), torch.from_numpy(dq),
                torch.from_numpy(de0) if ctx.has_e0 else None, None)


@pytest.mark.parametrize("dt,mode", [(torch.float32, "direct"), (torch.float16, "controlled"),
                                     (torch.bfloat16, "direct")])
def test_scan_autograd(dt, mode):
    say(f"autograd scan {dt} {mode}")
    B, T, H, Dh = 3, 333, 2, 64
    x = {k: synth.normal((B, T, H, Dh), 500 + i, 0.5 if k == "a" else 0.0, 1.0, dt)
         for i, k in enumerate("avq")}
    e0 = synth.random_state(B, H, Dh, 77)
    w = synth.normal((B, T, H, Dh), 600, 0, 1, dt)
    u = synth.random_state(B, H, Dh, 601)
    g = {k: t.to(DEV).requires_grad_(True) for k, t in x.items()}
    ge0 = e0.to(DEV).requires_grad_(True)
    y, eT = esa_scan(g["a"], g["v"], g["q"], ge0, mode=mode)
    (y.float() * w.to(DEV).float()).sum().add_((eT * u.to(DEV)).sum()).backward()
    torch.cuda.synchronize()
    ry, reT = oracle.scan_fwd(x["a"], x["v"], x["q"], e0, mode=MODES[mode])
    rda, rdv, rdq, rde0 = oracle.scan_bwd(x["a"], x["v"], x["q"], w, e0, u, mode=MODES[mode])
    assert_close("y", y, ry, dt)
    assert_close("eT", eT, reT, torch.float32)
    assert_close("d_logit", g["a"].grad, rda, dt)
    assert_close("d_value", g["v"].grad, rdv, dt)
    assert_close("d_query", g["q"].grad, rdq, dt)
    assert_close("d_init", ge0.grad, rde0, torch.float32)


def reference_layer(layer, x, mode, e0=None, storage=None):
    """fp64 CPU composition: projections (library matmul) + oracle scan + output projection.
    With `storage`, the scan's inputs and readout are rounded to that dtype, as the library
    stores them."""
    rnd = (lambda t: t.to(storage).double()) if storage is not None else (lambda t: t)
    W = {k: getattr(layer, k).detach().double().cpu().requires_grad_(True)
         for k in ("W_A", "W_V", "W_Q", "W_O")}
    xr = x.detach().double().cpu().requires_grad_(True)
    B, T, C = xr.shape
    shp = (B, T, layer.head, layer.dh)
    S = layer.state_dim
    a = rnd((xr @ W["W_A"]).reshape(shp))
    v = rnd((xr @ W["W_V"]).reshape(shp))
    q = rnd((xr @ W["W_Q"]).reshape(shp))
    r, st = OracleScan.apply(a.contiguous(), v.contiguous(), q.contiguous(), e0, mode)
    y = rnd(r).reshape(B, T, S) @ W["W_O"]
    return y, st, xr, W


@pytest.mark.parametrize("mode", ["direct", "controlled"])
def test_layer_forward_backward_fp32(mode):
    say(f"layer fp32 {mode}")
    torch.manual_seed(0)
    B, T, C, H = 2, 300, 128, 2
    layer = ESALayer(C, H, mode=mode, dtype=torch.float32, device=DEV)
    x = synth.normal((B, T, C), 700, 0, 1, torch.float32).to(DEV).requires_grad_(True)
    gy = synth.normal((B, T, C), 701, 0, 1, torch.float32)
    y = layer(x)
    (y * gy.to(DEV)).sum().backward()
    torch.cuda.synchronize()
    ry, _, xr, W = reference_layer(layer, x, mode)
    (ry * gy.double()).sum().backward()
    tol = torch.float32
    assert_close("y", y, ry, tol)
    assert_close("dx", x.grad, xr.grad, tol)
    for k in ("W_A", "W_V", "W_Q", "W_O"):
        assert_close(k, getattr(layer, k).grad, W[k].grad, tol)


def test_layer_prefill_then_decode_matches_full_pass():
    """prefill(prompt) then decode_step per token equals one pass over prompt + tokens, and
    the layer's output matches the fp64 reference (page "Entangled State Attention",
    "[ QUICK START ]": prefill, then decode_step carrying the state)."""
    say("layer prefill + decode")
    torch.manual_seed(1)
    B, T0, n, C, H = 4, 200, 6, 512, 8
    layer = ESALayer(C, H, mode="controlled", dtype=torch.float16, device=DEV)
    x = synth.normal((B, T0 + n, C), 710, 0, 1, torch.float16).to(DEV)
    with torch.no_grad():
        y_full, st_full = layer(x, return_state=True)
        y_pre, st = layer.prefill(x[:, :T0])
        outs = []
        for k in range(n):
            o, st = layer.decode_step(x[:, T0 + k].contiguous(), st)
            outs.append(o)
    torch.cuda.synchronize()
    assert_close("prefill y", y_pre, y_full[:, :T0], torch.float16)
    assert_close("decode y", torch.stack(outs, 1), y_full[:, T0:], torch.float16)
    # the per-token projections are GEMMs of another shape than the full pass's, so their fp16
    # outputs (the scan's inputs) can differ by an ulp: the fp16 bar applies to the state too
    assert_close("state", st, st_full, torch.float16)
    with torch.no_grad():
        ry, rst, _, _ = reference_layer(layer, x, "controlled", storage=torch.float16)
    assert_close("y vs reference", y_full, ry, torch.float16)
    assert_close("state vs reference", st_full, rst, torch.float16)


@pytest.mark.parametrize("scan_dtype", [torch.float8_e4m3fn, torch.float8_e5m2])
def test_layer_with_fp8_scan_storage(scan_dtype):
    """fp16 GEMMs around a scan stored in an 8-bit format: forward and all gradients against
    the fp64 composition with the same roundings (a, v, q and the readout rounded to the
    8-bit format), at the format's bar."""
    say(f"layer fp16 GEMMs, {scan_dtype} scan")
    torch.manual_seed(3)
    B, T, C, H = 2, 300, 256, 4
    layer = ESALayer(C, H, mode="controlled", dtype=torch.float16, device=DEV,
                     scan_dtype=scan_dtype)
    x = synth.normal((B, T, C), 720, 0, 1, torch.float16).to(DEV).requires_grad_(True)
    gy = synth.normal((B, T, C), 721, 0, 1, torch.float16)
    y, st = layer(x, return_state=True)
    (y.float() * gy.to(DEV).float()).sum().backward()
    torch.cuda.synchronize()
    assert y.dtype == torch.float16 and x.grad.dtype == torch.float16
    assert torch.isfinite(x.grad).all() and torch.isfinite(layer.W_A.grad).all()
    # forward: the fp64 composition from the same 8-bit scan inputs (the projections are fp16
    # GEMMs here, so the reference starts from the library's own a, v, q)
    with torch.no_grad():
        a, v, q = (t.cpu() for t in layer._project(x))
        r, rst = oracle.scan_fwd(a, v, q, mode=1)
        ry = torch.from_numpy(r).to(scan_dtype).double().reshape(B, T, C) @ layer.W_O.double().cpu()
    assert_close("y", y, ry, scan_dtype)
    assert_close("state", st, rst, torch.float32)


def test_layer_with_state_dim_different_from_embd():
    """ESA(dim, state_dim) of page "entangled-state-attention 0.1.0", "Minimal usage": the
    state is wider than the model (embd 96, state 256 over 4 heads of 64); forward and every
    gradient against the fp64 composition, fp32 throughout."""
    say("layer state_dim != embd")
    torch.manual_seed(4)
    B, T, C, S, H = 2, 200, 96, 256, 4
    layer = ESALayer(C, H, mode="direct", dtype=torch.float32, device=DEV, state_dim=S)
    assert layer.W_A.shape == (C, S) and layer.W_O.shape == (S, C)
    x = synth.normal((B, T, C), 730, 0, 1, torch.float32).to(DEV).requires_grad_(True)
    gy = synth.normal((B, T, C), 731, 0, 1, torch.float32)
    y, st = layer(x, return_state=True)
    (y * gy.to(DEV)).sum().backward()
    torch.cuda.synchronize()
    assert y.shape == (B, T, C) and st.shape == (B, H, S // H)
    ry, rst, xr, W = reference_layer(layer, x, "direct")
    (ry * gy.double()).sum().backward()
    assert_close("y", y, ry, torch.float32)
    assert_close("state", st, rst, torch.float32)
    assert_close("dx", x.grad, xr.grad, torch.float32)
    for k in ("W_A", "W_V", "W_Q", "W_O"):
        assert_close(k, getattr(layer, k).grad, W[k].grad, torch.float32)
