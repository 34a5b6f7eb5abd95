"""Autograd and layer wrappers over the library's scan.

``esa_scan(a, v, q, init_state=None, mode)`` is differentiable: its forward is
``esa_scan_fwd`` (keeping the fp32 state checkpoint), its backward ``esa_scan_bwd``.

``ESALayer`` is the ESA sequence layer of page "entangled-state-attention 0.1.0", section
"Core idea": gate logits, values and queries are projections of x, the scan runs in the
library, and the output projection maps the readout back:

    a = x W_A,  v = x W_V,  q = x W_Q                    (plain GEMMs, no bias)
    y_t = W_O (q_t * Norm(E_t)),  E_t = s_t E_{t-1} + B_t  (library kernels)

with the heads and the prefill / decode_step interface of page "Entangled State
Attention", section "[ QUICK START ]" (``esa = ESA(embd=512, head=8)``,
``out, state = esa.prefill(prompt)``, ``out, state = esa.decode_step(token, state)``).
The projections are ordinary library matrix products; everything of the recurrence runs
in the HIP kernels.
"""
from __future__ import annotations

import math

import torch

from . import binding


class _ScanFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, a, v, q, init_state, mode, deterministic):
        y, final_state, ckpt = binding.scan_fwd(a, v, q, init_state, mode=mode, return_ckpt=True,
                                                deterministic=deterministic)
        ctx.mode = mode
        ctx.deterministic = deterministic
        ctx.has_init = init_state is not None
        ctx.save_for_backward(a, v, q, init_state if init_state is not None else a.new_empty(0),
                              ckpt)
        return y, final_state

    @staticmethod
    def backward(ctx, dy, d_final):
        a, v, q, init_or_ckpt, ckpt = ctx.saved_tensors
        init_state = init_or_ckpt if ctx.has_init else None
        if dy is None:
            dy = torch.zeros_like(a)
        da, dv, dq, d_init = binding.scan_bwd(a, v, q, dy.contiguous(), init_state,
                                              None if d_final is None else d_final.contiguous(),
                                              ckpt=ckpt, mode=ctx.mode,
                                              deterministic=ctx.deterministic)
        return da, dv, dq, (d_init if ctx.has_init else None), None, None


def esa_scan(a, v, q, init_state=None, mode="controlled", deterministic=False):
    """Differentiable scan: returns (y [B,T,H,Dh], final_state fp32 [B,H,Dh]).
    deterministic=True: bitwise reproducible forward and backward."""
    return _ScanFn.apply(a, v, q, init_state, mode, deterministic)


class ESALayer(torch.nn.Module):
    """ESA layer: projections, the library's gated scan with per-head RMSNorm readout, and the
    output projection.  ``dtype`` is the dtype of the weights and of the GEMMs, and by default
    also the scan's storage dtype.  ``scan_dtype`` may instead name one of the 8-bit formats
    (torch.float8_e4m3fn, torch.float8_e5m2): the scan then reads a, v, q and writes its
    readout in that format (the experimental fp8 precision of page "Entangled State
    Attention v2.1", section "3. Precision"), with fp32 arithmetic and state; gradients
    cross the casts as usual.  ``state_dim`` (default ``embd``) is the width of the
    recurrent state, split over the heads, as the ``ESA(dim, state_dim, gate_mode)`` layer of
    page "entangled-state-attention 0.1.0", section "Minimal usage": W_A, W_V, W_Q map embd to
    state_dim and W_O maps it back."""

    def __init__(self, embd: int, head: int, mode: str = "controlled", dtype=torch.float16,
                 device=None, scan_dtype=None, state_dim: int | None = None):
        super().__init__()
        state_dim = embd if state_dim is None else state_dim
        if state_dim % head:
            raise ValueError("state_dim (default embd) must be a multiple of head")
        self.embd, self.head, self.state_dim, self.dh = embd, head, state_dim, state_dim // head
        if self.dh not in (16, 32, 64, 128):
            raise ValueError("head dimension state_dim / head must be 16, 32, 64 or 128")
        if dtype not in (torch.float32, torch.float16, torch.bfloat16):
            # the projections are torch GEMMs in this dtype; 8-bit storage is the scan_dtype
            raise ValueError("ESALayer dtype must be float32, float16 or bfloat16")
        self.scan_dtype = dtype if scan_dtype is None else scan_dtype
        if self.scan_dtype not in binding.DTYPES:
            raise ValueError(f"scan_dtype {self.scan_dtype} is not a storage dtype of the library")
        self.mode = mode
        kw = dict(device=device, dtype=dtype)
        self.W_A = torch.nn.Parameter(torch.empty(embd, state_dim, **kw))
        self.W_V = torch.nn.Parameter(torch.empty(embd, state_dim, **kw))
        self.W_Q = torch.nn.Parameter(torch.empty(embd, state_dim, **kw))
        self.W_O = torch.nn.Parameter(torch.empty(state_dim, embd, **kw))
        self.reset_parameters()

    def reset_parameters(self):
        for w in (self.W_A, self.W_V, self.W_Q, self.W_O):
            bound = 1.0 / math.sqrt(w.shape[0])  # fan-in
            torch.nn.init.uniform_(w, -bound, bound)

    def _project(self, x):
        shp = x.shape[:-1] + (self.head, self.dh)
        a = (x @ self.W_A).reshape(shp).to(self.scan_dtype)
        v = (x @ self.W_V).reshape(shp).to(self.scan_dtype)
        q = (x @ self.W_Q).reshape(shp).to(self.scan_dtype)
        return a, v, q

    def forward(self, x, init_state=None, return_state=False):
        """x: [B, T, embd] -> y [B, T, embd] (and the fp32 state [B, head, state_dim/head])."""
        a, v, q = self._project(x)
        r, state = esa_scan(a.contiguous(), v.contiguous(), q.contiguous(), init_state,
                            mode=self.mode)
        y = r.reshape(x.shape[:-1] + (self.state_dim,)).to(self.W_O.dtype) @ self.W_O
        return (y, state) if return_state else y

    def prefill(self, x, state=None):
        """Full-sequence pass that also returns the compact recurrent state."""
        return self.forward(x, init_state=state, return_state=True)

    @torch.no_grad()
    def decode_step(self, x_t, state):
        """One token: x_t [B, embd]; state fp32 [B, head, dh] is updated in place."""
        a, v, q = self._project(x_t)
        r = binding.state_step(a.contiguous(), v.contiguous(), q.contiguous(), state,
                               mode=self.mode)
        return r.reshape(x_t.shape[:-1] + (self.state_dim,)).to(self.W_O.dtype) @ self.W_O, state
