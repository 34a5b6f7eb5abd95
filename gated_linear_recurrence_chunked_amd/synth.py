"""Seeded synthetic inputs shaped like the ESA pages' workloads.

This module holds no part of the method's arithmetic: it only draws normal random numbers
with torch's seeded generators and casts them to the storage dtype (round to nearest even).
Both the GPU path and the oracle take their inputs from here.

Workloads (all sequences are [B, T, H, Dh], Dh fastest; states [B, H, Dh] fp32):

  small_fwd_f32     B=1,   T=256,   H=2, Dh=16  fp32 direct      a, v, q ~ N(0, 1)
  layer_fwd_f16     B=16,  T=1024,  H=4, Dh=32  fp16 controlled  a ~ N(0, 1.5), v, q ~ N(0, 1)
                    (the ESA layer example embd=128, head=4, batch=16, block=1024 of page
                    "Entangled State Attention v2.1", section "1. ESA layer")
  long64k_f16       B=64,  T=65536, H=8, Dh=64  fp16 controlled  a ~ N(2, 1), v, q, dy ~ N(0, 1)
                    (64K context, batch 64, FP16 of page "Entangled State Attention",
                    "[ H100 / LONG CONTEXT ]"; H=8, C=512 from its "[ QUICK START ]")
  train8k_bf16      B=16,  T=8192,  H=8, Dh=64  bf16 direct      a ~ N(1, 1), v, q, dy ~ N(0, 1)
  decode_f16        B=256, T in {512, 1024, 4096, 8192}, H=8, Dh=64, fp16 controlled, all
                    N(0, 1), then 1024 one-token steps with fresh N(0, 1) inputs
                    (prompt lengths of "[ GENERATION / MEMORY ]" on the same page)
  long64k_f8e4m3    the long64k_f16 shapes and draws, stored in the OCP E4M3 8-bit format
                    (the experimental fp8 precision mode of page "Entangled State Attention
                    v2.1", section "3. Precision")

The second parameter of N(mu, s) is the standard deviation.  Seed of tensor k of workload
number w is 1000 * w + k with k = 0 (a), 1 (v), 2 (q), 3 (dy), 4 + step (decode draws; the
three per-step tensors use sub-streams 0, 1, 2 of that seed).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    B: int
    T: int
    H: int
    Dh: int
    dtype: str  # "f32" | "f16" | "bf16"
    mode: str  # "direct" | "controlled"
    a_mean: float = 0.0
    a_std: float = 1.0
    prompts: tuple = field(default_factory=tuple)
    steps: int = 0


WORKLOADS = {
    "small_fwd_f32": Workload("small_fwd_f32", 1, 1, 256, 2, 16, "f32", "direct", 0.0, 1.0),
    "layer_fwd_f16": Workload("layer_fwd_f16", 2, 16, 1024, 4, 32, "f16", "controlled", 0.0, 1.5),
    "long64k_f16": Workload("long64k_f16", 3, 64, 65536, 8, 64, "f16", "controlled", 2.0, 1.0),
    "train8k_bf16": Workload("train8k_bf16", 4, 16, 8192, 8, 64, "bf16", "direct", 1.0, 1.0),
    "decode_f16": Workload("decode_f16", 5, 256, 512, 8, 64, "f16", "controlled", 0.0, 1.0,
                           prompts=(512, 1024, 4096, 8192), steps=1024),
    "long64k_f8e4m3": Workload("long64k_f8e4m3", 6, 64, 65536, 8, 64, "f8e4m3", "controlled",
                               2.0, 1.0),
}

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
                "f8e4m3": torch.float8_e4m3fn, "f8e5m2": torch.float8_e5m2}


def torch_dtype(name: str) -> torch.dtype:
    return TORCH_DTYPES[name]


def normal(shape, seed: int, mean: float = 0.0, std: float = 1.0, dtype=torch.float32,
           device="cpu", chunk_elems: int = 1 << 28) -> torch.Tensor:
    """N(mean, std) draws from a generator seeded with `seed`, cast to `dtype` (RNE).

    Large tensors are drawn in chunks along the first axis from one generator, so peak
    temporary memory stays bounded; the values depend only on (shape, seed, device).
    """
    shape = tuple(int(s) for s in shape)
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    out = torch.empty(shape, dtype=dtype, device=device)
    if out.numel() == 0:
        return out
    rows = shape[0]
    per_row = out.numel() // rows
    step = max(1, chunk_elems // max(1, per_row))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        x = torch.randn((r1 - r0,) + shape[1:], generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        if mean != 0.0:
            x.add_(mean)
        out[r0:r1].copy_(x)
        del x
    return out


def make_inputs(wl: Workload | str, device="cpu", B=None, T=None, with_dy=False,
                dtype=None, seed_base=None):
    """Inputs a, v, q (and dy) for a workload; B, T and dtype may be overridden."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    B = wl.B if B is None else B
    T = wl.T if T is None else T
    dt = torch_dtype(dtype or wl.dtype)
    base = 1000 * wl.index if seed_base is None else seed_base
    shape = (B, T, wl.H, wl.Dh)
    out = {
        "a": normal(shape, base + 0, wl.a_mean, wl.a_std, dt, device),
        "v": normal(shape, base + 1, 0.0, 1.0, dt, device),
        "q": normal(shape, base + 2, 0.0, 1.0, dt, device),
    }
    if with_dy:
        out["dy"] = normal(shape, base + 3, 0.0, 1.0, dt, device)
    return out


def decode_step_inputs(wl: Workload | str, step: int, device="cpu", dtype=None, B=None):
    """Per-step one-token inputs a, v, q ([B, H, Dh]) for decode step `step`."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    B = wl.B if B is None else B
    dt = torch_dtype(dtype or wl.dtype)
    seed = 1000 * wl.index + 4 + step
    shape = (B, wl.H, wl.Dh)
    return {
        "a": normal(shape, seed * 8 + 0, wl.a_mean, wl.a_std, dt, device),
        "v": normal(shape, seed * 8 + 1, 0.0, 1.0, dt, device),
        "q": normal(shape, seed * 8 + 2, 0.0, 1.0, dt, device),
    }


def random_state(B, H, Dh, seed, device="cpu", std=1.0):
    """An fp32 [B, H, Dh] state drawn from N(0, std)."""
    return normal((B, H, Dh), seed, 0.0, std, torch.float32, device)
