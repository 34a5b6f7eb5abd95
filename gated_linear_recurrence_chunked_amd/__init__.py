"""MI355X-native gated linear recurrence (Entangled State Attention hot path).

The compute lives in ``libesa.so`` (hand-written HIP kernels for gfx950 behind a C ABI,
declared in ``include/esa.h``).  This package is a thin binding: argument marshalling and
torch-owned device memory only.  Importing it does not load the library; the first call
does, and fails loudly when the library is missing.
"""
from __future__ import annotations

_BINDING = ["scan_fwd", "scan_bwd", "state_step", "StepPlan", "DecodeGraph", "segment_fwd",
            "segment_bwd", "segment_compose", "workspace_bytes", "ckpt_bytes", "EsaError",
            "library_path", "load_library", "workspace_status", "check_timeouts",
            "set_timeout_checks"]
_AUTOGRAD = ["esa_scan", "ESALayer"]
__all__ = _BINDING + _AUTOGRAD


def __getattr__(name):
    if name in _BINDING:
        from . import binding
        return getattr(binding, name)
    if name in _AUTOGRAD:
        from . import autograd
        return getattr(autograd, name)
    raise AttributeError(name)
