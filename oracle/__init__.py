"""Oracle for the ESA gated linear recurrence: fp64, sequential, CPU.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this package.  The product library never loads it, and it
shares no code with the HIP path.

The arithmetic lives in ``esa_oracle.c`` (plain C, fp64, built with gcc and floating-point
contraction off).  This module only builds that file, marshals numpy arrays into it, and
splits batch rows over threads (each row is an independent, sequential computation).

Layouts follow the library: sequences are ``[B, T, H, Dh]`` with Dh fastest; states are
``[B, H, Dh]``.  Modes: 0 = direct (A = sigma(a), B = v), 1 = controlled
(A = g = sigma(a), B = (1 - g) v), per page "entangled-state-attention 0.1.0", section
"Core idea".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "esa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_esa.so")
_lock = threading.Lock()
_lib = None

DIRECT = 0
CONTROLLED = 1


def build(force: bool = False) -> str:
    """Compile esa_oracle.c into liboracle_esa.so (gcc, -O2, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
               "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            I = ctypes.c_int64
            lib.oracle_sigmoid.argtypes = [ctypes.c_double]
            lib.oracle_sigmoid.restype = ctypes.c_double
            lib.oracle_rmsnorm_eps.argtypes = []
            lib.oracle_rmsnorm_eps.restype = ctypes.c_double
            lib.oracle_recurrence.argtypes = [I, I, P, P, P, P]
            lib.oracle_recurrence.restype = None
            lib.oracle_gates.argtypes = [I, ctypes.c_int, P, P, P, P]
            lib.oracle_gates.restype = None
            lib.oracle_readout.argtypes = [I, I, P, P, P]
            lib.oracle_readout.restype = None
            lib.oracle_scan_fwd.argtypes = [I, I, I, I, I, ctypes.c_int, P, P, P, P, P, P, P]
            lib.oracle_scan_fwd.restype = ctypes.c_int
            lib.oracle_scan_bwd.argtypes = [I, I, I, I, I, ctypes.c_int,
                                            P, P, P, P, P, P, P, P, P, P]
            lib.oracle_scan_bwd.restype = ctypes.c_int
            lib.oracle_state_step.argtypes = [I, I, I, ctypes.c_int, P, P, P, P, P]
            lib.oracle_state_step.restype = None
            _lib = lib
    return _lib


def _f64(x):
    """Exact upcast of an input (numpy array or CPU torch tensor) to contiguous fp64."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: fp16/bf16/fp32 -> fp64 is exact
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _p(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def _mode(mode) -> int:
    if isinstance(mode, str):
        return {"direct": DIRECT, "controlled": CONTROLLED}[mode]
    return int(mode)


def sigmoid(x: float) -> float:
    return _load().oracle_sigmoid(float(x))


def rmsnorm_eps() -> float:
    return _load().oracle_rmsnorm_eps()


def recurrence(A, Bt, E0=None):
    """E_t = A_t * E_{t-1} + B_t over the last axis as lanes: A, Bt are [T, nl]."""
    A, Bt, E0 = _f64(A), _f64(Bt), _f64(E0)
    T, nl = A.shape
    E = np.empty_like(A)
    _load().oracle_recurrence(T, nl, _p(A), _p(Bt), _p(E0), _p(E))
    return E


def gates(a, v, mode):
    a, v = _f64(a), _f64(v)
    A = np.empty_like(a)
    Bt = np.empty_like(a)
    _load().oracle_gates(a.size, _mode(mode), _p(a), _p(v), _p(A), _p(Bt))
    return A, Bt


def readout(E, q, Dh):
    E, q = _f64(E), _f64(q)
    y = np.empty_like(E)
    _load().oracle_readout(E.size // Dh, Dh, _p(E), _p(q), _p(y))
    return y


def _rows(B, threads):
    threads = max(1, min(int(threads or 1), B))
    step = (B + threads - 1) // threads
    return [(b, min(B, b + step)) for b in range(0, B, step)]


def scan_fwd(a, v, q, e0=None, mode=CONTROLLED, states=False, threads=1):
    """Forward scan with readout.  Returns (y, eT) or (y, eT, E_all) when states=True.

    a, v, q: [B, T, H, Dh]; e0: [B, H, Dh] or None.  q may be None (no readout; y is None).
    """
    a, v, q, e0 = _f64(a), _f64(v), _f64(q), _f64(e0)
    B, T, H, Dh = a.shape
    y = np.empty_like(a) if q is not None else None
    eT = np.empty((B, H, Dh), dtype=np.float64)
    E_all = np.empty_like(a) if states else None
    lib = _load()

    def run(r):
        rc = lib.oracle_scan_fwd(r[0], r[1], T, H, Dh, _mode(mode), _p(a), _p(v), _p(q),
                                 _p(e0), _p(y), _p(eT), _p(E_all))
        if rc:
            raise MemoryError("oracle_scan_fwd: out of memory")

    parts = _rows(B, threads)
    if len(parts) == 1:
        run(parts[0])
    else:
        with ThreadPoolExecutor(len(parts)) as ex:
            list(ex.map(run, parts))
    return (y, eT, E_all) if states else (y, eT)


def scan_bwd(a, v, q, dy, e0=None, dET=None, mode=CONTROLLED, threads=1):
    """Backward of scan_fwd.  Returns (da, dv, dq, de0)."""
    a, v, q, dy, e0, dET = (_f64(x) for x in (a, v, q, dy, e0, dET))
    B, T, H, Dh = a.shape
    da = np.empty_like(a)
    dv = np.empty_like(a)
    dq = np.empty_like(a)
    de0 = np.empty((B, H, Dh), dtype=np.float64)
    lib = _load()

    def run(r):
        rc = lib.oracle_scan_bwd(r[0], r[1], T, H, Dh, _mode(mode), _p(a), _p(v), _p(q),
                                 _p(e0), _p(dy), _p(dET), _p(da), _p(dv), _p(dq), _p(de0))
        if rc:
            raise MemoryError("oracle_scan_bwd: out of memory")

    parts = _rows(B, threads)
    if len(parts) == 1:
        run(parts[0])
    else:
        with ThreadPoolExecutor(len(parts)) as ex:
            list(ex.map(run, parts))
    return da, dv, dq, de0


def state_step(a, v, q, state, mode=CONTROLLED):
    """One-token update.  a, v, q, state: [B, H, Dh].  Returns (y, new_state)."""
    a, v, q = _f64(a), _f64(v), _f64(q)
    st = _f64(state).copy()
    B, H, Dh = a.shape
    y = np.empty_like(a)
    _load().oracle_state_step(B, H, Dh, _mode(mode), _p(a), _p(v), _p(q), _p(st), _p(y))
    return y, st
