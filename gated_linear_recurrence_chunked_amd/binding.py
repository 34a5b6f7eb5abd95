"""ctypes binding of libesa.so (include/esa.h), with torch for device memory and streams.

Argument marshalling only: every step of the computation runs in the library's HIP
kernels.  When the library is missing, every call raises; there is no fallback path.

    y, final_state = scan_fwd(a, v, q, init_state=None, mode="controlled")
    y, final_state, ckpt = scan_fwd(a, v, q, mode="controlled", return_ckpt=True)
    da, dv, dq, d_init = scan_bwd(a, v, q, dy, init_state=None, d_final_state=None,
                                  ckpt=None, mode="controlled")
    y = state_step(a, v, q, state, mode="controlled")        # state: fp32, updated in place

Sequence segments (the scan over T cut into consecutive pieces, e.g. one per device):

    seg_state, seg_prod = segment_fwd(a_k, v_k)              # per segment, from a zero state
    carry, final = segment_compose(P_all, E_all, init_state)  # [nseg, B, H, Dh] stacks
    seg_d_init = segment_bwd(a_k, v_k, q_k, dy_k, carry[k], ckpt_k)
    dcarry, d_init = segment_compose(P_all, D_all, d_final_state, reverse=True)

scan_fwd, scan_bwd, state_step and StepPlan go through _esa_torch, a small C++ binding of
the same C ABI built beside libesa.so that takes torch tensors directly (a few microseconds
of host time a call, against 5-17 us through ctypes with the checks in Python); the segment
calls and the size queries go through ctypes.

Sequence tensors are [B, T, H, Dh] (fp32, fp16, bf16, or the OCP 8-bit formats
float8_e4m3fn / float8_e5m2; one dtype per call); states are fp32 [B, H, Dh].
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libesa.so"

ESA_OK = 0
STATUS_NAMES = {0: "ESA_OK", 1: "ESA_ERR_INVALID_ARG", 2: "ESA_ERR_UNSUPPORTED",
                3: "ESA_ERR_WORKSPACE", 4: "ESA_ERR_HIP"}
DTYPES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2, torch.float8_e4m3fn: 3,
          torch.float8_e5m2: 4}
MODES = {"direct": 0, "controlled": 1}
DETERMINISTIC = 0x100  # ESA_DETERMINISTIC: OR-ed into the mode, bitwise reproducible scans
TEST_FORCE_TIMEOUT = 0x200  # ESA_TEST_FORCE_TIMEOUT: a look-back timeout forced for tests

# every function include/esa.h declares: name -> (restype, argtypes)
_P = ctypes.c_void_p
_I = ctypes.c_int64
_C = ctypes.c_int
_Z = ctypes.c_size_t
SIGNATURES = {
    "esa_abi_version": (_C, []),
    "esa_status_string": (ctypes.c_char_p, [_C]),
    "esa_scan_workspace_bytes": (_Z, [_I, _I, _I, _I, _C]),
    "esa_scan_ckpt_bytes": (_Z, [_I, _I, _I, _I]),
    "esa_workspace_init": (_C, [_P, _Z, _P]),
    "esa_scan_fwd": (_C, [_I, _I, _I, _I, _C, _C, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "esa_scan_bwd": (_C, [_I, _I, _I, _I, _C, _C, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                          _P, _P, _Z, _P]),
    "esa_state_step": (_C, [_I, _I, _I, _C, _C, _P, _P, _P, _P, _P, _P]),
    "esa_scan_segment_fwd": (_C, [_I, _I, _I, _I, _C, _C, _P, _P, _P, _P, _P, _Z, _P]),
    "esa_scan_segment_bwd": (_C, [_I, _I, _I, _I, _C, _C, _P, _P, _P, _P, _P, _P, _P, _P, _Z,
                                  _P]),
    "esa_segment_compose": (_C, [_I, _I, _C, _P, _P, _P, _P, _P, _P]),
}

_lock = threading.Lock()
_lib = None
_workspaces: dict = {}


def library_path() -> str:
    return os.path.join(_HERE, LIB_NAME)


_ext = None


def _torch_ext():
    """The torch-tensor call path of esa_scan_fwd, esa_scan_bwd and esa_state_step
    (_esa_torch, built beside libesa.so): the same C ABI without ctypes marshalling.
    Raises if it has not been built."""
    global _ext
    if _ext is None:
        load_library()
        try:
            from . import _esa_torch
        except ImportError as e:
            raise RuntimeError(
                "the _esa_torch extension is missing: build it with "
                "`python -m gated_linear_recurrence_chunked_amd.build`") from e
        _ext = _esa_torch
    return _ext


def load_library():
    """Load libesa.so (once).  Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            path = library_path()
            if not os.path.exists(path):
                raise RuntimeError(
                    f"{path} is missing: build it first with "
                    "`python -m gated_linear_recurrence_chunked_amd.build` (hipcc, gfx950)")
            lib = ctypes.CDLL(path)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


class EsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = load_library().esa_status_string(status).decode()
        super().__init__(f"{where}: {msg}")
        self.status = status


def _check(status: int, where: str):
    if status != ESA_OK:
        raise EsaError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _raw_stream(index: int) -> int:
    """The current HIP stream of device `index` as an integer handle (torch's raw accessor,
    without building a Python stream object: a decode step calls this once per token)."""
    return torch._C._cuda_getCurrentRawStream(index)


def _stream_handle(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(_raw_stream(device.index))


class _OnDevice:
    """Makes `index` the current device for the call, and skips the switch when it already
    is (the common case; a device switch costs more host time than a decode step's launch)."""
    __slots__ = ("index", "prev")

    def __init__(self, index: int):
        self.index = index
        self.prev = None

    def __enter__(self):
        cur = torch._C._cuda_getDevice()
        if cur != self.index:
            self.prev = cur
            torch._C._cuda_setDevice(self.index)

    def __exit__(self, *exc):
        if self.prev is not None:
            torch._C._cuda_setDevice(self.prev)
        return False


def _mode(mode, deterministic=False) -> int:
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    return m | DETERMINISTIC if deterministic else m


def _seq(name, t, like=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, T, H, Dh], got {tuple(t.shape)}")
    if t.dtype not in DTYPES:
        raise TypeError(f"{name}: dtype {t.dtype} not supported")
    if like is not None and (t.shape != like.shape or t.dtype != like.dtype or t.device != like.device):
        raise ValueError(f"{name} must match shape/dtype/device of the gate logits")
    return t.contiguous()


def _state(name, t, B, H, Dh, device):
    if t is None:
        return None
    if t.dtype != torch.float32 or tuple(t.shape) != (B, H, Dh) or t.device != device:
        raise ValueError(f"{name} must be fp32 [B, H, Dh] = {(B, H, Dh)} on {device}")
    return t.contiguous()


def _out(name, t, shape, dtype, device):
    """A caller-provided output is written in place, so it must already be what the library
    writes: contiguous, of the given shape, dtype and device (no copy is made)."""
    if (not isinstance(t, torch.Tensor) or tuple(t.shape) != tuple(shape) or t.dtype != dtype
            or t.device != device or not t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} "
                         f"on {device}")


def workspace_bytes(B, T, H, Dh, dtype) -> int:
    return int(load_library().esa_scan_workspace_bytes(B, T, H, Dh, DTYPES[dtype]))


def ckpt_bytes(B, T, H, Dh) -> int:
    return int(load_library().esa_scan_ckpt_bytes(B, T, H, Dh))


def get_workspace(nbytes: int, device) -> torch.Tensor:
    """A zero-initialised workspace of at least nbytes, cached per (device, stream).

    The library leaves a workspace ready for reuse after every call, so the cache only
    zero-fills on allocation.  One workspace per stream: calls on one stream are ordered.
    """
    if isinstance(device, int):
        index = device
    else:
        dev = torch.device(device)
        index = dev.index if dev.index is not None else torch.cuda.current_device()
    key = (index, _raw_stream(index))
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=torch.device("cuda", index))
        _workspaces[key] = ws
    return ws


_ws_need: dict = {}


def _workspace_for(a) -> torch.Tensor:
    """The cached workspace for a scan over the gate logits `a` ([B, T, H, Dh]); the size
    query runs once per shape and dtype."""
    if not isinstance(a, torch.Tensor) or not a.is_cuda:
        raise TypeError("gate_logit must be a CUDA (HIP) tensor")
    if a.dim() != 4:
        raise ValueError(f"gate_logit must be [B, T, H, Dh], got {tuple(a.shape)}")
    key = (a.shape, a.dtype)
    need = _ws_need.get(key)
    if need is None:
        if a.dtype not in DTYPES:
            raise TypeError(f"gate_logit: dtype {a.dtype} not supported")
        need = workspace_bytes(*a.shape, a.dtype)
        _ws_need[key] = need
    return get_workspace(need, a.get_device())


def scan_fwd(a, v, q, init_state=None, mode="controlled", return_ckpt=False, final_state=None,
             y=None, workspace=None, deterministic=False):
    """Forward scan with fused gate and readout (esa_scan_fwd).  deterministic=True makes the
    result bitwise reproducible (ESA_DETERMINISTIC).  Sequence inputs are made contiguous;
    caller-provided outputs (y, final_state) must already be contiguous and of the right
    shape, dtype and device."""
    ext = _ext if _ext is not None else _torch_ext()
    ws = workspace if workspace is not None else _workspace_for(a)
    st, y, final_state, ckpt = ext.scan_fwd(a, v, q, init_state, _mode(mode, deterministic),
                                            bool(return_ckpt), final_state, y, ws)
    if st:
        _check(st, "esa_scan_fwd")
    if return_ckpt:
        return y, final_state, ckpt
    return y, final_state


def scan_bwd(a, v, q, dy, init_state=None, d_final_state=None, ckpt=None, mode="controlled",
             workspace=None, deterministic=False, d_logit=None, d_value=None, d_query=None,
             d_init=None):
    """Backward of scan_fwd (esa_scan_bwd).  Returns (d_logit, d_value, d_query, d_init);
    any of the four may be passed in to be written in place."""
    ext = _ext if _ext is not None else _torch_ext()
    ws = workspace if workspace is not None else _workspace_for(a)
    st, da, dv, dq, d_init = ext.scan_bwd(a, v, q, dy, init_state, d_final_state, ckpt,
                                          _mode(mode, deterministic), ws, d_logit, d_value,
                                          d_query, d_init)
    if st:
        _check(st, "esa_scan_bwd")
    return da, dv, dq, d_init


def state_step(a, v, q, state, mode="controlled", y=None):
    """One-token update (esa_state_step): `state` (fp32 [B, H, Dh]) is updated in place.
    The tensors' shapes, dtypes, devices and layout are checked in the _esa_torch call path
    (ValueError on a mismatch)."""
    ext = _ext if _ext is not None else _torch_ext()
    for name, t in (("gate_logit", a), ("value", v), ("query", q), ("state", state)):
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a tensor")
    if y is None:
        y = torch.empty_like(a)
    elif not isinstance(y, torch.Tensor):
        raise ValueError("y must be a tensor")
    st = ext.state_step(state, a, v, q, y, _mode(mode))
    if st:
        _check(st, "esa_state_step")
    return y


def segment_fwd(a, v, mode="controlled", workspace=None, deterministic=False):
    """Aggregate of one sequence segment from a zero state (esa_scan_segment_fwd): returns
    (seg_state, seg_gate_prod), fp32 [B, H, Dh] each."""
    lib = load_library()
    a = _seq("gate_logit", a)
    v = _seq("value", v, a)
    B, T, H, Dh = a.shape
    seg_state = torch.empty((B, H, Dh), dtype=torch.float32, device=a.device)
    seg_prod = torch.empty_like(seg_state)
    need = workspace_bytes(B, T, H, Dh, a.dtype)
    ws = workspace if workspace is not None else get_workspace(need, a.device)
    if ws.device != a.device or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {a.device}")
    with _OnDevice(a.device.index):
        st = lib.esa_scan_segment_fwd(B, T, H, Dh, DTYPES[a.dtype], _mode(mode, deterministic),
                                      _ptr(a), _ptr(v),
                                      _ptr(seg_state), _ptr(seg_prod), _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream_handle(a.device))
    _check(st, "esa_scan_segment_fwd")
    return seg_state, seg_prod


def segment_bwd(a, v, q, dy, init_state=None, ckpt=None, mode="controlled", workspace=None,
                deterministic=False):
    """Gradient reaching a segment's initial state with none arriving at its end
    (esa_scan_segment_bwd): fp32 [B, H, Dh]."""
    lib = load_library()
    a = _seq("gate_logit", a)
    v = _seq("value", v, a)
    q = _seq("query", q, a)
    dy = _seq("dy", dy, a)
    B, T, H, Dh = a.shape
    init_state = _state("init_state", init_state, B, H, Dh, a.device)
    if ckpt is not None:
        if (ckpt.dtype != torch.float32 or ckpt.device != a.device
                or ckpt.numel() * 4 < ckpt_bytes(B, T, H, Dh)):
            raise ValueError("ckpt must be the fp32 checkpoint of scan_fwd(return_ckpt=True)")
        ckpt = ckpt.contiguous()
    seg_d_init = torch.empty((B, H, Dh), dtype=torch.float32, device=a.device)
    need = workspace_bytes(B, T, H, Dh, a.dtype)
    ws = workspace if workspace is not None else get_workspace(need, a.device)
    if ws.device != a.device or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {a.device}")
    with _OnDevice(a.device.index):
        st = lib.esa_scan_segment_bwd(B, T, H, Dh, DTYPES[a.dtype], _mode(mode, deterministic),
                                      _ptr(a), _ptr(v),
                                      _ptr(q), _ptr(init_state), _ptr(dy), _ptr(ckpt),
                                      _ptr(seg_d_init), _ptr(ws), ws.numel() * ws.element_size(),
                                      _stream_handle(a.device))
    _check(st, "esa_scan_segment_bwd")
    return seg_d_init


def segment_compose(seg_gate_prod, seg_agg, boundary=None, reverse=False):
    """Compose segment aggregates (esa_segment_compose).  seg_gate_prod, seg_agg: fp32
    [nseg, B, H, Dh]; boundary: fp32 [B, H, Dh] or None.  Returns (carry [nseg, B, H, Dh],
    total [B, H, Dh])."""
    lib = load_library()
    for name, t in (("seg_gate_prod", seg_gate_prod), ("seg_agg", seg_agg)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.float32:
            raise ValueError(f"{name} must be an fp32 CUDA (HIP) tensor")
    if seg_agg.shape != seg_gate_prod.shape or seg_agg.device != seg_gate_prod.device:
        raise ValueError("seg_gate_prod and seg_agg must share shape and device")
    p = seg_gate_prod.contiguous()
    x = seg_agg.contiguous()
    nseg = p.shape[0]
    lanes = p[0].numel()
    if boundary is not None:
        _out("boundary", boundary, p.shape[1:], torch.float32, p.device)
    carry = torch.empty_like(p)
    total = torch.empty(p.shape[1:], dtype=torch.float32, device=p.device)
    with _OnDevice(p.device.index):
        st = lib.esa_segment_compose(nseg, lanes, 1 if reverse else 0, _ptr(p), _ptr(x),
                                     _ptr(boundary), _ptr(carry), _ptr(total),
                                     _stream_handle(p.device))
    _check(st, "esa_segment_compose")
    return carry, total


class StepPlan:
    """The fixed arguments of a decode loop, validated once: the fp32 state [B, H, Dh] (updated
    in place by every step), the storage dtype and the mode.  Each call checks the step's
    tensors and launches esa_state_step on the current stream through the _esa_torch call
    path, which keeps the host's share of an eager step small (about 3.3 us a step, against
    5.3 us through ctypes with the checks in Python).

        plan = StepPlan(state, torch.float16, "controlled")
        for t in ...:
            plan(a_t, v_t, q_t, y_t)      # [B, H, Dh] each, y_t written
    """

    def __init__(self, state, dtype, mode="controlled"):
        if (not isinstance(state, torch.Tensor) or not state.is_cuda or state.dim() != 3
                or state.dtype != torch.float32 or not state.is_contiguous()):
            raise ValueError("state must be a contiguous fp32 [B, H, Dh] CUDA (HIP) tensor")
        if dtype not in DTYPES:
            raise TypeError(f"dtype {dtype} not supported")
        self._step = _torch_ext().state_step
        self.state = state
        self.shape = state.shape
        self.dtype = dtype
        self.device = state.device
        self._mode = _mode(mode)

    def __call__(self, a, v, q, y):
        # the call path checks that every tensor matches the state's shape and device, one
        # dtype and a contiguous layout; the plan adds only its own dtype
        if a.dtype is not self.dtype:
            raise ValueError(f"step tensors must be {self.dtype}, got {a.dtype}")
        st = self._step(self.state, a, v, q, y, self._mode)
        if st:
            _check(st, "esa_state_step")
        return y
