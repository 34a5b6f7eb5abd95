"""Python binding of libesa.so (include/esa.h), with torch for device memory and streams.

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

Every call goes through _esa_torch, a small C++ binding of the same C ABI built beside
libesa.so that takes torch tensors directly and checks them there (a few microseconds of
host time a call, against 5-17 us through ctypes with the checks in Python); ctypes loads
libesa.so for the size queries and the status strings.

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
ESA_ERR_TIMEOUT = 6
STATUS_NAMES = {0: "ESA_OK", 1: "ESA_ERR_INVALID_ARG", 2: "ESA_ERR_UNSUPPORTED",
                3: "ESA_ERR_WORKSPACE", 4: "ESA_ERR_HIP", 5: "ESA_ERR_SCRATCH_LIMIT",
                6: "ESA_ERR_TIMEOUT"}
DTYPES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2, torch.float8_e4m3fn: 3,
          torch.float8_e5m2: 4}
MODES = {"direct": 0, "controlled": 1}
DETERMINISTIC = 0x100  # ESA_DETERMINISTIC: OR-ed into the mode, bitwise reproducible scans
TEST_FORCE_TIMEOUT = 0x200  # ESA_TEST_FORCE_TIMEOUT: a look-back timeout forced for tests
LOOKBACK_STATS = 0x400  # ESA_LOOKBACK_STATS: the kernel instance that counts look-back walks

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
    "esa_workspace_status": (_C, [_P, ctypes.POINTER(ctypes.c_uint32), _P]),
    "esa_scan_fwd": (_C, [_I, _I, _I, _I, _C, _C, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "esa_scan_fwd_noalloc": (_C, [_I, _I, _I, _I, _C, _C, _P, _P, _P, _P, _P, _P, _P, _P]),
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
# Workspaces replaced by larger ones.  A HIP graph that recorded a scan keeps the raw address
# of the workspace it ran on and uses it on every replay, so a workspace is never freed once
# it has served a call: a superseded one stays alive here for the life of the process.
_retired: list = []
_check_each_call = os.environ.get("ESA_CHECK_TIMEOUTS", "") not in ("", "0")


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


def _raw_stream(index: int) -> int:
    """The current HIP stream of device `index` as an integer handle (torch's raw accessor,
    without building a Python stream object)."""
    return torch._C._cuda_getCurrentRawStream(index)


def _mode(mode, deterministic=False) -> int:
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    return m | DETERMINISTIC if deterministic else m


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
        if ws is not None:
            _retired.append(ws)  # a captured graph may still use it (see _retired)
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=torch.device("cuda", index))
        _workspaces[key] = ws
    return ws


STAT_NAMES = ("took_published", "walked", "tiles_folded", "longest_walk", "polls")


def workspace_status(workspace=None, stream=None) -> dict:
    """What a workspace's header records (esa_workspace_status; waits for the stream): the
    tag of the last scan launch whose cross-tile wait timed out (0: none since the workspace
    was initialised) and the look-back counters of ESA_LOOKBACK_STATS launches.  `workspace`
    is a workspace tensor, or None for the current device's no-allocation scratch."""
    lib = load_library()
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda:
            raise ValueError("workspace must be a CUDA (HIP) tensor")
        index = workspace.device.index
        ptr = workspace.data_ptr()
    else:
        index = torch.cuda.current_device()
        ptr = None
    if stream is None:
        stream = _raw_stream(index)
    info = (ctypes.c_uint32 * 6)()
    st = lib.esa_workspace_status(ptr, info, stream)
    if st not in (ESA_OK, ESA_ERR_TIMEOUT):
        _check(st, "esa_workspace_status")
    out = {"timeout_tag": int(info[0])}
    out.update({n: int(info[1 + k]) for k, n in enumerate(STAT_NAMES)})
    return out


def _raise_if_timed_out(ws: torch.Tensor, where: str):
    """Reads the workspace's timeout record (waiting for its stream); if a launch timed out,
    clears the record, so that each timeout is reported once, and raises EsaError."""
    if workspace_status(ws)["timeout_tag"]:
        ws[12:16].zero_()
        raise EsaError(ESA_ERR_TIMEOUT, where)


def check_timeouts():
    """Waits for the binding's workspaces' streams and raises EsaError (ESA_ERR_TIMEOUT) if a
    scan launched on one of them had a cross-tile wait time out since the last check; its
    outputs that depended on the missing value are NaN.  Never happens in a correct run."""
    for (index, stream), ws in list(_workspaces.items()):
        with torch.cuda.device(index):
            if workspace_status(ws, stream)["timeout_tag"]:
                ws[12:16].zero_()
                raise EsaError(ESA_ERR_TIMEOUT, f"scan on device {index}")


def set_timeout_checks(on: bool = True):
    """Debug mode (also set by the environment variable ESA_CHECK_TIMEOUTS=1): after every
    scan call, wait for it and raise EsaError if its cross-tile wait timed out.  Each check
    synchronises the stream."""
    global _check_each_call
    _check_each_call = bool(on)


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
    if _check_each_call:
        _raise_if_timed_out(ws, "esa_scan_fwd")
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
    if _check_each_call:
        _raise_if_timed_out(ws, "esa_scan_bwd")
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
    ext = _ext if _ext is not None else _torch_ext()
    ws = workspace if workspace is not None else _workspace_for(a)
    st, seg_state, seg_prod = ext.segment_fwd(a, v, _mode(mode, deterministic), ws)
    if st:
        _check(st, "esa_scan_segment_fwd")
    if _check_each_call:
        _raise_if_timed_out(ws, "esa_scan_segment_fwd")
    return seg_state, seg_prod


def segment_bwd(a, v, q, dy, init_state=None, ckpt=None, mode="controlled", workspace=None,
                deterministic=False):
    """Gradient reaching a segment's initial state with none arriving at its end
    (esa_scan_segment_bwd): fp32 [B, H, Dh]."""
    ext = _ext if _ext is not None else _torch_ext()
    ws = workspace if workspace is not None else _workspace_for(a)
    st, seg_d_init = ext.segment_bwd(a, v, q, dy, init_state, ckpt, _mode(mode, deterministic),
                                     ws)
    if st:
        _check(st, "esa_scan_segment_bwd")
    if _check_each_call:
        _raise_if_timed_out(ws, "esa_scan_segment_bwd")
    return seg_d_init


def segment_compose(seg_gate_prod, seg_agg, boundary=None, reverse=False):
    """Compose segment aggregates (esa_segment_compose).  seg_gate_prod, seg_agg: fp32
    [nseg, B, H, Dh]; boundary: fp32 [B, H, Dh] or None.  Returns (carry [nseg, B, H, Dh],
    total [B, H, Dh])."""
    ext = _ext if _ext is not None else _torch_ext()
    for name, t in (("seg_gate_prod", seg_gate_prod), ("seg_agg", seg_agg)):
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be an fp32 CUDA (HIP) tensor")
    st, carry, total = ext.segment_compose(seg_gate_prod, seg_agg, boundary, bool(reverse))
    if st:
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


class DecodeGraph:
    """A chain of `steps` one-token updates (esa_state_step) recorded once into a HIP graph and
    replayed with no host work per step: generation's decode loop without the per-launch
    cost (page "Entangled State Attention v2.1", sections 5 and 6: the step-wise decode
    interface and compiled generation).

    A graph replays fixed addresses, so the object owns every buffer its steps read and write:

        state      fp32 [B, H, Dh]            the recurrent state, updated in place by each step
        a, v, q    dtype [steps, B, H, Dh]    the steps' gate logits, values and queries
        y          dtype [steps, B, H, Dh]    each step's readout
        snapshots  fp32 [len(snapshot_steps), B, H, Dh]  the state after each listed step
                   (1-based: 1 is the state after the first step)

    Write the inputs and the starting state, then replay():

        dg = DecodeGraph(B, H, Dh, steps=1, dtype=torch.float16)   # one token per replay
        dg.state.copy_(prefill_state)
        for t in ...:
            dg.a[0].copy_(a_t); dg.v[0].copy_(v_t); dg.q[0].copy_(q_t)
            dg.replay()                                            # y_t in dg.y[0]

    With steps = n > 1 one replay runs n steps whose inputs are all known beforehand (teacher
    forcing, or timing).  Replays run on the current stream; a replay must not overlap another
    replay of the same object or eager use of its buffers.
    """

    def __init__(self, B, H, Dh, steps, dtype=torch.float16, mode="controlled", device=None,
                 snapshot_steps=()):
        if dtype not in DTYPES:
            raise TypeError(f"dtype {dtype} not supported")
        if steps < 1:
            raise ValueError("steps must be at least 1")
        snaps = tuple(int(k) for k in snapshot_steps)
        if any(k < 1 or k > steps for k in snaps):
            raise ValueError(f"snapshot steps must lie in 1..{steps}")
        dev = torch.device("cuda", torch.cuda.current_device()) if device is None else \
            torch.device(device)
        ext = _torch_ext()
        self.steps, self.dtype, self.mode = steps, dtype, _mode(mode)
        self.state = torch.zeros((B, H, Dh), dtype=torch.float32, device=dev)
        shp = (steps, B, H, Dh)
        self.a = torch.zeros(shp, dtype=dtype, device=dev)
        self.v = torch.zeros(shp, dtype=dtype, device=dev)
        self.q = torch.zeros(shp, dtype=dtype, device=dev)
        self.y = torch.empty(shp, dtype=dtype, device=dev)
        self.snapshots = torch.empty((len(snaps), B, H, Dh), dtype=torch.float32, device=dev)
        after = {}
        for i, k in enumerate(snaps):
            after.setdefault(k - 1, []).append(i)
        # one eager step on a copy of the state, on the capture stream, before recording
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            st = ext.state_step(self.state.clone(), self.a[0], self.v[0], self.q[0], self.y[0],
                                self.mode)
            if st:
                _check(st, "esa_state_step")
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize(dev)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph, stream=side):
            for k in range(steps):
                st = ext.state_step(self.state, self.a[k], self.v[k], self.q[k], self.y[k],
                                    self.mode)
                if st:
                    _check(st, "esa_state_step")
                for i in after.get(k, ()):
                    self.snapshots[i].copy_(self.state)
        torch.cuda.synchronize(dev)

    def replay(self):
        """Runs the recorded steps on the current stream."""
        self.graph.replay()
