"""The C-ABI library on the host: it loads, exports every function include/esa.h declares,
and rejects bad arguments with the documented status codes before any HIP call.

No test here launches a kernel: every call below fails validation, which returns before
the first HIP runtime call.  Pointers are never dereferenced on the host, so the fake but
aligned addresses used here are safe.
"""
import ctypes
import os
import re

import pytest

from gated_linear_recurrence_chunked_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "esa.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, SCRATCH_LIMIT = 0, 1, 2, 3, 5


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(esa_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.library_path()):
        pytest.skip("libesa.so not built")
    return binding.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"esa_scan_fwd", "esa_scan_bwd", "esa_state_step"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
        assert n in binding.SIGNATURES, n


def header_abi_version() -> int:
    import re
    text = open(os.path.join(ROOT, "include", "esa.h")).read()
    return int(re.search(r"#define ESA_ABI_VERSION (\d+)", text).group(1))


def test_version_and_status_strings(lib):
    assert lib.esa_abi_version() == header_abi_version() == 5
    names = ["ESA_OK", "ESA_ERR_INVALID_ARG", "ESA_ERR_UNSUPPORTED", "ESA_ERR_WORKSPACE",
             "ESA_ERR_HIP", "ESA_ERR_SCRATCH_LIMIT", "ESA_ERR_TIMEOUT"]
    for s, name in enumerate(names):
        assert lib.esa_status_string(s).decode().startswith(name)
        assert binding.STATUS_NAMES[s] == name
    assert lib.esa_status_string(99)


def test_workspace_and_ckpt_sizes(lib):
    ws = lib.esa_scan_workspace_bytes
    assert ws(1, 256, 2, 16, 0) > 256
    assert ws(64, 65536, 8, 64, 1) > ws(16, 8192, 8, 64, 1)
    assert ws(1, 0, 2, 16, 0) >= 256
    assert ws(1, 10, 2, 48, 1) == 0  # unsupported Dh
    assert ws(0, 10, 2, 16, 1) == 0
    assert ws(1, 10, 2, 16, 7) == 0
    assert ws(1, 10, 2, 16, 5) == 0
    # fp8 storage (3 = E4M3, 4 = E5M2): 128-channel blocks, shorter tiles, so more
    # look-back words than 16-bit storage at the same shape
    assert ws(1, 256, 2, 16, 3) > 256 and ws(1, 256, 2, 16, 4) == ws(1, 256, 2, 16, 3)
    assert ws(64, 65536, 8, 64, 3) > ws(64, 65536, 8, 64, 1)
    ck = lib.esa_scan_ckpt_bytes
    assert ck(2, 64, 3, 16) == 2 * 1 * 3 * 16 * 4
    assert ck(2, 65, 3, 16) == 2 * 2 * 3 * 16 * 4
    assert ck(2, 0, 3, 16) == 0


# fake, 16-byte aligned, non-overlapping device addresses (never dereferenced)
def addr(k):
    return ctypes.c_void_p(0x100000000 + k * 0x10000000)


def fwd(lib, B=2, T=100, H=2, Dh=16, dt=1, mode=1, a=1, v=2, q=3, e0=None, y=4, eT=5, ck=None,
        ws=6, wsb=None):
    def p(k):
        if k is None:
            return None
        return k if isinstance(k, ctypes.c_void_p) else addr(k)

    if wsb is None:
        wsb = 0
    return lib.esa_scan_fwd(B, T, H, Dh, dt, mode, p(a), p(v), p(q), p(e0), p(y), p(eT), p(ck),
                            p(ws), wsb, None)


def test_fwd_validation(lib):
    assert fwd(lib, a=None) == INVALID
    # T = 0 needs no sequence pointers; with no final state nothing is launched
    assert fwd(lib, a=None, v=None, q=None, y=None, eT=None, T=0, ws=None) == OK
    assert fwd(lib, y=None) == INVALID
    assert fwd(lib, B=0) == INVALID
    assert fwd(lib, T=-1) == INVALID
    assert fwd(lib, dt=5) == INVALID
    assert fwd(lib, mode=0x102) == INVALID  # deterministic flag with a bad form
    assert fwd(lib, mode=0x800) == INVALID  # unknown flag
    assert fwd(lib, mode=0x202) == INVALID  # test flag with a bad form
    assert fwd(lib, Dh=64, mode=0x301, y=1) == INVALID  # both flags: the rest still validates
    assert fwd(lib, mode=0x101, y=1) == INVALID  # a valid flagged mode still validates the rest
    assert fwd(lib, dt=-1) == INVALID
    assert fwd(lib, mode=2) == INVALID
    assert fwd(lib, Dh=48) == UNSUPPORTED
    assert fwd(lib, Dh=256) == UNSUPPORTED
    assert fwd(lib, B=1 << 40, T=1 << 40) == INVALID  # element count overflows int64
    mis = ctypes.c_void_p(0x100000000 + 8)
    assert fwd(lib, v=mis) == INVALID
    assert fwd(lib, ws=None) == WORKSPACE
    assert fwd(lib, wsb=100) == WORKSPACE
    # y overlapping an input
    assert fwd(lib, y=1) == INVALID
    # final state overlapping the workspace
    assert fwd(lib, eT=6, wsb=1000) == INVALID


def test_bwd_validation(lib):
    def bwd(**kw):
        args = dict(B=2, T=100, H=2, Dh=64, dt=2, mode=0)
        args.update({k: kw.pop(k) for k in list(kw) if k in args})
        ptr = dict(a=1, v=2, q=3, e0=None, dy=4, dET=None, ck=None, da=5, dv=6, dq=7, de0=None,
                   ws=8)
        ptr.update(kw)
        p = {k: (None if x is None else addr(x)) for k, x in ptr.items()}
        return lib.esa_scan_bwd(args["B"], args["T"], args["H"], args["Dh"], args["dt"],
                                args["mode"], p["a"], p["v"], p["q"], p["e0"], p["dy"], p["dET"],
                                p["ck"], p["da"], p["dv"], p["dq"], p["de0"], p["ws"], 0, None)

    assert bwd(dy=None) == INVALID
    assert bwd(dq=None) == INVALID
    assert bwd(Dh=8) == UNSUPPORTED
    assert bwd(ws=None) == WORKSPACE
    assert bwd(da=4) == INVALID  # gradient output overlaps dy
    assert bwd(dv=5) == INVALID  # two outputs overlap


def test_step_validation(lib):
    def step(B=4, H=2, Dh=64, dt=1, mode=1, a=1, v=2, q=3, st=4, y=5):
        p = [None if x is None else addr(x) for x in (a, v, q, st, y)]
        return lib.esa_state_step(B, H, Dh, dt, mode, *p, None)

    assert step(st=None) == INVALID
    assert step(y=None) == INVALID
    assert step(Dh=24) == UNSUPPORTED
    assert step(y=2) == INVALID
    assert step(st=1) == INVALID
    assert step(mode=-1) == INVALID


def test_workspace_init_validation(lib):
    assert lib.esa_workspace_init(None, 256, None) == INVALID
    assert lib.esa_workspace_init(ctypes.c_void_p(0x100000008), 256, None) == INVALID


def test_segment_validation(lib):
    def seg_fwd(B=2, T=100, H=2, Dh=64, dt=1, mode=1, a=1, v=2, st=3, pr=4, ws=5, wsb=0):
        p = [None if x is None else (x if isinstance(x, ctypes.c_void_p) else addr(x))
             for x in (a, v, st, pr, ws)]
        return lib.esa_scan_segment_fwd(B, T, H, Dh, dt, mode, *p[:4], p[4], wsb, None)

    assert seg_fwd(st=None) == INVALID
    assert seg_fwd(pr=None) == INVALID
    assert seg_fwd(a=None) == INVALID
    assert seg_fwd(dt=5) == INVALID
    assert seg_fwd(Dh=48) == UNSUPPORTED
    assert seg_fwd(v=ctypes.c_void_p(0x100000000 + 8)) == INVALID
    assert seg_fwd(st=4) == INVALID  # the two outputs overlap
    assert seg_fwd(ws=None) == WORKSPACE

    def seg_bwd(B=2, T=100, H=2, Dh=64, dt=2, mode=0, a=1, v=2, q=3, e0=None, dy=4, ck=None,
                out=5, ws=6):
        p = [None if x is None else addr(x) for x in (a, v, q, e0, dy, ck, out, ws)]
        return lib.esa_scan_segment_bwd(B, T, H, Dh, dt, mode, *p[:7], p[7], 0, None)

    assert seg_bwd(out=None) == INVALID
    assert seg_bwd(dy=None) == INVALID
    assert seg_bwd(out=4) == INVALID  # output overlaps dy
    assert seg_bwd(ws=None) == WORKSPACE

    def compose(nseg=3, lanes=64, rev=0, p=1, x=2, bnd=None, carry=3, total=None):
        ptr = [None if k is None else (k if isinstance(k, ctypes.c_void_p) else addr(k))
               for k in (p, x, bnd, carry, total)]
        return lib.esa_segment_compose(nseg, lanes, rev, *ptr, None)

    assert compose(nseg=0) == INVALID
    assert compose(lanes=0) == INVALID
    assert compose(rev=2) == INVALID
    assert compose(p=None) == INVALID
    assert compose(carry=None) == INVALID
    assert compose(carry=1) == INVALID  # carry overlaps the products
    assert compose(total=3) == INVALID  # total overlaps carry
    assert compose(x=ctypes.c_void_p(0x100000000 + 0x20000000 + 2)) == INVALID  # misaligned
    assert compose(nseg=1 << 40, lanes=1 << 40) == INVALID  # size overflows


def test_public_names_resolve():
    """Every name the package exports resolves (the pages' test list includes the public
    imports); none needs a GPU to be looked up."""
    import gated_linear_recurrence_chunked_amd as pkg

    for name in pkg.__all__:
        assert getattr(pkg, name) is not None, name
    from gated_linear_recurrence_chunked_amd import ESALayer, esa_scan, scan_fwd, state_step  # noqa: F401


def test_force_timeout_flag_validation(lib):
    """ESA_TEST_FORCE_TIMEOUT (0x200) is accepted by esa_scan_fwd and esa_scan_bwd for fp16
    storage with Dh = 64 only, and rejected by the other calls; every check returns before
    any launch (a valid flagged call here stops at the zero-byte workspace)."""
    F = 0x200
    assert fwd(lib, dt=1, Dh=64, mode=1 | F) == WORKSPACE
    assert fwd(lib, dt=1, Dh=64, mode=0 | F | 0x100) == WORKSPACE
    assert fwd(lib, dt=0, Dh=64, mode=1 | F) == UNSUPPORTED
    assert fwd(lib, dt=2, Dh=64, mode=1 | F) == UNSUPPORTED
    assert fwd(lib, dt=1, Dh=32, mode=1 | F) == UNSUPPORTED
    p = [addr(k) for k in range(1, 6)]
    assert lib.esa_state_step(4, 2, 64, 1, 1 | F, *p, None) == INVALID
    assert lib.esa_scan_segment_fwd(2, 100, 2, 64, 1, 1 | F, addr(1), addr(2), addr(3), addr(4),
                                    addr(5), 0, None) == INVALID
    assert lib.esa_scan_segment_bwd(2, 100, 2, 64, 1, 1 | F, addr(1), addr(2), addr(3), None,
                                    addr(4), None, addr(5), addr(6), 0, None) == INVALID


def test_torch_call_path_loads():
    """The torch-tensor call path (_esa_torch, built beside libesa.so) imports without a GPU
    and exposes every call of the binding."""
    from gated_linear_recurrence_chunked_amd import _esa_torch

    for name in ("scan_fwd", "scan_bwd", "state_step", "segment_fwd", "segment_bwd",
                 "segment_compose"):
        assert callable(getattr(_esa_torch, name))


def test_stats_flag_validation(lib):
    """ESA_LOOKBACK_STATS (0x400) is accepted by esa_scan_fwd and esa_scan_bwd for fp16 and
    fp8 E4M3 storage with Dh = 64, alone; every check returns before any launch (a valid
    flagged call here stops at the zero-byte workspace)."""
    S = 0x400
    assert fwd(lib, dt=1, Dh=64, mode=1 | S) == WORKSPACE
    assert fwd(lib, dt=3, Dh=64, mode=0 | S) == WORKSPACE
    for dt in (0, 2, 4):
        assert fwd(lib, dt=dt, Dh=64, mode=1 | S) == UNSUPPORTED
    assert fwd(lib, dt=1, Dh=32, mode=1 | S) == UNSUPPORTED
    assert fwd(lib, dt=1, Dh=64, mode=1 | S | 0x100) == INVALID
    assert fwd(lib, dt=1, Dh=64, mode=1 | S | 0x200) == INVALID
    p = [addr(k) for k in range(1, 6)]
    assert lib.esa_state_step(4, 2, 64, 1, 1 | S, *p, None) == INVALID
    assert lib.esa_scan_segment_fwd(2, 100, 2, 64, 1, 1 | S, addr(1), addr(2), addr(3), addr(4),
                                    addr(5), 0, None) == INVALID


def test_workspace_status_validation(lib):
    info = (ctypes.c_uint32 * 6)()
    assert lib.esa_workspace_status(addr(1), None, None) == INVALID
    assert lib.esa_workspace_status(ctypes.c_void_p(0x100000008), info, None) == INVALID


def test_noalloc_validation(lib):
    """esa_scan_fwd_noalloc refuses, before any HIP call, a problem whose look-back words
    exceed its static array, the forced-timeout flag, and what esa_scan_fwd refuses."""
    def big(k):  # fake device addresses 8 GiB apart (the sequences here are 2 GiB)
        return ctypes.c_void_p(0x1000000000 + k * (1 << 33))

    def na(B=256, T=8192, H=8, Dh=64, dt=1, mode=1, a=1, y=4, eT=5):
        pa = None if a is None else big(a)
        py = None if y is None else big(y)
        pe = None if eT is None else big(eT)
        return lib.esa_scan_fwd_noalloc(B, T, H, Dh, dt, mode, pa, big(2), big(3), None, py,
                                        pe, None, None)

    assert na() == SCRATCH_LIMIT  # 64 MiB + 256 B of look-back words
    assert lib.esa_status_string(SCRATCH_LIMIT).decode().startswith("ESA_ERR_SCRATCH_LIMIT")
    assert na(T=100, mode=1 | 0x200) == INVALID
    assert na(a=None) == INVALID
    assert na(y=2) == INVALID
    assert na(Dh=48) == UNSUPPORTED
    assert na(T=0, a=None, y=None, eT=None) == OK  # nothing to launch
