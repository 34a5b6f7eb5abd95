"""Builds libesa.so in-tree with hipcc for gfx950 (cross-compiles; no GPU needed).

    python -m gated_linear_recurrence_chunked_amd.build [--jobs N]

Each kernel translation unit compiles in its own hipcc process, then one link step makes
``gated_linear_recurrence_chunked_amd/libesa.so``.  Beside it, g++ builds ``_esa_torch``, the
decode step's torch-tensor call path into the library (argument marshalling only; torch's
headers, no hipify).  Objects go to ``_build/``.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libesa.so")
SOURCES = ["esa_api.hip", "esa_fwd.hip", "esa_bwd.hip", "esa_step.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
TORCH_EXT = "esa_torch.cpp"  # the torch-tensor call path of the scans and the step
TORCH_MOD = "_esa_torch"

# -packed-fp32-ops: never emit packed fp32 arithmetic (v_pk_*_f32); plain fp32 ops only.
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + CFLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def _torch_paths():
    import sysconfig

    import torch

    tdir = os.path.dirname(torch.__file__)
    inc = [os.path.join(tdir, "include"), os.path.join(tdir, "include", "torch", "csrc", "api",
                                                       "include"),
           sysconfig.get_paths()["include"]]
    return inc, os.path.join(tdir, "lib"), sysconfig.get_config_var("EXT_SUFFIX"), int(
        torch._C._GLIBCXX_USE_CXX11_ABI)


def _compile_torch_ext() -> str:
    inc, _, _, abi = _torch_paths()
    obj = os.path.join(BUILD, "esa_torch.o")
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__",
           f"-DTORCH_EXTENSION_NAME={TORCH_MOD}", f"-D_GLIBCXX_USE_CXX11_ABI={abi}",
           "-I", INCLUDE, "-I", os.path.join(ROCM, "include")]
    for d in inc:
        cmd += ["-I", d]
    cmd += ["-c", os.path.join(CSRC, TORCH_EXT), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"g++ failed on {TORCH_EXT}")
    return obj


def _link_torch_ext(obj: str) -> str:
    _, tlib, suffix, _ = _torch_paths()
    out = os.path.join(PKG, TORCH_MOD + suffix)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["g++", "-shared", "-fPIC", "-o", tmp, obj, "-L", PKG, "-lesa", "-L", tlib, "-lc10",
           "-lc10_hip", "-ltorch", "-ltorch_cpu", "-ltorch_hip", "-ltorch_python",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN", "-Wl,-rpath," + tlib, "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"linking {TORCH_MOD} failed")
    os.replace(tmp, out)
    return out


def build(jobs: int | None = None, verbose: bool = True) -> str:
    """Compile every kernel source for gfx950 and link libesa.so, then the torch-tensor
    binding of the decode step (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES) + 1, os.cpu_count() or 1)
    with ThreadPoolExecutor(jobs) as ex:
        ext_obj = ex.submit(_compile_torch_ext)
        objs = list(ex.map(_compile, SOURCES))
        ext_obj = ext_obj.result()
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc link failed")
    os.replace(tmp, LIB)
    ext = _link_torch_ext(ext_obj)
    if verbose:
        print(f"built {LIB}")
        print(f"built {ext}")
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    args = ap.parse_args()
    build(args.jobs)


if __name__ == "__main__":
    main()
