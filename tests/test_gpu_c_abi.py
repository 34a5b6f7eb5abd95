"""libesa.so driven from plain C (tests/c_abi_gpu.c): hipMalloc'd buffers, a HIP stream,
esa_workspace_init, esa_scan_fwd, esa_scan_bwd and esa_state_step, checked inside the program
against the oracle's C entry points at the fp32 bar.  The program is built by
__graft_entry__.build() and runs here as a child process."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_bin", "c_abi_gpu")


def test_c_program_matches_the_oracle():
    assert os.path.exists(EXE), f"{EXE} is missing: run __graft_entry__.build() first"
    print("c_abi_gpu", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    sys.stdout.write(r.stdout)
    sys.stderr.write(r.stderr)
    assert r.returncode == 0, f"c_abi_gpu exited with {r.returncode}"
    assert "PASS" in r.stdout
