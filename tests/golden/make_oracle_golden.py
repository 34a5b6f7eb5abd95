"""Writes oracle_small.json: a small seeded problem and the oracle's outputs for it.

Calls only the oracle.  The stored file guards against unintended changes to the oracle's
arithmetic; any intended change must regenerate it in the same commit and say why.
Run:  python tests/golden/make_oracle_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402


def main():
    rng = np.random.default_rng(20261203)
    B, T, H, Dh = 1, 6, 2, 4
    shp = (B, T, H, Dh)
    a = rng.normal(0.5, 1.5, size=shp)
    v = rng.normal(size=shp)
    q = rng.normal(size=shp)
    dy = rng.normal(size=shp)
    e0 = rng.normal(size=(B, H, Dh))
    dET = rng.normal(size=(B, H, Dh))
    cases = []
    for mode in (0, 1):
        y, eT = oracle.scan_fwd(a, v, q, e0, mode=mode)
        da, dv, dq, de0 = oracle.scan_bwd(a, v, q, dy, e0, dET, mode=mode)
        ys, st = oracle.state_step(a[:, 0], v[:, 0], q[:, 0], e0, mode=mode)
        cases.append({"mode": mode, "y": y.tolist(), "eT": eT.tolist(), "da": da.tolist(),
                      "dv": dv.tolist(), "dq": dq.tolist(), "de0": de0.tolist(),
                      "step_y": ys.tolist(), "step_state": st.tolist()})
    out = {
        "_about": "Oracle regression values, written by make_oracle_golden.py (oracle only).",
        "shape": list(shp),
        "inputs": {"a": a.tolist(), "v": v.tolist(), "q": q.tolist(), "dy": dy.tolist(),
                   "e0": e0.tolist(), "dET": dET.tolist()},
        "cases": cases,
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
