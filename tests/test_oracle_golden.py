"""The oracle reproduces its stored regression values (tests/golden/oracle_small.json,
written by tests/golden/make_oracle_golden.py, which calls only the oracle)."""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "oracle_small.json")


@pytest.mark.parametrize("mode", [0, 1])
def test_oracle_regression(mode):
    g = json.load(open(GOLD))
    x = {k: np.array(v) for k, v in g["inputs"].items()}
    case = g["cases"][mode]
    assert case["mode"] == mode
    y, eT = oracle.scan_fwd(x["a"], x["v"], x["q"], x["e0"], mode=mode)
    da, dv, dq, de0 = oracle.scan_bwd(x["a"], x["v"], x["q"], x["dy"], x["e0"], x["dET"],
                                      mode=mode)
    ys, st = oracle.state_step(x["a"][:, 0], x["v"][:, 0], x["q"][:, 0], x["e0"], mode=mode)
    got = {"y": y, "eT": eT, "da": da, "dv": dv, "dq": dq, "de0": de0, "step_y": ys,
           "step_state": st}
    for k, val in got.items():
        np.testing.assert_allclose(val, np.array(case[k]), rtol=1e-14, atol=1e-15, err_msg=k)
