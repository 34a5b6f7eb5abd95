"""Pins for the oracle's backward pass.

No page states the backward; it is the chain rule through the forward of page
"entangled-state-attention 0.1.0" ("Core idea").  It is pinned against central finite
differences of the (separately pinned) forward, against the adjoint identity
<w, J d> = <J^T w, d>, and against special cases of the reverse recurrence
(A = 1: the upstream state gradient passes through unchanged; A = 0: nothing passes).
"""
import numpy as np
import pytest

import oracle


def loss_and_grads(a, v, q, e0, dy, dET, mode):
    """L = <dy, y> + <dET, E_T>; its gradients are what scan_bwd returns."""
    y, eT = oracle.scan_fwd(a, v, q, e0, mode=mode)
    L = float(np.sum(dy * y) + np.sum(dET * eT))
    return L


def inputs(seed, B=2, T=7, H=2, Dh=4, a_mean=0.5):
    rng = np.random.default_rng(seed)
    shp = (B, T, H, Dh)
    a = rng.normal(a_mean, 1.5, size=shp)
    v = rng.normal(size=shp)
    q = rng.normal(size=shp)
    e0 = rng.normal(size=(B, H, Dh))
    dy = rng.normal(size=shp)
    dET = rng.normal(size=(B, H, Dh))
    return a, v, q, e0, dy, dET


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("which", ["a", "v", "q", "e0"])
def test_finite_differences(mode, which):
    a, v, q, e0, dy, dET = inputs(10 + mode)
    da, dv, dq, de0 = oracle.scan_bwd(a, v, q, dy, e0, dET, mode=mode)
    args = {"a": a, "v": v, "q": q, "e0": e0}
    grad = {"a": da, "v": dv, "q": dq, "e0": de0}[which]
    x = args[which]
    h = 1e-6
    num = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        old = x[idx]
        x[idx] = old + h
        lp = loss_and_grads(a, v, q, e0, dy, dET, mode)
        x[idx] = old - h
        lm = loss_and_grads(a, v, q, e0, dy, dET, mode)
        x[idx] = old
        num[idx] = (lp - lm) / (2 * h)
    scale = max(1.0, float(np.max(np.abs(num))))
    np.testing.assert_allclose(grad, num, rtol=1e-6, atol=2e-7 * scale)


@pytest.mark.parametrize("mode", [0, 1])
def test_adjoint_identity(mode):
    """<dy, J delta> + <dET, J_E delta> = <grad, delta> for a random joint direction delta,
    with J delta measured by a central difference along delta."""
    a, v, q, e0, dy, dET = inputs(40 + mode, B=3, T=33, H=2, Dh=8)
    da, dv, dq, de0 = oracle.scan_bwd(a, v, q, dy, e0, dET, mode=mode)
    rng = np.random.default_rng(99)
    d = [rng.normal(size=x.shape) for x in (a, v, q, e0)]
    h = 1e-5

    def L(s):
        return loss_and_grads(a + s * d[0], v + s * d[1], q + s * d[2], e0 + s * d[3], dy, dET,
                              mode)

    lhs = (L(h) - L(-h)) / (2 * h)
    rhs = sum(float(np.sum(g * dd)) for g, dd in zip((da, dv, dq, de0), d))
    assert lhs == pytest.approx(rhs, rel=1e-7)


def test_retain_all_passes_state_gradient_through():
    """A = 1 (a = +1000) and dy = 0: every dE_t equals dE_T, so dv_t = dE_T (direct) and the
    initial-state gradient is dE_T as well; the gate gradient vanishes (s (1 - s) = 0)."""
    a, v, q, e0, dy, dET = inputs(5, T=50)
    a[:] = 1000.0
    dy[:] = 0.0
    da, dv, dq, de0 = oracle.scan_bwd(a, v, q, dy, e0, dET, mode=0)
    np.testing.assert_array_equal(dv, np.broadcast_to(dET[:, None], dv.shape))
    np.testing.assert_array_equal(de0, dET)
    np.testing.assert_array_equal(da, np.zeros_like(da))
    np.testing.assert_array_equal(dq, np.zeros_like(dq))


def test_retain_all_reverse_cumsum():
    """A = 1, direct: dv_t = sum_{s >= t} gE_s + dE_T, a reverse prefix sum of the readout
    gradients; gE_s is read off the T = 1 problems, each of which is a single readout."""
    a, v, q, e0, dy, dET = inputs(6, B=1, T=20)
    a[:] = 1000.0
    _, dv, _, de0 = oracle.scan_bwd(a, v, q, dy, e0, dET, mode=0)
    _, _, E = oracle.scan_fwd(a, v, q, e0, mode=0, states=True)
    # readout gradient at each t alone: a T=1 problem starting from E_{t-1} with A = 1
    gE = np.zeros_like(dv)
    for t in range(a.shape[1]):
        start = e0 if t == 0 else E[:, t - 1]
        _, g, _, _ = oracle.scan_bwd(a[:, t : t + 1], v[:, t : t + 1], q[:, t : t + 1],
                                     dy[:, t : t + 1], start, None, mode=0)
        gE[:, t] = g[:, 0]
    rev = np.flip(np.cumsum(np.flip(gE, axis=1), axis=1), axis=1) + dET[:, None]
    np.testing.assert_allclose(dv, rev, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(de0, rev[:, 0], rtol=1e-12, atol=1e-13)


def test_forget_all_blocks_state_gradient():
    """A = 0 (a = -1000), direct: dE_t = gE_t only, the initial state gets no gradient."""
    a, v, q, e0, dy, dET = inputs(7)
    a[:] = -1000.0
    da, dv, dq, de0 = oracle.scan_bwd(a, v, q, dy, e0, dET, mode=0)
    np.testing.assert_array_equal(de0, np.zeros_like(de0))
    # each step is then an independent readout of E_t = v_t
    for t in range(a.shape[1]):
        _, g, _, _ = oracle.scan_bwd(a[:, t : t + 1], v[:, t : t + 1], q[:, t : t + 1],
                                     dy[:, t : t + 1], None, dET if t == a.shape[1] - 1 else None,
                                     mode=0)
        np.testing.assert_allclose(dv[:, t], g[:, 0], rtol=1e-13, atol=1e-14)


def test_zero_upstream_gives_zero_gradients():
    a, v, q, e0, dy, dET = inputs(8)
    z = oracle.scan_bwd(a, v, q, np.zeros_like(dy), e0, None, mode=1)
    for g in z:
        np.testing.assert_array_equal(g, np.zeros_like(g))
