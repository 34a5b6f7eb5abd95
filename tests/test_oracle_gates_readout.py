"""Pins for the oracle's gates and readout, and for the forward scan they compose into.

Gates and readout follow page "entangled-state-attention 0.1.0", section "Core idea":
direct A = sigma(a), B = V; controlled g = sigma(a), B = (1 - g) V; readout q * Norm(E)
with Norm read as per-head RMSNorm (eps 1e-6, no gain).  The pins are library routines
(scipy's logistic function, torch's rms_norm), the textbook RMSNorm invariants, special
cases of the gates (saturated logits give A = 1 or A = 0 exactly) and the closed form of the
whole forward scan.
"""
import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle

EPS = 1e-6


def test_eps_is_the_fixed_reading():
    assert oracle.rmsnorm_eps() == EPS


@pytest.mark.parametrize("x", [0.0, 1e-3, -1e-3, 0.5, -0.5, 2.0, -2.0, 17.0, -17.0, 36.0,
                               -36.0, 100.0, -100.0, 700.0, -700.0, 1000.0, -1000.0])
def test_sigmoid_matches_library(x):
    s = oracle.sigmoid(x)
    ref = expit(x)
    assert s == pytest.approx(ref, rel=2e-16 * 4, abs=0.0)
    # 1 - sigma(x) = sigma(-x), also far in the tail where 1 - s would cancel
    assert oracle.sigmoid(-x) == pytest.approx(expit(-x), rel=8e-16, abs=0.0)


def test_sigmoid_saturates_exactly():
    assert oracle.sigmoid(1000.0) == 1.0
    assert oracle.sigmoid(-1000.0) == 0.0
    assert oracle.sigmoid(0.0) == 0.5


@pytest.mark.parametrize("mode", [0, 1])
def test_gates_against_library(mode):
    rng = np.random.default_rng(3)
    a = rng.normal(0, 4, size=1000)
    v = rng.normal(size=1000)
    A, Bt = oracle.gates(a, v, mode)
    np.testing.assert_allclose(A, expit(a), rtol=1e-15)
    ref_B = v if mode == 0 else expit(-a) * v
    np.testing.assert_allclose(Bt, ref_B, rtol=1e-15, atol=0)


def test_readout_matches_library_rmsnorm():
    rng = np.random.default_rng(4)
    G, Dh = 37, 16
    E = rng.normal(0, 3, size=(G, Dh))
    q = rng.normal(size=(G, Dh))
    y = oracle.readout(E, q, Dh)
    n = torch.nn.functional.rms_norm(torch.from_numpy(E), (Dh,), eps=EPS).numpy()
    np.testing.assert_allclose(y, q * n, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("Dh", [1, 4, 64])
def test_readout_invariants(Dh):
    rng = np.random.default_rng(Dh)
    G = 50
    E = rng.normal(0, 1, size=(G, Dh)) * rng.uniform(1e-4, 10, size=(G, 1))
    ones = np.ones_like(E)
    n = oracle.readout(E, ones, Dh)
    m = np.mean(E * E, axis=1)
    # sum_d n_d^2 = Dh * m / (m + eps)
    np.testing.assert_allclose(np.sum(n * n, axis=1), Dh * m / (m + EPS), rtol=1e-13)
    # |n_d| <= sqrt(Dh)
    assert np.all(np.abs(n) <= np.sqrt(Dh) * (1 + 1e-15))
    if Dh == 1:
        np.testing.assert_allclose(n[:, 0], E[:, 0] / np.sqrt(E[:, 0] ** 2 + EPS), rtol=1e-14)


def test_readout_groups_are_heads():
    """Changing one head's state changes only that head's outputs (grouping axis is Dh)."""
    rng = np.random.default_rng(9)
    H, Dh = 4, 8
    E = rng.normal(size=(3, H * Dh))
    q = rng.normal(size=(3, H * Dh))
    y = oracle.readout(E, q, Dh)
    E2 = E.copy()
    E2[1, 2 * Dh + 3] += 5.0
    y2 = oracle.readout(E2, q, Dh)
    changed = np.argwhere(y2 != y)
    assert set(map(tuple, changed)) <= {(1, c) for c in range(2 * Dh, 3 * Dh)}
    assert len(changed) == Dh


def rand_inputs(B, T, H, Dh, seed, a_mean=0.0, a_std=1.5):
    rng = np.random.default_rng(seed)
    a = rng.normal(a_mean, a_std, size=(B, T, H, Dh))
    v = rng.normal(size=(B, T, H, Dh))
    q = rng.normal(size=(B, T, H, Dh))
    e0 = rng.normal(size=(B, H, Dh))
    return a, v, q, e0


@pytest.mark.parametrize("mode", [0, 1])
def test_scan_fwd_closed_form(mode):
    """The full forward against the closed form of the recurrence with library gates and
    library RMSNorm, on a tiny problem."""
    B, T, H, Dh = 2, 12, 2, 4
    a, v, q, e0 = rand_inputs(B, T, H, Dh, 21 + mode)
    y, eT = oracle.scan_fwd(a, v, q, e0, mode=mode)
    A = expit(a)
    Bt = v if mode == 0 else expit(-a) * v
    E = np.zeros_like(a)
    for b in range(B):
        for t in range(T):
            acc = np.prod(A[b, : t + 1], axis=0) * e0[b]
            for s in range(t + 1):
                acc = acc + np.prod(A[b, s + 1 : t + 1], axis=0) * Bt[b, s]
            E[b, t] = acc
    n = torch.nn.functional.rms_norm(torch.from_numpy(E), (Dh,), eps=EPS).numpy()
    np.testing.assert_allclose(y, q * n, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(eT, E[:, -1], rtol=1e-12, atol=1e-12)


def test_controlled_is_direct_with_gated_write():
    """Controlled mode equals direct mode fed B = sigma(-a) * v ("Core idea")."""
    a, v, q, e0 = rand_inputs(2, 40, 3, 8, 31)
    yc, ec = oracle.scan_fwd(a, v, q, e0, mode=1)
    yd, ed = oracle.scan_fwd(a, expit(-a) * v, q, e0, mode=0)
    np.testing.assert_allclose(yc, yd, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(ec, ed, rtol=1e-13, atol=1e-14)


def test_saturated_logits_reach_special_cases():
    """a = +1000 gives A = 1 (prefix sum); a = -1000 gives A = 0 (E = B) through the scan."""
    B, T, H, Dh = 1, 64, 1, 4
    rng = np.random.default_rng(2)
    v = rng.normal(size=(B, T, H, Dh))
    q = np.ones_like(v)
    _, _, E = oracle.scan_fwd(np.full_like(v, 1000.0), v, q, mode=0, states=True)
    np.testing.assert_array_equal(E, np.cumsum(v, axis=1))
    _, _, E = oracle.scan_fwd(np.full_like(v, -1000.0), v, q, mode=0, states=True)
    np.testing.assert_array_equal(E, v)
    # controlled with a = -1000: g = 0, write amount 1 - g = 1 -> E = v
    _, _, E = oracle.scan_fwd(np.full_like(v, -1000.0), v, q, mode=1, states=True)
    np.testing.assert_array_equal(E, v)
    # controlled with a = +1000: g = 1, nothing written -> the initial state is kept
    e0 = rng.normal(size=(B, H, Dh))
    _, eT = oracle.scan_fwd(np.full_like(v, 1000.0), v, q, e0, mode=1)
    np.testing.assert_array_equal(eT, e0)


def test_empty_sequence_returns_initial_state():
    a = np.zeros((2, 0, 2, 4))
    e0 = np.arange(16, dtype=np.float64).reshape(2, 2, 4)
    y, eT = oracle.scan_fwd(a, a, a, e0, mode=1)
    assert y.shape == a.shape
    np.testing.assert_array_equal(eT, e0)
    _, eT0 = oracle.scan_fwd(a, a, a, None, mode=1)
    np.testing.assert_array_equal(eT0, np.zeros((2, 2, 4)))


def test_threaded_rows_identical():
    a, v, q, e0 = rand_inputs(5, 33, 2, 8, 77)
    y1, e1 = oracle.scan_fwd(a, v, q, e0, mode=1, threads=1)
    y4, e4 = oracle.scan_fwd(a, v, q, e0, mode=1, threads=4)
    np.testing.assert_array_equal(y1, y4)
    np.testing.assert_array_equal(e1, e4)
