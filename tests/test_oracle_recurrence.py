"""Pins for the oracle's core recurrence E_t = A_t * E_{t-1} + B_t.

The recurrence is the one printed on page "Entangled State Attention v2.1" (introduction)
and page "Entangled State Attention" ("[ ARCHITECTURE ]", core recurrence).  Each test
checks the oracle against something that is not the oracle's own loop: the O(T^2) closed
form, the special cases A = 0 and A = 1 (numpy's prefix sum), the constant-A geometric
series, and the bracketing invariance of the pair combine
(a1, b1) o (a2, b2) = (a1 a2, a2 b1 + b2) that the same page's "Associative composition"
relies on.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle


def closed_form(A, Bt, E0):
    """E_t = sum_{s<=t} (prod_{r=s+1..t} A_r) B_s + (prod_{r<=t} A_r) E_{-1}, by brute force."""
    T, nl = A.shape
    E = np.zeros((T, nl))
    for t in range(T):
        acc = np.prod(A[: t + 1], axis=0) * E0
        for s in range(t + 1):
            acc = acc + np.prod(A[s + 1 : t + 1], axis=0) * Bt[s]
        E[t] = acc
    return E


@pytest.mark.parametrize("T,nl,seed", [(1, 3, 0), (5, 4, 1), (33, 6, 2), (64, 2, 3)])
def test_closed_form(T, nl, seed):
    rng = np.random.default_rng(seed)
    A = rng.uniform(0.0, 1.0, size=(T, nl))
    Bt = rng.normal(size=(T, nl))
    E0 = rng.normal(size=nl)
    E = oracle.recurrence(A, Bt, E0)
    ref = closed_form(A, Bt, E0)
    np.testing.assert_allclose(E, ref, rtol=1e-12, atol=1e-12)


def test_zero_initial_state_default():
    rng = np.random.default_rng(7)
    A = rng.uniform(size=(9, 3))
    Bt = rng.normal(size=(9, 3))
    np.testing.assert_array_equal(oracle.recurrence(A, Bt), oracle.recurrence(A, Bt, np.zeros(3)))


def test_A_zero_gives_B():
    rng = np.random.default_rng(11)
    Bt = rng.normal(size=(17, 5))
    E = oracle.recurrence(np.zeros_like(Bt), Bt, rng.normal(size=5))
    np.testing.assert_array_equal(E, Bt)


def test_A_one_gives_prefix_sum():
    rng = np.random.default_rng(12)
    Bt = rng.normal(size=(200, 4))
    E = oracle.recurrence(np.ones_like(Bt), Bt)
    np.testing.assert_array_equal(E, np.cumsum(Bt, axis=0))


@pytest.mark.parametrize("c", [0.0, 0.25, 0.9, 0.999])
def test_constant_A_geometric_series(c):
    T = 300
    E0 = np.array([2.0, -3.0])
    E = oracle.recurrence(np.full((T, 2), c), np.ones((T, 2)), E0)
    t = np.arange(T)[:, None] + 1.0
    ref = c**t * E0 + (1.0 - c**t) / (1.0 - c)
    np.testing.assert_allclose(E, ref, rtol=1e-13, atol=1e-13)


def combine(x, y):
    """(a1, b1) o (a2, b2) = (a1 a2, a2 b1 + b2): x covers earlier steps than y."""
    return (x[0] * y[0], y[0] * x[1] + y[1])


def fold_bracketed(pairs, cuts):
    """Combine a list of (A_t, B_t) pairs with an arbitrary bracketing given by `cuts`."""
    if len(pairs) == 1:
        return pairs[0]
    k = cuts[0] % (len(pairs) - 1) + 1
    left = fold_bracketed(pairs[:k], cuts[1:] or [0])
    right = fold_bracketed(pairs[k:], cuts[1:] or [0])
    return combine(left, right)


@settings(max_examples=150, deadline=None)
@given(
    st.lists(st.tuples(st.sampled_from([0.0, 0.25, 0.5, 0.75, 1.0]),
                       st.integers(-8, 8)), min_size=1, max_size=40),
    st.lists(st.integers(0, 1000), min_size=1, max_size=12),
    st.integers(-8, 8),
)
def test_bracketing_invariance_exact(steps, cuts, e0):
    """Any bracketing of the pair combine reproduces the sequential loop bit for bit
    (dyadic A and small integer B keep every fp64 operation exact)."""
    A = np.array([[s[0]] for s in steps])
    Bt = np.array([[float(s[1])] for s in steps])
    E = oracle.recurrence(A, Bt, np.array([float(e0)]))
    agg = fold_bracketed([(a, b) for a, b in zip(A[:, 0], Bt[:, 0])], cuts)
    assert agg[1] + agg[0] * e0 == E[-1, 0]
    # the prefix up to any t, too
    for t in range(len(steps)):
        pre = fold_bracketed([(a, b) for a, b in zip(A[: t + 1, 0], Bt[: t + 1, 0])], cuts)
        assert pre[1] + pre[0] * e0 == E[t, 0]


def test_chunked_composition_matches_random():
    """Chunk aggregates combined left to right equal the sequential loop to rounding."""
    rng = np.random.default_rng(5)
    T, nl, L = 257, 7, 16
    A = rng.uniform(0.5, 1.0, size=(T, nl))
    Bt = rng.normal(size=(T, nl))
    E0 = rng.normal(size=nl)
    E = oracle.recurrence(A, Bt, E0)
    carry = E0.copy()
    for t0 in range(0, T, L):
        P = np.prod(A[t0 : t0 + L], axis=0)
        Eloc = oracle.recurrence(A[t0 : t0 + L], Bt[t0 : t0 + L])[-1]
        carry = Eloc + P * carry
        np.testing.assert_allclose(carry, E[min(T, t0 + L) - 1], rtol=1e-12, atol=1e-12)
