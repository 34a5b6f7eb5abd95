"""Pins for the oracle's one-token update, and sequence invariants of the forward.

Page "Entangled State Attention" ("[ ARCHITECTURE ]") states that the same recurrence is
composed over the sequence for prefill and carried one token at a time for generation, and
that the state shape [B, H, D] does not depend on the prompt length ("[ GENERATION /
MEMORY ]").  Page "entangled-state-attention 0.1.0" lists a "causal behavior" test.
Pinned here: the step equals a T = 1 scan, prefill followed by steps equals one long scan
(bit for bit, same operation order), resuming a scan from its final state equals the
unsplit scan, and outputs before t0 ignore every input at or after t0.
"""
import json
import os

import numpy as np
import pytest

import oracle


def inputs(seed, B, T, H, Dh, a_mean=0.0, a_std=1.0):
    rng = np.random.default_rng(seed)
    shp = (B, T, H, Dh)
    return (rng.normal(a_mean, a_std, size=shp), rng.normal(size=shp), rng.normal(size=shp),
            rng.normal(size=(B, H, Dh)))


@pytest.mark.parametrize("mode", [0, 1])
def test_step_equals_length_one_scan(mode):
    a, v, q, e0 = inputs(1, 3, 1, 2, 8)
    y_scan, e_scan = oracle.scan_fwd(a, v, q, e0, mode=mode)
    y_step, e_step = oracle.state_step(a[:, 0], v[:, 0], q[:, 0], e0, mode=mode)
    np.testing.assert_array_equal(y_step, y_scan[:, 0])
    np.testing.assert_array_equal(e_step, e_scan)


@pytest.mark.parametrize("mode", [0, 1])
def test_prefill_then_steps_equals_full_scan(mode):
    B, T1, n, H, Dh = 2, 23, 9, 2, 8
    a, v, q, _ = inputs(2, B, T1 + n, H, Dh)
    y_full, e_full = oracle.scan_fwd(a, v, q, None, mode=mode)
    y_pre, state = oracle.scan_fwd(a[:, :T1], v[:, :T1], q[:, :T1], None, mode=mode)
    np.testing.assert_array_equal(y_pre, y_full[:, :T1])
    for k in range(n):
        t = T1 + k
        y_t, state = oracle.state_step(a[:, t], v[:, t], q[:, t], state, mode=mode)
        np.testing.assert_array_equal(y_t, y_full[:, t])
    np.testing.assert_array_equal(state, e_full)


@pytest.mark.parametrize("mode", [0, 1])
def test_resume_from_final_state(mode):
    B, T1, T2, H, Dh = 2, 31, 17, 3, 4
    a, v, q, e0 = inputs(3, B, T1 + T2, H, Dh)
    y_full, e_full = oracle.scan_fwd(a, v, q, e0, mode=mode)
    y1, e1 = oracle.scan_fwd(a[:, :T1], v[:, :T1], q[:, :T1], e0, mode=mode)
    y2, e2 = oracle.scan_fwd(a[:, T1:], v[:, T1:], q[:, T1:], e1, mode=mode)
    np.testing.assert_array_equal(np.concatenate([y1, y2], axis=1), y_full)
    np.testing.assert_array_equal(e2, e_full)


@pytest.mark.parametrize("mode", [0, 1])
def test_causality(mode):
    B, T, H, Dh, t0 = 2, 40, 2, 4, 17
    a, v, q, e0 = inputs(4, B, T, H, Dh)
    y, _ = oracle.scan_fwd(a, v, q, e0, mode=mode)
    rng = np.random.default_rng(5)
    a2, v2, q2 = a.copy(), v.copy(), q.copy()
    for x in (a2, v2, q2):
        x[:, t0:] += rng.normal(size=x[:, t0:].shape)
    y2, _ = oracle.scan_fwd(a2, v2, q2, e0, mode=mode)
    np.testing.assert_array_equal(y2[:, :t0], y[:, :t0])
    assert np.all(y2[:, t0] != y[:, t0])


def test_lanes_are_independent():
    """Each (b, h, d) lane's state depends only on that lane's inputs."""
    B, T, H, Dh = 2, 16, 2, 4
    a, v, q, e0 = inputs(6, B, T, H, Dh)
    _, eT = oracle.scan_fwd(a, v, q, e0, mode=1)
    v2 = v.copy()
    v2[1, :, 0, 2] += 1.0
    _, eT2 = oracle.scan_fwd(a, v2, q, e0, mode=1)
    diff = np.argwhere(eT2 != eT)
    assert [tuple(d) for d in diff] == [(1, 0, 2)]


def test_state_shape_independent_of_prompt_length():
    """The state keeps the shape [B, H, Dh] for every prompt length."""
    golden = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                         "pages_shapes.json")))
    fact = golden["state_shape"]
    B, H, Dh = 2, 2, 4
    for T in fact["prompt_lengths"]:
        a, v, q, _ = inputs(7, B, T, H, Dh)
        _, eT = oracle.scan_fwd(a, v, q, None, mode=1)
        assert list(eT.shape) == [B, H, Dh]
