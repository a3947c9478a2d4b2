"""Pins of the oracle's per-token L2 normalisation (CPU only).

The normalisation divides each (token, head) 128-vector of q and k by its
Euclidean norm.  Pins: rows of integer norm worked by hand, the unit length
and direction of every normalised row, scale invariance (the method's result
with normalised q and k does not change when raw q or k rows are scaled by
positive factors), equality with inputs that are already unit, and planted
mistakes that some pin rejects.
"""

import json
import os

import numpy as np
import pytest

from oracle import gdn_recurrence, l2_normalize

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_worked_rows():
    with open(os.path.join(GOLDEN, "l2norm_hand.json")) as f:
        gold = json.load(f)
    np.testing.assert_allclose(l2_normalize(np.array(gold["x"], float)), np.array(gold["x_hat"]), rtol=0,
                               atol=1e-16)


def _checks(fn, rng):
    """The pins as one predicate over a normalisation function: True when
    every pin holds."""
    x = rng.standard_normal((50, 3, 128)) * rng.uniform(0.01, 100, (50, 3, 1))
    xh = fn(x)
    norms = np.linalg.norm(xh, axis=-1)
    if not np.allclose(norms, 1.0, rtol=0, atol=1e-14):
        return False
    # same direction: x_hat . x = |x| per (token, head)
    if not np.allclose(np.sum(xh * x, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-14, atol=0):
        return False
    c = rng.uniform(0.001, 1000, (50, 3, 1))
    if not np.allclose(fn(c * x), xh, rtol=0, atol=1e-15):
        return False
    with open(os.path.join(GOLDEN, "l2norm_hand.json")) as f:
        gold = json.load(f)
    got = fn(np.array(gold["x"], float)[:, None, :])[:, 0]
    return np.allclose(got, np.array(gold["x_hat"]), rtol=0, atol=1e-16)


def test_unit_length_direction_and_scale_invariance():
    assert _checks(l2_normalize, np.random.default_rng(0))


def test_zero_vector_stays_zero_and_unit_rows_stay():
    x = np.zeros((2, 4, 128))
    assert np.array_equal(l2_normalize(x), x)
    u = np.random.default_rng(1).standard_normal((16, 2, 128))
    u /= np.linalg.norm(u, axis=-1, keepdims=True)
    np.testing.assert_allclose(l2_normalize(u), u, rtol=0, atol=1e-15)


@pytest.mark.parametrize("mistake", ["squared_norm", "wrong_axis", "epsilon", "l1_norm"])
def test_planted_mistakes_are_rejected(mistake):
    def bad(x):
        x = np.asarray(x, float)
        if mistake == "squared_norm":
            n = np.sum(x * x, axis=-1, keepdims=True)
        elif mistake == "wrong_axis":  # over the heads instead of the components
            n = np.sqrt(np.sum(x * x, axis=-2, keepdims=True))
        elif mistake == "epsilon":     # a sizeable epsilon inside the root
            n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + 1e-2)
        else:
            n = np.sum(np.abs(x), axis=-1, keepdims=True)
        return np.divide(x, n, out=np.zeros_like(x), where=n > 0)
    assert not _checks(bad, np.random.default_rng(0))


def _problem(rng, T=70, nk=2, nv=4, d=128):
    q = rng.standard_normal((T, nk, d))
    k = rng.standard_normal((T, nk, d))
    v = rng.standard_normal((T, nv, d))
    g = -np.logaddexp(0.0, rng.standard_normal((T, nv)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, nv))))
    h0 = 0.02 * rng.standard_normal((nv, d, d))
    return q, k, v, g, beta, h0


def test_recurrence_on_normalised_inputs_is_scale_invariant():
    """Scaling raw query and key rows by positive per-token factors leaves the
    method's result unchanged once they are normalised."""
    rng = np.random.default_rng(2)
    q, k, v, g, beta, h0 = _problem(rng)
    o1, h1, _ = gdn_recurrence(l2_normalize(q), l2_normalize(k), v, g, beta, h0)
    cq = rng.uniform(0.01, 50, q.shape[:2] + (1,))
    ck = rng.uniform(0.01, 50, k.shape[:2] + (1,))
    o2, h2, _ = gdn_recurrence(l2_normalize(cq * q), l2_normalize(ck * k), v, g, beta, h0)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(h2, h1, rtol=0, atol=1e-12)


def test_normalising_unit_inputs_changes_nothing():
    rng = np.random.default_rng(3)
    q, k, v, g, beta, h0 = _problem(rng)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    o1, h1, _ = gdn_recurrence(q, k, v, g, beta, h0)
    o2, h2, _ = gdn_recurrence(l2_normalize(q), l2_normalize(k), v, g, beta, h0)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(h2, h1, rtol=0, atol=1e-12)
