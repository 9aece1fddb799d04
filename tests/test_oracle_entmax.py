"""Pins for the oracle's alpha-entmax (CPU only).

Each check ties the bisection solver to something other than itself: hand-derived
closed forms (tests/golden), the sort-based closed forms of sparsemax and 1.5-entmax,
the KKT conditions of the Tsallis maximisation, the softmax limit alpha -> 1, and brute
force over the simplex for tiny n.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import dash_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _golden("entmax_closed_forms.json")["cases"])
def test_golden_closed_forms(case):
    x = np.array(case["x"])
    p_ref = np.array(case["p"])
    p = O.entmax(x, case["alpha"])
    np.testing.assert_allclose(p, p_ref, rtol=0, atol=1e-14)
    # exact zeros where the closed form has zeros
    assert np.all(p[p_ref == 0.0] == 0.0)
    if case["alpha"] == 2.0:
        np.testing.assert_allclose(O.sparsemax_sorted(x), p_ref, atol=1e-14)
    if case["alpha"] == 1.5:
        np.testing.assert_allclose(O.entmax15_sorted(x), p_ref, atol=1e-14)
    np.testing.assert_allclose(O.entmax_sorted_general(x, case["alpha"]), p_ref, atol=1e-12)


ALPHAS = [1.25, 1.5, 2.0, 3.0]


@pytest.mark.parametrize("alpha", ALPHAS)
@pytest.mark.parametrize("n", [1, 2, 3, 7, 64, 300])
def test_simplex_zeros_and_kkt(alpha, n):
    rng = np.random.default_rng(1000 + n)
    for trial in range(5):
        x = rng.normal(size=n) * rng.uniform(0.3, 4.0)
        p, tau, y = O.entmax(x, alpha, return_tau=True)
        assert abs(p.sum() - 1.0) <= 1e-12
        assert np.all(p >= 0.0)
        off = y <= tau
        assert np.all(p[off] == 0.0), "entries at or below the threshold must be exactly zero"
        on = ~off
        # stationarity: p_c^(alpha-1) = y_c - tau on the support
        np.testing.assert_allclose(p[on] ** (alpha - 1.0), y[on] - tau, rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("alpha", ALPHAS)
def test_special_inputs(alpha):
    assert O.entmax(np.array([0.37]), alpha).tolist() == [1.0]
    for n in (2, 5, 2048):
        p = O.entmax(np.full(n, -1.7), alpha)
        np.testing.assert_allclose(p, 1.0 / n, rtol=1e-12)


@pytest.mark.parametrize("alpha", ALPHAS)
def test_translation_and_permutation(alpha):
    rng = np.random.default_rng(7)
    x = rng.normal(size=40) * 2
    p = O.entmax(x, alpha)
    np.testing.assert_allclose(O.entmax(x + 3.25, alpha), p, atol=1e-12)
    perm = rng.permutation(x.size)
    np.testing.assert_allclose(O.entmax(x[perm], alpha), p[perm], atol=1e-12)


def test_batched_equals_rowwise():
    rng = np.random.default_rng(3)
    X = rng.normal(size=(6, 4, 33)) * 3
    P = O.entmax(X, 1.5)
    for idx in np.ndindex(6, 4):
        np.testing.assert_allclose(P[idx], O.entmax(X[idx], 1.5), atol=1e-15)


@pytest.mark.parametrize("n", [2, 3, 10, 129, 2048])
def test_alpha2_is_sparsemax(n):
    rng = np.random.default_rng(n)
    for _ in range(5):
        x = rng.normal(size=n) * rng.uniform(0.2, 5.0)
        np.testing.assert_allclose(O.entmax(x, 2.0), O.sparsemax_sorted(x), atol=1e-12)


@pytest.mark.parametrize("n", [2, 3, 10, 129, 2048])
def test_alpha15_matches_sorted_exact(n):
    rng = np.random.default_rng(50 + n)
    for _ in range(5):
        x = rng.normal(size=n) * rng.uniform(0.2, 5.0)
        np.testing.assert_allclose(O.entmax(x, 1.5), O.entmax15_sorted(x), atol=1e-12)


@pytest.mark.parametrize("alpha", [1.1, 1.25, 1.75, 3.0])
def test_general_alpha_matches_sorted_search(alpha):
    rng = np.random.default_rng(int(alpha * 100))
    for n in (2, 9, 100):
        x = rng.normal(size=n) * 2
        np.testing.assert_allclose(O.entmax(x, alpha), O.entmax_sorted_general(x, alpha),
                                   atol=1e-11)


@pytest.mark.parametrize("eps", [1e-1, 1e-2, 1e-3])
def test_alpha_to_one_is_softmax(eps):
    rng = np.random.default_rng(11)
    worst = 0.0
    for n in (2, 5, 16, 64):
        for _ in range(5):
            x = rng.uniform(-3.0, 3.0, size=n)
            worst = max(worst, np.abs(O.entmax(x, 1.0 + eps) - O.softmax(x)).max())
    assert worst <= 2.0 * eps


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0])
@pytest.mark.parametrize("n", [2, 3, 4])
def test_brute_force_maximiser(alpha, n):
    rng = np.random.default_rng(17 * n)
    for _ in range(3):
        x = rng.normal(size=n) * 1.5
        p = O.entmax(x, alpha)
        best = O.tsallis_objective(p, x, alpha)
        cands = rng.dirichlet(np.full(n, 0.5), size=10000)
        vals = cands @ x + (cands - cands ** alpha).sum(axis=1) / (alpha * (alpha - 1.0))
        assert best >= vals.max() - 1e-12
        # vertices and a local neighbourhood on the simplex
        for i in range(n):
            e = np.zeros(n)
            e[i] = 1.0
            assert best >= O.tsallis_objective(e, x, alpha) - 1e-12
        for _ in range(200):
            d = rng.normal(size=n) * 1e-3
            d -= d.mean()
            q = p + d
            if np.all(q >= 0):
                assert best >= O.tsallis_objective(q, x, alpha) - 1e-12


def test_rejects_bad_alpha():
    with pytest.raises(ValueError):
        O.entmax(np.zeros(3), 1.0)
    with pytest.raises(ValueError):
        O.entmax(np.zeros(3), float("nan"))
