"""Pins of the STS fitting oracle (oracle/sts_fit.py) to things other than
itself: a hand-worked fixture of the binned ECE and of a two-position fit
(tests/golden/sts_fit_tiny.json), the ECE rebuilt from scikit-learn's
reliability curve and numpy's histogram, the label-flip symmetry and bounds
of the ECE, independence of a position's fit from the positions after it,
and recovery of the known over-confidence factors of a synthetic head (the
world of synth.sts_calibration_set, where sigmoid(l / T*_k) is exactly the
true acceptance probability, so the survival product under T* is the true
probability of the label).
"""
import json
import math
import os

import numpy as np
import pytest

import synth
from oracle.sts_fit import ece, labels, candidate_scores, sts_fit

GOLD = os.path.join(os.path.dirname(__file__), "golden", "sts_fit_tiny.json")


def _gold():
    with open(GOLD) as f:
        return json.load(f)


def _logit(tok: str) -> float:
    sign = -1.0 if tok.startswith("-") else 1.0
    return sign * math.log(float(tok.lstrip("-")[2:]))


@pytest.mark.parametrize("i", range(5))
def test_ece_hand_cases(i):
    c = _gold()["ece_cases"][i]
    assert ece(c["score"], c["label"], c["n_bins"]) == pytest.approx(c["ece"], abs=1e-15)


def test_two_position_fit_by_hand():
    c = _gold()["fit_case"]
    l = np.array([[_logit(t) for t in row] for row in c["logit"]])
    fit = sts_fit(l, c["accept_len"], c["grid"], c["n_bins"])
    assert list(fit.T) == c["T"]
    assert list(fit.index) == [c["grid"].index(t) for t in c["T"]]
    np.testing.assert_allclose(fit.ece, np.array(c["ece"]), rtol=1e-13, atol=0)
    # the second position scored with an unscaled first position: a fit that
    # forgot the earlier temperature would pick the other candidate
    wrong = sts_fit(l, c["accept_len"], c["grid"], c["n_bins"], T_fixed=[1.0, 1.0])
    np.testing.assert_allclose(wrong.ece[1], c["ece_if_prefix_unscaled"], rtol=1e-13, atol=0)
    assert wrong.T[1] != fit.T[1]


def _random_scores(n, seed):
    rs = np.random.default_rng(seed)
    s = rs.random(n)
    y = (rs.random(n) < s ** 1.3).astype(np.float64)
    return s, y


@pytest.mark.parametrize("n_bins", [1, 2, 10, 15, 37])
def test_ece_equals_reliability_curve_gap(n_bins):
    from sklearn.calibration import calibration_curve
    s, y = _random_scores(5000, 11 + n_bins)
    prob_true, prob_pred = calibration_curve(y, s, n_bins=n_bins, strategy="uniform")
    counts, _ = np.histogram(s, bins=np.linspace(0.0, 1.0, n_bins + 1))
    counts = counts[counts > 0]
    want = float(np.sum(np.abs(prob_true - prob_pred) * counts) / s.size)
    assert ece(s, y, n_bins) == pytest.approx(want, rel=1e-12, abs=1e-15)


def test_ece_label_flip_symmetry_and_bounds():
    s, y = _random_scores(3000, 5)
    for M in (3, 15, 64):
        e = ece(s, y, M)
        assert 0.0 <= e <= 1.0
        # bins mirror when no score sits on an edge
        assert ece(1.0 - s, 1.0 - y, M) == pytest.approx(e, rel=1e-12)
    # perfect scores
    assert ece(y, y, 15) == 0.0
    # a single bin: |mean label - mean score|
    assert ece(s, y, 1) == pytest.approx(abs(y.mean() - s.mean()), rel=1e-12)


def test_labels_are_leading_acceptance():
    a = np.array([0, 1, 3, 3, 2])
    assert list(labels(a, 1)) == [0, 1, 1, 1, 1]
    assert list(labels(a, 3)) == [0, 0, 1, 1, 0]


def test_candidate_scores_are_the_scaled_product():
    rs = np.random.default_rng(3)
    l = rs.normal(size=(6, 3)) * 2
    S = candidate_scores(l, 3, [0.5, 2.0], [1.0, 4.0])
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))
    for n in range(6):
        pre = sig(l[n, 0] / 0.5) * sig(l[n, 1] / 2.0)
        assert S[0, n] == pytest.approx(pre * sig(l[n, 2]), rel=1e-14)
        assert S[1, n] == pytest.approx(pre * sig(l[n, 2] / 4.0), rel=1e-14)


def test_fit_of_a_position_ignores_later_positions():
    d = synth.sts_calibration_set(4000, 5, seed=2)
    l, a = d["logit"].numpy(), d["accept_len"].numpy()
    grid = synth.sts_grid(24, 0.6, 0.1).numpy()
    full = sts_fit(l, a, grid, 15)
    part = sts_fit(l[:, :3], np.minimum(a, 3), grid, 15)
    assert np.array_equal(full.T[:3], part.T)
    assert np.array_equal(full.ece[:3], part.ece)


def test_ties_and_single_candidate():
    d = synth.sts_calibration_set(500, 2, seed=4)
    l, a = d["logit"].numpy(), d["accept_len"].numpy()
    one = sts_fit(l, a, [1.7], 10)
    assert list(one.T) == [1.7, 1.7] and list(one.index) == [0, 0]
    tie = sts_fit(l, a, [2.0, 2.0, 0.5], 10)
    assert tie.ece[0, 0] == tie.ece[0, 1]
    assert tie.index[0] in (0, 2) and tie.index[0] != 1
    empty = sts_fit(np.zeros((0, 3)), np.zeros(0, dtype=np.int32), [1.0, 2.0], 10)
    assert list(empty.index) == [0, 0, 0] and not empty.ece.any()


def test_recovers_the_over_confidence_of_a_synthetic_head():
    # sigmoid(l / T*_k) is the true acceptance probability of position k, so
    # T* is the calibrated choice; the grid search must land within two grid
    # steps of it, and calibrating must beat the raw scores (T = 1)
    true_T = np.array([1.3, 1.85, 1.1, 1.6])
    d = synth.sts_calibration_set(200_000, 4, seed=17, true_T=true_T)
    l, a = d["logit"].numpy(), d["accept_len"].numpy()
    grid = synth.sts_grid().numpy()
    fit = sts_fit(l, a, grid, 15)
    assert np.all(np.abs(fit.T - true_T) <= 0.1 + 1e-6), (fit.T, true_T)
    raw = int(np.argmin(np.abs(grid - 1.0)))
    assert np.all(fit.ece.min(axis=1) < 0.5 * fit.ece[:, raw])
    assert fit.ece.min(axis=1).max() < 0.01
