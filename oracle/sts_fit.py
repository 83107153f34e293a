"""Fitting the sequential temperature scaling (STS) of the confidence head.

TEST INFRASTRUCTURE ONLY (see the package header).

[blog] "校准问题：原始置信度不可靠": the per-position temperatures T_k are
learnt on held-out drafts, one position after another.  For position k the
temperature is picked by a one-dimensional grid search minimising the
expected calibration error (ECE) of the temperature-scaled survival
probability against the measured acceptance of positions 1..k.  [summary]
section 4 describes the same calibration: a left-to-right search, position by
position, for the temperature that brings the calibrated joint probability
closest to the measured acceptance (ECE of 3-8 % before, about 1 % after).

Readings (the pages leave these open):
  - Sequential means the earlier positions keep the temperatures already
    fitted: the score of sample n at position k under candidate T is
        S_n(T) = prod_{i<k} sigmoid(l_{n,i} / T_i) * sigmoid(l_{n,k} / T)
    with T_i the fitted temperatures of positions i < k.  (The blog's step 3
    writes one T_k inside the whole product; applying a per-position T_k at
    serving time, as both pages do, needs the per-position form above.)
  - The label of sample n at position k is 1 when its first k drafted tokens
    were all accepted (accepted length >= k), else 0: the event whose
    probability the survival product a_k predicts.
  - ECE is the textbook binned form with equal-width bins on [0, 1]: bin
    m = min(floor(S * M), M - 1) (so bin m holds [m/M, (m+1)/M) and 1.0 falls
    in the last bin), ECE = sum over non-empty bins of
    (n_m / N) * |mean label - mean score|.  An empty sample set has ECE 0.
  - The candidate temperatures and M are the caller's; ties go to the
    lowest candidate index.
"""
from __future__ import annotations

import dataclasses

import numpy as np


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def ece(score, label, n_bins: int) -> float:
    """Binned expected calibration error of scores in [0, 1] against 0/1
    labels, equal-width bins (see the module readings)."""
    s = np.asarray(score, dtype=np.float64).reshape(-1)
    y = np.asarray(label, dtype=np.float64).reshape(-1)
    n = s.size
    if n == 0:
        return 0.0
    m = np.minimum(np.floor(s * n_bins).astype(np.int64), n_bins - 1)
    total = 0.0
    for b in range(n_bins):
        sel = m == b
        nb = int(sel.sum())
        if nb == 0:
            continue
        total += (nb / n) * abs(float(y[sel].mean()) - float(s[sel].mean()))
    return total


def labels(accept_len, k: int) -> np.ndarray:
    """0/1 label of every sample at 1-based position k: accepted length >= k."""
    return (np.asarray(accept_len, dtype=np.int64) >= k).astype(np.float64)


def candidate_scores(logit, k: int, T_prev, grid) -> np.ndarray:
    """Calibrated survival at 1-based position k for every candidate
    temperature: S[g, n] = prod_{i<k} sigmoid(l[n, i] / T_prev[i]) *
    sigmoid(l[n, k-1] / grid[g])."""
    l = np.asarray(logit, dtype=np.float64)
    T_prev = np.asarray(T_prev, dtype=np.float64).reshape(-1)
    assert T_prev.size == k - 1
    prefix = np.ones(l.shape[0])
    for i in range(k - 1):
        prefix = prefix * _sigmoid(l[:, i] / T_prev[i])
    g = np.asarray(grid, dtype=np.float64).reshape(-1)
    return prefix[None, :] * _sigmoid(l[None, :, k - 1] / g[:, None])


@dataclasses.dataclass
class StsFit:
    T: np.ndarray       # float64 [gamma]: fitted temperature of every position
    index: np.ndarray   # int64 [gamma]: its index in the candidate grid
    ece: np.ndarray     # float64 [gamma, n_grid]: ECE of every candidate


def sts_fit(logit, accept_len, grid, n_bins: int, T_fixed=None) -> StsFit:
    """Fit T_1..T_gamma left to right.

    logit: [N, gamma] raw confidence logits l = logit(c) of held-out drafts;
    accept_len: [N] accepted lengths in 0..gamma; grid: candidate
    temperatures (> 0).  T_fixed, if given, replaces the fitted temperature
    of each earlier position by its own entry when later positions are
    scored (the tables of every position are then those that follow from
    that choice); the reported T and index are still each position's own
    minimiser."""
    l = np.asarray(logit, dtype=np.float64)
    N, gamma = l.shape
    g = np.asarray(grid, dtype=np.float64).reshape(-1)
    table = np.zeros((gamma, g.size))
    T = np.zeros(gamma)
    idx = np.zeros(gamma, dtype=np.int64)
    used = []
    for k in range(1, gamma + 1):
        S = candidate_scores(l, k, used, g)
        y = labels(accept_len, k)
        for j in range(g.size):
            table[k - 1, j] = ece(S[j], y, n_bins)
        best = int(np.argmin(table[k - 1]))      # first minimum
        idx[k - 1] = best
        T[k - 1] = g[best]
        used.append(T[k - 1] if T_fixed is None else float(T_fixed[k - 1]))
    return StsFit(T, idx, table)
