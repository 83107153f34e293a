"""Pins of the oracle's greedy prefix scheduler (CPU only)."""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden", "schedule_tiny.json")


@pytest.mark.parametrize("case", json.load(open(GOLD))["cases"], ids=lambda c: c["name"])
def test_hand_worked_cases(case):
    s = oracle.schedule(np.asarray(case["surv"], dtype=np.float32),
                        np.asarray(case["sps"], dtype=np.float32))
    assert s.K.tolist() == case["K"]
    assert s.n_selected == case["n_selected"]
    assert s.theta == case["theta"]


def _brute_force(a, sps):
    """Best Theta over every allocation K in {0..gamma}^B (prefixes per request)."""
    B, gamma = a.shape
    best = -np.inf
    best_by_n = {}
    for K in itertools.product(range(gamma + 1), repeat=B):
        n = sum(K)
        N = B + n
        if N > len(sps):
            continue
        S = sum(a[b, :K[b]].sum() for b in range(B))
        th = (B + S) * sps[N - 1]
        best = max(best, th)
        best_by_n[n] = max(best_by_n.get(n, -np.inf), th)
    return best, best_by_n


def _unimodal(seq):
    i = 0
    while i + 1 < len(seq) and seq[i + 1] > seq[i]:
        i += 1
    return all(seq[j + 1] <= seq[j] for j in range(i, len(seq) - 1))


@pytest.mark.parametrize("seed", range(40))
def test_matches_brute_force_when_objective_unimodal(seed):
    rs = np.random.default_rng(seed)
    B, gamma = int(rs.integers(1, 5)), int(rs.integers(1, 4))
    a = synth.survival_rows(B, gamma, seed).double().numpy()
    n_max = B * gamma
    # smooth, decreasing table: SPS(N) = c / (1 + s N)^p
    s_, p = rs.uniform(0.05, 0.6), rs.uniform(0.5, 2.0)
    sps = (100.0 / (1.0 + s_ * np.arange(1, B + n_max + 1)) ** p).astype(np.float32)
    best, by_n = _brute_force(a, sps.astype(np.float64))
    profile = [by_n[n] for n in sorted(by_n)]
    res = oracle.schedule(a.astype(np.float32), sps)
    if _unimodal(profile):
        assert abs(res.theta - best) <= 1e-12 * best
    else:
        assert res.theta <= best * (1 + 1e-12)
    # the greedy's value for its n equals the best allocation with that many tokens
    assert abs(res.theta - by_n[res.n_selected]) <= 1e-12 * best


@pytest.mark.parametrize("seed", range(10))
def test_cliffs_give_at_most_the_global_optimum(seed):
    rs = np.random.default_rng(100 + seed)
    B, gamma = 3, 3
    a = synth.survival_rows(B, gamma, seed + 50).double().numpy()
    sps = np.linspace(10, 8, B + B * gamma).astype(np.float32)
    sps[B + 1:] *= 0.8   # a cliff right after the first admission
    best, _ = _brute_force(a, sps.astype(np.float64))
    res = oracle.schedule(a.astype(np.float32), sps)
    assert res.theta <= best * (1 + 1e-12)


def test_admitted_sets_are_prefixes_and_respect_capacity():
    a = synth.survival_rows(64, 7, 3, ties=True)
    sps = synth.sps_table(200)
    s = oracle.schedule(a, sps)
    assert s.K.sum() == s.n_selected
    assert 64 + s.n_selected <= 200
    # the admitted survivals are the n largest under (a desc, b asc, j asc)
    cands = sorted(((float(a[b, j]), b, j) for b in range(64) for j in range(7)),
                   key=lambda e: (-e[0], e[1], e[2]))
    chosen = {(b, j) for _, b, j in cands[:s.n_selected]}
    assert chosen == {(b, j) for b in range(64) for j in range(int(s.K[b]))}


def test_synthetic_sps_table_shape():
    t = synth.sps_table(4096).double().numpy()
    assert np.all(np.diff(t) <= 0)
    steps = np.nonzero(np.diff(t))[0] + 2          # N at which the value changes
    assert set(synth.SPS_CLIFFS) <= set(steps.tolist())
    assert all((n - 1) % synth.SPS_STEP == 0 or n in synth.SPS_CLIFFS for n in steps)
