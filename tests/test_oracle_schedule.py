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


# ---------------------------------------------------------------------------
# asynchronous variant: capacity from history, order from the current step
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(30))
def test_async_capacity_is_the_global_optimum_of_history(seed):
    """n* attains the best value over every allocation of the historical survivals
    (brute force over {0..gamma}^B), jagged tables included (no early stop)."""
    rs = np.random.default_rng(300 + seed)
    B, gamma = int(rs.integers(1, 5)), int(rs.integers(1, 4))
    hist = synth.survival_rows(B, gamma, seed + 7).double().numpy()
    now = synth.survival_rows(B, gamma, seed + 8).double().numpy()
    sps = rs.uniform(5, 10, size=B + B * gamma).astype(np.float32)
    sps = np.sort(sps)[::-1].copy()
    sps[B + int(rs.integers(0, B * gamma)):] *= 0.85      # a cliff somewhere
    best, by_n = _brute_force(hist, sps.astype(np.float64))
    res = oracle.schedule_async(now.astype(np.float32), hist.astype(np.float32), sps)
    assert abs(res.theta - best) <= 1e-12 * best
    assert abs(by_n[res.n_selected] - best) <= 1e-12 * best
    assert all(by_n[n] < best * (1 - 1e-12) for n in by_n if n < res.n_selected)   # first maximum


@pytest.mark.parametrize("seed", range(10))
def test_async_admits_the_best_current_allocation_of_that_size(seed):
    rs = np.random.default_rng(400 + seed)
    B, gamma = 3, 3
    hist = synth.survival_rows(B, gamma, seed + 1).double().numpy()
    now = synth.survival_rows(B, gamma, seed + 2).double().numpy()
    sps = np.linspace(10, 7, B + B * gamma).astype(np.float32)
    res = oracle.schedule_async(now.astype(np.float32), hist.astype(np.float32), sps)
    # among all prefix allocations with n* candidates, K maximises the current survival sum
    best = max(sum(now[b, :K[b]].sum() for b in range(B))
               for K in itertools.product(range(gamma + 1), repeat=B) if sum(K) == res.n_selected)
    got = sum(now[b, :int(res.K[b])].sum() for b in range(B))
    assert abs(got - best) <= 1e-12
    assert int(res.K.sum()) == res.n_selected


@pytest.mark.parametrize("seed", range(20))
def test_async_equals_sync_when_history_is_current_and_objective_unimodal(seed):
    rs = np.random.default_rng(500 + seed)
    B, gamma = int(rs.integers(1, 6)), int(rs.integers(1, 5))
    a = synth.survival_rows(B, gamma, seed + 3)
    s_, p = rs.uniform(0.05, 0.6), rs.uniform(0.5, 2.0)
    sps = (100.0 / (1.0 + s_ * np.arange(1, B + B * gamma + 1)) ** p).astype(np.float32)
    _, by_n = _brute_force(a.double().numpy(), sps.astype(np.float64))
    if not _unimodal([by_n[n] for n in sorted(by_n)]):
        pytest.skip("profile not unimodal for this draw")
    sy = oracle.schedule(a, sps)
    asy = oracle.schedule_async(a, a, sps)
    assert np.array_equal(sy.K, asy.K) and sy.n_selected == asy.n_selected and sy.theta == asy.theta


def test_async_beats_the_early_stop_on_a_cliff():
    """With a cliff right after the first admissions the early stop halts in a
    local optimum; the global search over the same survivals goes past it."""
    a = synth.survival_rows(8, 4, 11)
    sps = np.linspace(1000, 990, 8 + 32).astype(np.float32)
    sps[8 + 2:8 + 6] *= 0.9          # a dip the early stop cannot cross
    sy = oracle.schedule(a, sps)
    asy = oracle.schedule_async(a, a, sps)
    assert asy.theta > sy.theta and asy.n_selected > sy.n_selected


def test_async_capacity_depends_on_history_only_through_its_values():
    a = synth.survival_rows(16, 5, 21)
    h = synth.survival_rows(16, 5, 22)
    sps = synth.sps_table(64)
    base = oracle.schedule_async(a, h, sps)
    perm = h.flatten()[torch.randperm(80, generator=torch.Generator().manual_seed(1))].reshape(16, 5)
    assert oracle.schedule_async(a, perm, sps).n_selected == base.n_selected
    # and the admitted set follows the current order only: a positive scale keeps K
    assert np.array_equal(oracle.schedule_async(a * 0.5, h, sps).K, base.K)
