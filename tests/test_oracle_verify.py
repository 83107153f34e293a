"""Pins of the oracle's lossless accept/reject, residual and bonus (CPU only)."""
import itertools
import json
import os

import numpy as np
import pytest
import torch
from scipy import stats
from scipy.special import softmax, logsumexp

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden", "verify_greedy_tiny.json")


@pytest.mark.parametrize("case", json.load(open(GOLD))["cases"], ids=lambda c: c["name"])
def test_greedy_hand_worked(case):
    g = json.load(open(GOLD))
    V, gamma = g["V"], g["gamma"]
    tgt = torch.tensor(case["target"], dtype=torch.float32)[None]
    dummy = torch.zeros((1, gamma + 1, V))
    W = torch.zeros((V, 2))
    r = oracle.verify(tgt, [g["draft"]], np.zeros((1, gamma)), np.zeros((1, gamma)), dummy, W, W,
                      [0], [case["K"]], [0], 0.0, 0, gamma)
    assert int(r.accept_len[0]) == case["accept_len"]
    n = case["accept_len"] + 1
    assert r.out_tokens[0, :n].tolist() == case["out"]
    assert np.all(r.out_tokens[0, n:] == -1)


def test_greedy_accepts_longest_matching_prefix():
    rs = np.random.default_rng(1)
    B, gamma, V = 50, 7, 40
    tgt = rs.normal(size=(B, gamma + 1, V)).astype(np.float32)
    star = tgt.argmax(-1)
    draft = star[:, :gamma].copy()
    mismatch_at = rs.integers(0, gamma + 1, size=B)     # gamma = all match
    for b in range(B):
        if mismatch_at[b] < gamma:
            draft[b, mismatch_at[b]] = (star[b, mismatch_at[b]] + 1) % V
    W = np.zeros((V, 2))
    r = oracle.verify(tgt, draft, np.zeros((B, gamma)), np.zeros((B, gamma)), np.zeros_like(tgt),
                      W, W, np.zeros(B, dtype=int), None, np.arange(B), 0.0, 0, gamma)
    for b in range(B):
        m = int(mismatch_at[b])
        assert r.accept_len[b] == m
        assert r.out_tokens[b, :m].tolist() == draft[b, :m].tolist()
        assert r.out_tokens[b, m] == star[b, m]          # compensation or bonus (row gamma+1)


def _markov_case(V=3, gamma=2, seed=0):
    g = torch.Generator().manual_seed(seed)
    U = torch.randn((1, gamma + 1, V), generator=g) * 1.0
    tgt = torch.randn((1, gamma + 1, V), generator=g) * 1.0
    W1 = torch.randn((V, 2), generator=g) * 0.9
    W2 = torch.randn((V, 2), generator=g) * 0.9
    return U, tgt, W1, W2


def _pd(U, W1, W2, k, prev, T=1.0):
    """draft law at position k given the previous token, P3 one-hot form."""
    V = U.shape[-1]
    e = np.zeros(V)
    e[prev] = 1.0
    z = U[0, k - 1].double().numpy() + W2.double().numpy() @ (W1.double().numpy().T @ e)
    return softmax(z / T)


@pytest.mark.parametrize("seed,T", [(0, 1.0), (1, 1.0), (2, 0.7)])
def test_lossless_law_exact_enumeration(seed, T):
    """Sum over drafts and accept/reject paths of the oracle's ratio and residual
    pieces; the emitted sequence (padded with independent target draws after it
    stops) has law prod_j p_t^j.  [blog] 'Formal definition': output law equals
    the target's."""
    V, gamma = 3, 2
    U, tgt, W1, W2 = _markov_case(V, gamma, seed)
    anchor = 1
    lpt = [oracle.target_logprobs(tgt[0, j].double().numpy(), T) for j in range(gamma + 1)]
    pt = [np.exp(x) for x in lpt]
    law = np.zeros((V,) * (gamma + 1))
    for x in itertools.product(range(V), repeat=gamma):
        prevs = (anchor,) + x[:-1]
        pds = [_pd(U, W1, W2, k + 1, prevs[k], T) for k in range(gamma)]
        q = np.prod([pds[k][x[k]] for k in range(gamma)])
        alive = q
        for k in range(gamma):
            rho = oracle.accept_ratio(lpt[k][x[k]], np.log(pds[k][x[k]]))
            acc = min(1.0, rho)
            # reject at k: residual token, then independent target draws after it
            res = oracle.residual_weights(lpt[k], np.log(pds[k]))
            if res.sum() > 0:
                res = res / res.sum()
            rej = alive * (1 - acc)
            if rej > 0:
                for s in itertools.product(range(V), repeat=gamma + 1 - k):
                    p = rej * res[s[0]]
                    for j in range(1, gamma + 1 - k):
                        p *= pt[k + j][s[j]]
                    law[tuple(x[:k]) + s] += p
            alive *= acc
        for s in range(V):
            law[tuple(x) + (s,)] += alive * pt[gamma][s]
    target_law = np.einsum("i,j,k->ijk", pt[0], pt[1], pt[2])
    assert abs(law.sum() - 1) < 1e-12
    assert np.max(np.abs(law - target_law)) < 1e-12


def test_residual_mass_is_total_variation():
    rs = np.random.default_rng(0)
    for _ in range(20):
        a = rs.normal(size=50)
        b = rs.normal(size=50)
        la, lb = a - logsumexp(a), b - logsumexp(b)
        tv = 0.5 * np.abs(np.exp(la) - np.exp(lb)).sum()
        assert abs(oracle.residual_weights(la, lb).sum() - tv) < 1e-13


def _mc_run(seed, n, T=1.0, V=3, gamma=2, base_seed=2024):
    U, tgt, W1, W2 = _markov_case(V, gamma, seed)
    Ur = U.repeat(n, 1, 1)
    tr = tgt.repeat(n, 1, 1)
    anchor = np.full(n, 1)
    req = np.arange(n)
    d = oracle.draft_markov(Ur, W1, W2, anchor, req, T, base_seed, gamma)
    r = oracle.verify(tr, d.tokens, d.lse, d.ytok, Ur, W1, W2, anchor, None, req, T, base_seed, gamma)
    return U, tgt, W1, W2, d, r


@pytest.mark.parametrize("seed,T", [(0, 1.0), (3, 0.8)])
def test_lossless_law_monte_carlo(seed, T):
    """The oracle's own sampler (hash RNG, Gumbel-max, u < rho) reproduces prod p_t."""
    V, gamma, n = 3, 2, 30000
    U, tgt, W1, W2, d, r = _mc_run(seed, n, T, V, gamma)
    pt = [softmax(tgt[0, j].double().numpy() / T) for j in range(gamma + 1)]
    rs = np.random.default_rng(7)
    seqs = np.zeros((n, gamma + 1), dtype=int)
    for i in range(n):
        m = int(r.accept_len[i]) + 1
        seqs[i, :m] = r.out_tokens[i, :m]
        for j in range(m, gamma + 1):
            seqs[i, j] = rs.choice(V, p=pt[j])
    idx = seqs[:, 0] * V * V + seqs[:, 1] * V + seqs[:, 2]
    counts = np.bincount(idx, minlength=V ** 3)
    expect = n * np.einsum("i,j,k->ijk", *pt).reshape(-1)
    assert stats.chisquare(counts, expect).pvalue > 1e-4
    # first-position acceptance = sum_v min(p_d, p_t) = 1 - TV  ([summary] section 4)
    pd1 = _pd(U, W1, W2, 1, 1, T)
    p_acc = np.minimum(pd1, pt[0]).sum()
    emp = np.mean(r.accept_len >= 1)
    assert abs(emp - p_acc) < 5 * np.sqrt(p_acc * (1 - p_acc) / n)


def test_identical_laws_accept_everything():
    wl = synth.WORKLOADS["sample"].with_(B=16, V=500, conf=False)
    inp = synth.make_inputs(wl)
    W = torch.zeros_like(inp["W1"])
    d = oracle.draft_markov(inp["U"], W, W, inp["anchor"], inp["req_ids"], 1.0, 5, 7)
    r = oracle.verify(inp["U"], d.tokens, d.lse, d.ytok, inp["U"], W, W, inp["anchor"], None,
                      inp["req_ids"], 1.0, 5, 7)
    assert np.all(r.accept_len == 7)
    assert np.all(r.resid_row == 0)


def test_bonus_uses_row_after_last_verified():
    # K_b = 2 for all: the bonus (when all accepted) comes from row 3 with BONUS stream pos 3
    wl = synth.WORKLOADS["sample"].with_(B=32, V=300, conf=False)
    inp = synth.make_inputs(wl)
    W = torch.zeros_like(inp["W1"])
    d = oracle.draft_markov(inp["U"], W, W, inp["anchor"], inp["req_ids"], 1.0, 5, 7)
    K = np.full(32, 2)
    r = oracle.verify(inp["U"], d.tokens, d.lse, d.ytok, inp["U"], W, W, inp["anchor"], K,
                      inp["req_ids"], 1.0, 5, 7)
    for b in range(32):
        assert r.accept_len[b] == 2
        bonus, _ = oracle.gumbel_draw(inp["U"][b, 2].double().numpy(),
                                    oracle.row_key(5, int(inp["req_ids"][b]) & 0xFFFFFFFF, 3, oracle.BONUS))
        assert r.out_tokens[b, 2] == bonus
        assert np.all(r.out_tokens[b, 3:] == -1)


def test_accept_prob_is_one_minus_total_variation_and_matches_acceptance():
    """alpha = sum min(p_d, p_t) = 1 - TV (closed form on the rebuilt laws) and is the
    empirical first-position acceptance rate of the oracle's own sampler."""
    V, gamma, n, T = 3, 2, 30000, 1.0
    U, tgt, W1, W2, d, r = _mc_run(5, n, T, V, gamma)
    a = oracle.accept_prob(tgt.repeat(2, 1, 1), d.tokens[:2], d.lse[:2], U.repeat(2, 1, 1), W1, W2,
                           np.full(2, 1), T, gamma)
    pd1 = _pd(U, W1, W2, 1, 1, T)
    pt1 = softmax(tgt[0, 0].double().numpy() / T)
    assert abs(a[0, 0] - (1 - 0.5 * np.abs(pd1 - pt1).sum())) < 1e-12
    emp = np.mean(r.accept_len >= 1)
    assert abs(emp - a[0, 0]) < 5 * np.sqrt(a[0, 0] * (1 - a[0, 0]) / n)
    # position 2 given x_1: the same identity with the conditional draft law
    for i in range(2):
        pd2 = _pd(U, W1, W2, 2, int(d.tokens[i, 0]), T)
        pt2 = softmax(tgt[0, 1].double().numpy() / T)
        assert abs(a[i, 1] - np.minimum(pd2, pt2).sum()) < 1e-12


def test_accept_prob_limits():
    wl = synth.WORKLOADS["sample"].with_(B=4, V=300, conf=False)
    inp = synth.make_inputs(wl)
    W = torch.zeros_like(inp["W1"])
    d = oracle.draft_markov(inp["U"], W, W, inp["anchor"], inp["req_ids"], 1.0, 5, 7)
    same = oracle.accept_prob(inp["U"], d.tokens, d.lse, inp["U"], W, W, inp["anchor"], 1.0, 7)
    assert np.allclose(same, 1.0, atol=1e-12)          # identical laws: always accepted
    far = inp["U"].clone()
    far[:, :, :150] -= 60.0                           # target mass on the upper half only
    U2 = inp["U"].clone()
    U2[:, :, 150:] -= 60.0                            # draft mass on the lower half only
    d2 = oracle.draft_markov(U2, W, W, inp["anchor"], inp["req_ids"], 1.0, 5, 7)
    tiny = oracle.accept_prob(far, d2.tokens, d2.lse, U2, W, W, inp["anchor"], 1.0, 7)
    assert np.all(tiny < 1e-20)
