"""Pins of the oracle's Markov-head draft (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch
from scipy import stats
from scipy.special import logsumexp, softmax

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden", "markov_bias_tiny.json")


def _storage_w2(w2_r_by_v):
    # the boundary stores the r x V matrix column-major: row v = column v
    return np.ascontiguousarray(np.asarray(w2_r_by_v, dtype=np.float64).T)


def test_bias_hand_worked_fixture():
    g = json.load(open(GOLD))
    W1 = np.asarray(g["W1_rows_by_token"], dtype=np.float64)
    W2 = _storage_w2(g["W2_r_by_V"])
    got = oracle.markov_bias(W1, W2, np.arange(g["V"]))
    assert np.array_equal(got, np.asarray(g["bias_by_prev"], dtype=np.float64))


def test_greedy_draft_hand_worked_fixture():
    g = json.load(open(GOLD))
    ex = g["draft_example"]
    W1 = torch.tensor(g["W1_rows_by_token"], dtype=torch.float32)
    W2 = torch.tensor(_storage_w2(g["W2_r_by_V"]), dtype=torch.float32)
    U = torch.tensor(ex["U"], dtype=torch.float32)[None]        # [1, 3, V]
    d = oracle.draft_markov(U, W1, W2, [ex["anchor"]], [0], 0.0, 0, 3, keep_logits=True)
    assert d.tokens[0].tolist() == ex["tokens"]
    assert np.array_equal(d.z[0], np.asarray(ex["z"], dtype=np.float64))
    # greedy lse is that of z itself; ytok is z at the token
    assert np.allclose(d.lse[0], logsumexp(np.asarray(ex["z"]), axis=1), rtol=0, atol=1e-12)
    assert np.array_equal(d.ytok[0], np.max(np.asarray(ex["z"]), axis=1))


def test_bias_equals_teardown_one_hot_form():
    """Logits_adj = Logits_par + B (A e_prev), A in R^{r x V}, B in R^{V x r}."""
    rs = np.random.default_rng(0)
    V, r = 37, 5
    W1 = rs.normal(size=(V, r))
    W2 = rs.normal(size=(V, r))
    A = W1.T                 # r x V: compresses the one-hot previous token
    Bm = W2                  # V x r: projects back to the vocabulary
    for prev in (0, 1, 17, V - 1):
        e = np.zeros(V)
        e[prev] = 1.0
        ref = Bm @ (A @ e)
        got = oracle.markov_bias(W1, W2, np.array([prev]))[0]
        assert np.allclose(got, ref, rtol=1e-13, atol=1e-13)


def _tiny_inputs(V=4, gamma=3, B=1, seed=0, zero_w=False, u_std=1.0, w_std=0.7):
    g = torch.Generator().manual_seed(seed)
    U = torch.randn((B, gamma + 1, V), generator=g) * u_std
    W1 = torch.randn((V, 3), generator=g) * w_std
    W2 = torch.randn((V, 3), generator=g) * w_std
    if zero_w:
        W1.zero_()
        W2.zero_()
    anchor = torch.randint(0, V, (B,), generator=g).to(torch.int32)
    return U, W1, W2, anchor


def test_zero_weights_reduce_to_parallel_draft_greedy():
    wl = synth.WORKLOADS["tiny"].with_(B=3, V=300)
    inp = synth.make_inputs(wl)
    W1 = torch.zeros_like(inp["W1"])
    W2 = torch.zeros_like(inp["W2"])
    d = oracle.draft_markov(inp["U"], W1, W2, inp["anchor"], inp["req_ids"], 0.0, 1, 7)
    assert np.array_equal(d.tokens, np.argmax(inp["U"][:, :7].numpy(), axis=-1))
    assert np.allclose(d.lse, logsumexp(inp["U"][:, :7].double().numpy(), axis=-1), atol=1e-12)


def test_zero_weights_stochastic_ignores_previous_token():
    # with W1 = W2 = 0 position k no longer depends on x_{k-1}: anchors do not matter
    U, W1, W2, anchor = _tiny_inputs(V=50, gamma=5, B=4, zero_w=True)
    d1 = oracle.draft_markov(U, W1, W2, [0, 1, 2, 3], [5, 6, 7, 8], 1.0, 3, 5)
    d2 = oracle.draft_markov(U, W1, W2, [9, 9, 9, 9], [5, 6, 7, 8], 1.0, 3, 5)
    assert np.array_equal(d1.tokens, d2.tokens)
    # and with nonzero weights the anchor does matter somewhere
    U, W1, W2, _ = _tiny_inputs(V=50, gamma=5, B=4, w_std=2.0)
    d1 = oracle.draft_markov(U, W1, W2, [0, 1, 2, 3], [5, 6, 7, 8], 1.0, 3, 5)
    d2 = oracle.draft_markov(U, W1, W2, [9, 9, 9, 9], [5, 6, 7, 8], 1.0, 3, 5)
    assert not np.array_equal(d1.lse, d2.lse)


def test_draws_follow_softmax():
    """The draft token at one position ~ softmax(y).  V = 8, chi-square."""
    V = 8
    y = np.array([0.3, -1.0, 2.0, 0.0, 1.1, -0.4, 0.8, 1.5])
    U = torch.tensor(y, dtype=torch.float32)[None, None, :].repeat(1, 2, 1)
    W = torch.zeros((V, 2))
    n = 20000
    counts = np.zeros(V)
    # requests as the varying counter: one call covers many independent draws
    reqs = np.arange(n)
    d = oracle.draft_markov(U.repeat(n, 1, 1), W, W, np.zeros(n, dtype=np.int32), reqs, 1.0, 11, 1)
    counts = np.bincount(d.tokens[:, 0], minlength=V)
    p = softmax(y.astype(np.float32).astype(np.float64))
    assert stats.chisquare(counts, n * p).pvalue > 1e-4


def test_temperature_scales_the_law():
    V = 6
    y = np.array([0.5, 1.0, -0.5, 2.0, 0.0, 1.5], dtype=np.float32)
    U = torch.tensor(y)[None, None, :].repeat(1, 2, 1)
    W = torch.zeros((V, 2))
    n = 20000
    T = 0.5
    d = oracle.draft_markov(U.repeat(n, 1, 1), W, W, np.zeros(n, dtype=np.int32), np.arange(n), T, 5, 1)
    counts = np.bincount(d.tokens[:, 0], minlength=V)
    p = softmax(y.astype(np.float64) / T)
    assert stats.chisquare(counts, n * p).pvalue > 1e-4
    assert np.allclose(d.lse[:, 0], logsumexp(y.astype(np.float64) / T), atol=1e-12)


def test_sequential_joint_law_exact_enumeration():
    """q(x1..x3) = prod_k softmax(U_k + B(x_{k-1}))[x_k], bias in the one-hot form."""
    V, gamma = 4, 3
    U, W1, W2, anchor = _tiny_inputs(V=V, gamma=gamma, B=1, seed=3, w_std=1.2)
    Ud = U.double().numpy()[0]
    A = W1.double().numpy().T
    Bm = W2.double().numpy()

    def cond(k, prev):
        e = np.zeros(V)
        e[prev] = 1.0
        return softmax(Ud[k - 1] + Bm @ (A @ e))

    probs = np.zeros((V,) * gamma)
    a0 = int(anchor[0])
    for x1 in range(V):
        for x2 in range(V):
            for x3 in range(V):
                probs[x1, x2, x3] = cond(1, a0)[x1] * cond(2, x1)[x2] * cond(3, x2)[x3]
    assert abs(probs.sum() - 1) < 1e-12
    n = 40000
    d = oracle.draft_markov(U.repeat(n, 1, 1), W1, W2, np.full(n, a0), np.arange(n), 1.0, 99, gamma)
    idx = d.tokens[:, 0] * V * V + d.tokens[:, 1] * V + d.tokens[:, 2]
    counts = np.bincount(idx, minlength=V ** gamma)
    expected = n * probs.reshape(-1)
    keep = expected > 5
    obs = counts[keep].astype(float)
    exp_ = expected[keep]
    obs = np.append(obs, counts[~keep].sum())
    exp_ = np.append(exp_, expected[~keep].sum())
    assert stats.chisquare(obs, exp_ * obs.sum() / exp_.sum()).pvalue > 1e-4
    # the draft reports y at its token and the log-normaliser of the position
    for i in range(50):
        x1, x2 = d.tokens[i, 0], d.tokens[i, 1]
        e = np.zeros(V)
        e[x1] = 1
        z2 = Ud[1] + Bm @ (A @ e)
        assert abs(d.ytok[i, 1] - z2[x2]) < 1e-12
        assert abs(d.lse[i, 1] - logsumexp(z2)) < 1e-12


def test_low_temperature_limit_is_greedy():
    wl = synth.WORKLOADS["tiny"].with_(B=4, V=500)
    inp = synth.make_inputs(wl)
    g = oracle.draft_markov(inp["U"], inp["W1"], inp["W2"], inp["anchor"], inp["req_ids"], 0.0, 1, 7)
    s = oracle.draft_markov(inp["U"], inp["W1"], inp["W2"], inp["anchor"], inp["req_ids"], 1e-5, 1, 7)
    # gaps above 1e-3 become >100 at T = 1e-5, beyond any Gumbel difference (< 40)
    assert np.min(g.margin) > 1e-3
    assert np.array_equal(g.tokens, s.tokens)


def test_margin_is_top2_gap():
    U, W1, W2, anchor = _tiny_inputs(V=30, gamma=2, B=2, seed=8)
    d = oracle.draft_markov(U, W1, W2, anchor, [0, 1], 0.0, 0, 2, keep_logits=True)
    for b in range(2):
        for k in range(2):
            srt = np.sort(d.z[b, k])
            assert abs(d.margin[b, k] - (srt[-1] - srt[-2])) < 1e-12
