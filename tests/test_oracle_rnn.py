"""Pins of the oracle's GRU (RNN) head draft (CPU only).

Tied to: torch.nn.GRUCell in float64 (an independent implementation of the
textbook cell), closed forms of the cell, W2 = 0 reducing to the independent
parallel draft, the sequential joint law by exact enumeration with states
from torch's cell, the dependence of a position's bias on every earlier
token, and the lossless verify law with the GRU draft (Monte-Carlo chi-square).
"""
import itertools

import numpy as np
import pytest
import torch
from scipy import stats
from scipy.special import softmax

import oracle
import synth


def _gru(r, std, seed, dtype=torch.float64):
    g = torch.Generator().manual_seed(seed)
    return dict(W_ih=torch.randn((3 * r, r), generator=g, dtype=dtype) * std,
                W_hh=torch.randn((3 * r, r), generator=g, dtype=dtype) * std,
                b_ih=torch.randn((3 * r,), generator=g, dtype=dtype) * std,
                b_hh=torch.randn((3 * r,), generator=g, dtype=dtype) * std,
                s0=torch.randn((r,), generator=g, dtype=dtype) * std)


def _torch_cell(p):
    r = p["s0"].shape[0]
    cell = torch.nn.GRUCell(r, r).double()
    with torch.no_grad():
        cell.weight_ih.copy_(p["W_ih"])
        cell.weight_hh.copy_(p["W_hh"])
        cell.bias_ih.copy_(p["b_ih"])
        cell.bias_hh.copy_(p["b_hh"])
    return cell


def test_cell_matches_library_gru():
    p = _gru(24, 0.4, 1)
    cell = _torch_cell(p)
    rs = np.random.default_rng(2)
    x = rs.normal(size=(9, 24))
    s = rs.normal(size=(9, 24))
    got = oracle.gru_cell(x, s, *(p[k].numpy() for k in ("W_ih", "W_hh", "b_ih", "b_hh")))
    with torch.no_grad():
        want = cell(torch.tensor(x), torch.tensor(s)).numpy()
    assert np.max(np.abs(got - want)) < 1e-13


def test_cell_closed_forms():
    r = 5
    Z = np.zeros((3 * r, r))
    zb = np.zeros(3 * r)
    s = np.linspace(-1, 1, r)[None]
    # no weights, no biases: both gates 1/2, candidate tanh(0) = 0 -> s' = s / 2
    assert np.allclose(oracle.gru_cell(np.ones((1, r)), s, Z, Z, zb, zb), 0.5 * s, atol=1e-15)
    # update gate saturated open (large z bias): the state is kept
    b = zb.copy()
    b[r:2 * r] = 50.0
    assert np.allclose(oracle.gru_cell(np.ones((1, r)), s, Z, Z, b, zb), s, atol=1e-15)
    # update gate shut, reset gate shut: s' = tanh(W_in x + b_in)
    b = zb.copy()
    b[:r] = -50.0
    b[r:2 * r] = -50.0
    W = np.zeros((3 * r, r))
    W[2 * r:] = np.eye(r) * 0.3
    x = np.arange(r, dtype=float)[None] / r
    want = np.tanh(0.3 * x)
    assert np.allclose(oracle.gru_cell(x, s, W, Z, b, zb), want, atol=1e-15)


def test_zero_projection_is_the_parallel_draft():
    wl = synth.WORKLOADS["rnn_tiny"]
    inp = synth.make_inputs(wl)
    W0 = torch.zeros_like(inp["W2"])
    d_rnn = oracle.draft_rnn(inp["U"], inp["W1"], W0, inp["gru"], inp["req_ids"], 1.0, 7, wl.gamma)
    d_par = oracle.draft_markov(inp["U"], W0, W0, inp["anchor"], inp["req_ids"], 1.0, 7, wl.gamma)
    assert np.array_equal(d_rnn.tokens, d_par.tokens)
    assert np.allclose(d_rnn.lse, d_par.lse, atol=1e-12)


def test_states_start_at_s0_and_follow_the_cell():
    wl = synth.WORKLOADS["rnn_tiny"]
    inp = synth.make_inputs(wl)
    d = oracle.draft_rnn(inp["U"], inp["W1"], inp["W2"], inp["gru"], inp["req_ids"], 1.0, 3, wl.gamma)
    s0 = inp["gru"]["s0"].double().numpy()
    assert np.allclose(d.states[:, 0, :], s0[None], atol=0)
    cell = _torch_cell({k: v.double() for k, v in inp["gru"].items()})
    W1 = inp["W1"].double()
    s = torch.tensor(d.states[:, 0, :])
    with torch.no_grad():
        for k in range(1, wl.gamma):
            s = cell(W1[torch.tensor(d.tokens[:, k - 1])], s)
            assert np.max(np.abs(s.numpy() - d.states[:, k, :])) < 1e-12


def test_bias_depends_on_every_earlier_token():
    """Unlike the Markov head, position 3's bias changes with x_1 at fixed x_2."""
    p = _gru(6, 0.8, 3)
    cell = _torch_cell(p)
    W1 = torch.randn((10, 6), generator=torch.Generator().manual_seed(4), dtype=torch.float64)
    with torch.no_grad():
        def state_after(x1, x2):
            s = p["s0"][None]
            s = cell(W1[[x1]], s)
            return cell(W1[[x2]], s)
        a = state_after(1, 5)
        b = state_after(2, 5)
    assert torch.max(torch.abs(a - b)) > 1e-3


def test_sequential_joint_law_exact_enumeration():
    """q(x1..x3) = prod_k softmax(U_k + s_{k-1}(x_<k) . W2)[x_k], states from torch's cell."""
    V, r, gamma = 4, 3, 3
    g = torch.Generator().manual_seed(11)
    U = torch.randn((1, gamma + 1, V), generator=g)
    W1 = torch.randn((V, r), generator=g) * 1.1
    W2 = torch.randn((V, r), generator=g) * 1.1
    p = _gru(r, 0.9, 12)
    cell = _torch_cell(p)
    Ud = U.double().numpy()[0]
    W2d = W2.double().numpy()

    def law(prefix):
        s = p["s0"][None]
        with torch.no_grad():
            for x in prefix:
                s = cell(W1.double()[[x]], s)
        k = len(prefix)
        return softmax(Ud[k] + W2d @ s[0].numpy())

    probs = np.zeros((V,) * gamma)
    for xs in itertools.product(range(V), repeat=gamma):
        q = 1.0
        for k in range(gamma):
            q *= law(xs[:k])[xs[k]]
        probs[xs] = q
    assert abs(probs.sum() - 1) < 1e-12
    n = 30000
    d = oracle.draft_rnn(U.repeat(n, 1, 1), W1, W2, {k: v.double() for k, v in p.items()},
                         np.arange(n), 1.0, 99, gamma)
    idx = d.tokens[:, 0] * V * V + d.tokens[:, 1] * V + d.tokens[:, 2]
    counts = np.bincount(idx, minlength=V ** gamma)
    expected = n * probs.reshape(-1)
    keep = expected > 5
    obs = np.append(counts[keep].astype(float), counts[~keep].sum())
    exp_ = np.append(expected[keep], expected[~keep].sum())
    assert stats.chisquare(obs, exp_ * obs.sum() / exp_.sum()).pvalue > 1e-4


@pytest.mark.parametrize("T", [1.0, 0.8])
def test_lossless_law_with_gru_draft(T):
    """Draft with the GRU head, verify with its states: the emitted sequence (padded with
    independent target draws) follows prod p_t ([blog] formal definition)."""
    V, r, gamma, n = 3, 2, 2, 30000
    g = torch.Generator().manual_seed(21)
    U = torch.randn((1, gamma + 1, V), generator=g)
    tgt = torch.randn((1, gamma + 1, V), generator=g)
    W1 = torch.randn((V, r), generator=g)
    W2 = torch.randn((V, r), generator=g)
    p = {k: v.double() for k, v in _gru(r, 0.8, 22).items()}
    Ur, tr = U.repeat(n, 1, 1), tgt.repeat(n, 1, 1)
    req = np.arange(n)
    d = oracle.draft_rnn(Ur, W1, W2, p, req, T, 2024, gamma)
    v = oracle.verify(tr, d.tokens, d.lse, d.ytok, Ur, W1, W2, None, None, req, T, 2024, gamma,
                      states=d.states)
    pt = [softmax(tgt[0, j].double().numpy() / T) for j in range(gamma + 1)]
    rs = np.random.default_rng(7)
    seqs = np.zeros((n, gamma + 1), dtype=int)
    for i in range(n):
        m = int(v.accept_len[i]) + 1
        seqs[i, :m] = v.out_tokens[i, :m]
        for j in range(m, gamma + 1):
            seqs[i, j] = rs.choice(V, p=pt[j])
    idx = seqs[:, 0] * V * V + seqs[:, 1] * V + seqs[:, 2]
    counts = np.bincount(idx, minlength=V ** 3)
    expect = n * np.einsum("i,j,k->ijk", *pt).reshape(-1)
    assert stats.chisquare(counts, expect).pvalue > 1e-4
    assert np.any(v.resid_row > 0) and np.any(v.accept_len == gamma)
