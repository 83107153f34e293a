"""Pins of the oracle's confidence head, STS and survival products (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden", "confidence_tiny.json")


def _fixture():
    g = json.load(open(GOLD))
    h = torch.tensor(g["h"], dtype=torch.bfloat16)[None]
    E = torch.tensor(g["E"], dtype=torch.bfloat16)
    wc = torch.tensor(g["wc"], dtype=torch.bfloat16)
    return g, h, E, wc


def test_hand_worked_fixture():
    g, h, E, wc = _fixture()
    c = oracle.confidence(h, E, [g["anchor"]], [g["tokens"]], wc, g["bc"], None)
    assert np.array_equal(c.logit[0], np.asarray(g["logit"], dtype=np.float64))
    assert np.allclose(c.conf[0], g["conf"], rtol=1e-15, atol=0)
    assert np.allclose(c.surv[0], g["surv"], rtol=1e-15, atol=0)


def test_hand_worked_fixture_with_sts():
    g, h, E, wc = _fixture()
    T = torch.tensor(g["sts_T"], dtype=torch.float32)
    c = oracle.confidence(h, E, [g["anchor"]], [g["tokens"]], wc, g["bc"], T)
    assert np.allclose(c.conf[0], g["conf_sts"], rtol=1e-15, atol=0)
    assert np.allclose(c.surv[0], g["surv_sts"], rtol=1e-15, atol=0)


def _random_case(B=16, gamma=7, V=200, d=64, sts=False, seed=0):
    wl = synth.WORKLOADS["sample"].with_(B=B, gamma=gamma, V=V, d_h=d, d_e=d, sts=sts)
    inp = synth.make_inputs(wl, seed=seed)
    g = torch.Generator().manual_seed(seed + 1)
    tokens = torch.randint(0, V, (B, gamma), generator=g)
    return inp, tokens


def test_survival_non_increasing_and_in_unit_interval():
    inp, tok = _random_case(sts=True)
    c = oracle.confidence(inp["h"], inp["E"], inp["anchor"], tok, inp["wc"], inp["bc"], inp["sts_T"])
    assert np.all(c.conf > 0) and np.all(c.conf < 1)
    assert np.all(np.diff(c.surv, axis=1) <= 0)
    assert np.all(c.surv > 0) and np.all(c.surv <= 1)
    assert np.allclose(c.surv[:, 0], c.conf[:, 0], rtol=0, atol=0)


def test_sts_preserves_order_within_a_position():
    inp, tok = _random_case(B=64, sts=True)
    raw = oracle.confidence(inp["h"], inp["E"], inp["anchor"], tok, inp["wc"], inp["bc"], None)
    cal = oracle.confidence(inp["h"], inp["E"], inp["anchor"], tok, inp["wc"], inp["bc"], inp["sts_T"])
    for k in range(tok.shape[1]):
        assert np.array_equal(np.argsort(raw.conf[:, k], kind="stable"),
                              np.argsort(cal.conf[:, k], kind="stable"))
    # calibration with T >= 1 pulls every score towards 1/2
    assert np.all(np.abs(cal.conf - 0.5) <= np.abs(raw.conf - 0.5) + 1e-15)


def test_unit_temperatures_equal_no_sts():
    inp, tok = _random_case()
    a = oracle.confidence(inp["h"], inp["E"], inp["anchor"], tok, inp["wc"], inp["bc"], None)
    b = oracle.confidence(inp["h"], inp["E"], inp["anchor"], tok, inp["wc"], inp["bc"],
                          torch.ones(tok.shape[1]))
    assert np.array_equal(a.conf, b.conf)


def test_sigmoid_is_the_library_logistic():
    inp, tok = _random_case()
    c = oracle.confidence(inp["h"], inp["E"], inp["anchor"], tok, inp["wc"], inp["bc"], None)
    assert np.allclose(c.conf, expit(c.logit), rtol=1e-15, atol=1e-300)


def test_embedding_of_previous_token_is_used():
    # E zero except token 5: only positions whose previous token is 5 change
    B, gamma, V, d = 3, 4, 10, 8
    h = torch.zeros((B, gamma, d), dtype=torch.bfloat16)
    E = torch.zeros((V, d), dtype=torch.bfloat16)
    E[5] = 1.0
    wc = torch.cat([torch.zeros(d), torch.ones(d)]).to(torch.bfloat16)
    anchor = [5, 0, 1]
    tokens = [[1, 5, 2, 3], [5, 5, 1, 1], [2, 3, 4, 5]]
    c = oracle.confidence(h, E, anchor, tokens, wc, 0.0, None)
    expect = np.array([[8, 0, 8, 0], [0, 8, 8, 0], [0, 0, 0, 0]], dtype=np.float64)
    assert np.array_equal(c.logit, expect)
