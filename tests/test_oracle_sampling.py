"""Pins of the oracle's categorical draw (two-level exponential race).

Tied to: the law of each draw (chi-square against w / sum w, including a
ragged last group and zero weights), the textbook Gumbel-max trick it reduces
to when every group holds one nonzero weight, and invariances of the
definition (scale of the weights, zero weights never drawn).
"""
import numpy as np
import pytest
from scipy import stats

import oracle

KEYS = [oracle.row_key(77, r, 1, oracle.DRAFT) for r in range(20000)]


def _draws(logw, keys=KEYS):
    return np.array([oracle.race_draw(logw, k)[0] for k in keys])


@pytest.mark.parametrize("w", [
    [0.05, 0.3, 0.1, 0.55, 2.0, 0.01, 0.7, 1.2],                 # two groups, unequal masses
    [1.0, 2.0, 3.0, 0.5, 0.25, 4.0, 1.5],                        # ragged last group of 3
    [0.0, 1.0, 0.0, 0.0, 3.0, 0.0, 2.0, 0.5, 0.0, 0.0, 0.0, 0.0, 1.0],   # zeros, an empty group
    [5.0, 1.0, 1.0],                                             # a single (short) group
])
def test_race_draws_follow_the_weights(w):
    w = np.asarray(w, dtype=np.float64)
    with np.errstate(divide="ignore"):
        x = _draws(np.log(w))
    counts = np.bincount(x, minlength=w.size)
    assert np.all(counts[w == 0] == 0)
    p = w / w.sum()
    keep = p > 0
    assert stats.chisquare(counts[keep], len(x) * p[keep]).pvalue > 1e-4


def test_choice_inside_a_group_is_independent_of_the_race():
    # group masses 1 : 3, members strongly unequal; the joint law must factor
    w = np.array([0.9, 0.05, 0.05, 0.0, 0.1, 0.2, 0.3, 2.4])
    x = _draws(np.log(np.where(w > 0, w, 1e-300)))
    counts = np.bincount(x, minlength=8)[[0, 1, 2, 4, 5, 6, 7]]
    p = w[[0, 1, 2, 4, 5, 6, 7]] / w.sum()
    assert stats.chisquare(counts, len(x) * p).pvalue > 1e-4


def test_one_member_per_group_is_gumbel_max():
    """With one nonzero weight per group the race key is ln w_v - ln(-ln a_g):
    the textbook Gumbel-max draw with the Gumbel of the group's element 4g."""
    rs = np.random.default_rng(3)
    V = 64
    lw = np.full(V, -np.inf)
    pos = 4 * np.arange(V // 4) + rs.integers(0, 4, V // 4)
    lw[pos] = rs.normal(size=V // 4)
    for key in KEYS[:300]:
        u = oracle.uniforms(key, V)
        gumbel = -np.log(-np.log(u[0::4]))
        expect = pos[int(np.argmax(lw[pos] + gumbel))]
        assert oracle.race_draw(lw, key)[0] == expect


def test_scale_of_the_weights_does_not_matter():
    rs = np.random.default_rng(5)
    lw = rs.normal(size=40) * 3
    same = 0
    for key in KEYS[:500]:
        a, m = oracle.race_draw(lw, key)
        b, _ = oracle.race_draw(lw + 123.25, key)
        if m > 1e-9:
            assert a == b
            same += 1
    assert same > 490


def test_single_nonzero_weight_is_always_drawn():
    lw = np.full(37, -np.inf)
    lw[22] = 0.3
    assert all(oracle.race_draw(lw, k)[0] == 22 for k in KEYS[:200])


def test_margin_bounds_the_decision():
    # a draw whose margin is large is stable under a perturbation smaller than it
    rs = np.random.default_rng(9)
    lw = rs.normal(size=24)
    for key in KEYS[:300]:
        v, m = oracle.race_draw(lw, key)
        assert m >= 0
        if m > 1e-3:
            assert oracle.race_draw(lw + rs.uniform(-1e-6, 1e-6, size=24), key)[0] == v
