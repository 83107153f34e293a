"""Pins of the oracle's categorical draw (per-entry Gumbel-max).

Tied to things other than the draw's own formula: the law of each draw
(chi-square against w / sum w, with zero weights), the max-stability of the
Gumbel family (the winning key minus ln sum w is a standard Gumbel: mean the
Euler-Mascheroni constant, variance pi^2 / 6, Kolmogorov-Smirnov against
scipy's gumbel_r), independence of draws taken from different streams of one
request, and invariances of the definition.  Planted mistakes (a flipped
Gumbel sign, an exponential in place of the Gumbel, the minimum in place of
the maximum, one uniform shared by every entry) are put into the oracle on
the CPU and each must fail the law pin.
"""
import numpy as np
import pytest
from scipy import stats

import oracle
import oracle.sampling as sampling

KEYS = [oracle.row_key(77, r, 1, oracle.DRAFT) for r in range(20000)]

LAWS = [
    [0.05, 0.3, 0.1, 0.55, 2.0, 0.01, 0.7, 1.2],
    [1.0, 2.0, 3.0, 0.5, 0.25, 4.0, 1.5],
    [0.0, 1.0, 0.0, 0.0, 3.0, 0.0, 2.0, 0.5, 0.0, 0.0, 0.0, 0.0, 1.0],   # zero weights
    [5.0, 1.0, 1.0],
    [1.0, 3.0],                                                          # P(0) = 1/4 in closed form
]


def _draws(logw, keys=KEYS):
    return np.array([oracle.gumbel_draw(logw, k)[0] for k in keys])


def _law_pvalue(w, keys=KEYS):
    w = np.asarray(w, dtype=np.float64)
    with np.errstate(divide="ignore"):
        x = _draws(np.log(w), keys)
    counts = np.bincount(x, minlength=w.size)
    p = w / w.sum()
    keep = p > 0
    return counts, stats.chisquare(counts[keep], len(x) * p[keep]).pvalue


@pytest.mark.parametrize("w", LAWS)
def test_draws_follow_the_weights(w):
    counts, pv = _law_pvalue(w)
    assert np.all(counts[np.asarray(w) == 0] == 0)
    assert pv > 1e-4


def test_winning_key_is_a_standard_gumbel_about_the_log_mass():
    """max_v (ln w_v + g_v) ~ Gumbel(ln sum w, 1): the max-stability that makes
    the argmax a draw from w / sum w."""
    rs = np.random.default_rng(4)
    lw = rs.normal(size=40) * 1.5
    lse = np.log(np.exp(lw).sum())
    top = np.array([np.max(oracle.gumbel_keys(lw, k)) for k in KEYS[:8000]]) - lse
    assert abs(top.mean() - np.euler_gamma) < 5 * (np.pi / np.sqrt(6)) / np.sqrt(top.size)
    assert abs(top.var() - np.pi ** 2 / 6) < 0.12
    assert stats.kstest(top, stats.gumbel_r.cdf).pvalue > 1e-4


def test_draws_of_two_streams_are_independent():
    """The draft draw at position 1 and the bonus draw at position 1 of the same
    request come from different streams: their joint law factors."""
    w = np.array([1.0, 2.0, 0.5, 1.5])
    lw = np.log(w)
    a = np.array([oracle.gumbel_draw(lw, oracle.row_key(5, r, 1, oracle.DRAFT))[0] for r in range(12000)])
    b = np.array([oracle.gumbel_draw(lw, oracle.row_key(5, r, 1, oracle.BONUS))[0] for r in range(12000)])
    counts = np.bincount(a * 4 + b, minlength=16)
    p = w / w.sum()
    assert stats.chisquare(counts, len(a) * np.outer(p, p).reshape(-1)).pvalue > 1e-4


def test_scale_of_the_weights_does_not_matter():
    rs = np.random.default_rng(5)
    lw = rs.normal(size=40) * 3
    same = 0
    for key in KEYS[:500]:
        a, m = oracle.gumbel_draw(lw, key)
        b, _ = oracle.gumbel_draw(lw + 123.25, key)
        if m > 1e-9:
            assert a == b
            same += 1
    assert same > 490


def test_single_nonzero_weight_is_always_drawn():
    lw = np.full(37, -np.inf)
    lw[22] = 0.3
    assert all(oracle.gumbel_draw(lw, k)[0] == 22 for k in KEYS[:200])


def test_all_zero_weights_are_refused():
    with pytest.raises(ValueError):
        oracle.gumbel_draw(np.full(5, -np.inf), KEYS[0])


def test_equal_keys_go_to_the_lowest_index():
    # two entries of equal weight whose uniforms coincide (23-bit uniforms repeat
    # within a row of 2^15 entries): the lower index wins, with margin 0
    key = KEYS[0]
    n = 1 << 15
    u = oracle.uniforms(key, n)
    order = np.argsort(u, kind="stable")
    same = np.nonzero(u[order[1:]] == u[order[:-1]])[0]
    assert same.size > 0
    i, j = sorted((int(order[same[0]]), int(order[same[0] + 1])))
    lw = np.full(n, -np.inf)
    lw[i] = lw[j] = 0.0
    assert oracle.gumbel_draw(lw, key) == (i, 0.0)


def test_margin_bounds_the_decision():
    rs = np.random.default_rng(9)
    lw = rs.normal(size=24)
    for key in KEYS[:300]:
        v, m = oracle.gumbel_draw(lw, key)
        assert m >= 0
        if m > 1e-3:
            assert oracle.gumbel_draw(lw + rs.uniform(-1e-6, 1e-6, size=24), key)[0] == v


@pytest.mark.parametrize("mistake", ["flipped_sign", "exponential", "argmin", "shared_uniform"])
def test_planted_mistakes_fail_the_law_pin(monkeypatch, mistake):
    good = sampling.gumbels
    if mistake == "flipped_sign":
        monkeypatch.setattr(sampling, "gumbels", lambda key, n: -good(key, n))
    elif mistake == "exponential":
        monkeypatch.setattr(sampling, "gumbels", lambda key, n: -np.log(oracle.uniforms(key, n)))
    elif mistake == "argmin":
        keys = sampling.gumbel_keys
        monkeypatch.setattr(sampling, "gumbel_keys", lambda lw, key: -keys(lw, key))
    elif mistake == "shared_uniform":
        monkeypatch.setattr(sampling, "gumbels", lambda key, n: np.full(n, good(key, 1)[0]))
    try:
        _, pv = _law_pvalue([0.5, 2.0, 1.0, 3.0, 0.25], KEYS[:6000])
    finally:
        monkeypatch.undo()
    assert pv < 1e-6
