"""Categorical draws by a two-level exponential race, float64 (test oracle).

Every stochastic choice of the step -- the draft token at each position, the
residual token at the first rejection, the bonus token -- is a draw from a
law proportional to nonnegative weights w_v over the vocabulary.  The pages
fix no sampling procedure (only the laws); this is the oracle's reading,
chosen so that one uniform of the counter stream serves four entries:

  * the vocabulary is cut into aligned groups G_g = {4g, .., 4g+3} (the last
    one shorter when V is not a multiple of 4), with masses S_g = sum of w_v;
  * group g gets the exponential variate E_g = -ln a_g, a_g the uniform of
    element 4g of the row's stream; the group with the largest
    ln S_g - ln E_g wins (lowest g on ties) -- the exponential race, so
    P(g) = S_g / sum S (the minimum of E_g / S_g over independent
    exponentials falls on g with that probability);
  * inside the winner, the uniform c of element 4g+1 picks the first member
    i with c * S_g < w_{4g} + .. + w_{4g+i} (inverse CDF), so
    P(v | g) = w_v / S_g.

Together P(v) = w_v / sum w, the law asked for.  Zero weights are never
drawn.  The decision margin reported for parity is the smaller of the top-2
gap of the group keys and the distance of c from the nearest inner CDF
boundary (relative to S_g).
"""
from __future__ import annotations

import numpy as np

from .rng import uniforms

GROUP = 4


def group_keys(logw: np.ndarray, key: int):
    """Per-group log-mass, race key and the row's uniforms.

    logw: [V] float64 log-weights (-inf for a zero weight).  Returns
    (lse_g [G], race key [G], lw [G, 4] padded with -inf, u [4G]).
    """
    V = logw.shape[0]
    G = (V + GROUP - 1) // GROUP
    lw = np.full(G * GROUP, -np.inf)
    lw[:V] = logw
    lw = lw.reshape(G, GROUP)
    m = lw.max(axis=1)
    safe = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(divide="ignore"):
        lse = safe + np.log(np.exp(lw - safe[:, None]).sum(axis=1))
    lse = np.where(np.isfinite(m), lse, -np.inf)
    u = uniforms(key, G * GROUP)
    E = -np.log(u[0::GROUP])
    return lse, lse - np.log(E), lw, u


def race_draw(logw: np.ndarray, key: int) -> tuple[int, float]:
    """Draw v ~ w_v / sum w by the two-level race; returns (v, margin)."""
    lse, gk, lw, u = group_keys(logw, key)
    g = int(np.argmax(gk))                      # first maximum: lowest group on ties
    if not np.isfinite(gk[g]):
        raise ValueError("all weights are zero")
    rest = np.delete(gk, g)
    key_margin = float(gk[g] - rest.max()) if rest.size else np.inf
    w = np.exp(lw[g] - lse[g])                  # member weights relative to S_g
    C = np.cumsum(w)
    c = float(u[GROUP * g + 1])
    hits = np.nonzero(c < C)[0]
    i = int(hits[0]) if hits.size else int(np.nonzero(w > 0)[0][-1])
    n_real = min(GROUP, logw.shape[0] - GROUP * g)   # members of the group (last may be short)
    inner = C[: n_real - 1]
    choice_margin = float(np.min(np.abs(c - inner))) if inner.size else np.inf
    return GROUP * g + i, min(key_margin, choice_margin)
