"""Categorical draws by the Gumbel-max trick, float64 (test oracle).

Every stochastic choice of the step -- the draft token at each position, the
residual token at the first rejection, the bonus token -- is a draw from a
law proportional to nonnegative weights w_v over the vocabulary.  The pages
give the laws only ([blog] "形式化定义": the draft softmax, the normalised
residual at the first rejection, the target's law for the compensation
token), not a procedure.  The reading taken is the textbook Gumbel-max draw
(E. J. Gumbel 1954; e.g. Maddison, Tarlow & Minka, "A* Sampling", 2014):

    x = the lowest index v attaining  max_v ( ln w_v + g_v ),
    g_v = -ln(-ln u_v),  u_v the row's counter-based uniforms (rng.py).

Because the g_v are independent standard Gumbels, P(x = v) = w_v / sum w.
Zero weights (ln w = -inf) are never drawn.  The decision margin reported
for parity is the gap between the best key and the best key at any other
index: a perturbation of every key by less than half of it cannot change
the draw.
"""
from __future__ import annotations

import numpy as np

from .rng import gumbels


def gumbel_keys(logw: np.ndarray, key: int) -> np.ndarray:
    """Per-entry keys ln w_v + g_v of one row (-inf where w_v = 0)."""
    logw = np.asarray(logw, dtype=np.float64)
    return logw + gumbels(key, logw.shape[0])


def gumbel_draw(logw: np.ndarray, key: int) -> tuple[int, float]:
    """Draw v ~ w_v / sum w by Gumbel-max; returns (v, margin).

    logw: [V] float64 log-weights (-inf for a zero weight); key: the row's
    64-bit stream key.
    """
    keys = gumbel_keys(logw, key)
    v = int(np.argmax(keys))                 # first maximum: lowest index on ties
    if not np.isfinite(keys[v]):
        raise ValueError("all weights are zero")
    rest = np.delete(keys, v)
    margin = float(keys[v] - rest.max()) if rest.size else np.inf
    return v, margin
