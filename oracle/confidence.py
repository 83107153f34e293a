"""Confidence head, sequential temperature scaling and survival products.

[blog] "置信度头：预测自己的命运": for each draft position k a scalar
c_k = sigmoid(linear([h_k ; emb(x_{k-1})])) -- h_k the backbone hidden state at
k, emb the embedding of the token drafted at k-1 -- read as the probability that
position k is accepted given that positions before it were.  [summary] section 4
describes the same head (a light linear map of the draft hidden state and the
previous token's embedding followed by a sigmoid).

[blog] "校准问题：原始置信度不可靠" and [summary] section 4: sequential
temperature scaling rescales each position by its own temperature,
c'_k = sigmoid(logit(c_k) / T_k), which keeps the order of scores at a position.

[blog] "硬件感知前缀调度器" step 1, [teardown] "硬件感知前缀调度器", [summary]
section 4: the survival (prefix) probability a_j = prod_{i<=j} c_i.

Readings: the linear map is  l = w_h . h_k + w_e . E[x_{k-1}] + b  with w = [w_h; w_e]
one vector over the concatenation (the embedding table E and its width are
parameters; the blog reuses W1, the configs use a separate 4096-wide table);
with no STS vector every T_k = 1.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .markov import decode_weights, _ints


@dataclasses.dataclass
class ConfidenceResult:
    logit: np.ndarray   # float64 [B, gamma]: l_k before temperature
    conf: np.ndarray    # float64 [B, gamma]: c'_k
    surv: np.ndarray    # float64 [B, gamma]: a_k


def confidence(h, E, anchor, tokens, wc, bc: float, sts_T=None) -> ConfidenceResult:
    """h: [B][gamma][d_h] bf16; E: [V][d_e] bf16; tokens: [B][gamma]; wc: [d_h+d_e]."""
    hd = decode_weights(h)
    B, gamma, d_h = hd.shape
    wcd = decode_weights(wc)
    w_h, w_e = wcd[:d_h], wcd[d_h:]
    anc = _ints(anchor)
    tok = _ints(tokens)
    prev = np.concatenate([anc[:, None], tok[:, :gamma - 1]], axis=1)   # x_{k-1}
    Erows = decode_weights(E[prev.reshape(-1)]).reshape(B, gamma, -1)
    logit = hd @ w_h + Erows @ w_e + float(bc)
    if sts_T is None:
        T = np.ones(gamma)
    else:
        T = decode_weights(sts_T).reshape(gamma)
    conf = 1.0 / (1.0 + np.exp(-logit / T[None, :]))
    surv = np.cumprod(conf, axis=1)
    return ConfidenceResult(logit, conf, surv)
