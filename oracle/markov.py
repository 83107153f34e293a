"""Markov-head semi-autoregressive draft, float64.

Follows [blog] "形式化定义" / "整体架构" (draft distribution at position k is the
backbone logit U_k plus a transition bias B_k that depends on the token sampled
at k-1, so sampling runs position by position) and [blog] "Markov Head：一阶转移
偏置" (h_{k-1} = W1[x_{k-1}] in R^r; B_k(v) = h_{k-1} . W2[v], W2[v] the v-th
column of the r x |V| matrix W2).  [teardown] "DSpark 的解法" writes the same map
as Logits_adjusted = Logits_parallel + B (A e_{t-1}) with A in R^{r x V},
B in R^{V x r}; its one-hot form is used as an independent pin in the tests.

Readings:
  * the draft law is softmax((U_k + B_k) / T); T = 0 means argmax of U_k + B_k;
  * the bias is applied at every position, B_1 from the anchor token x_0;
  * a stochastic draw is the Gumbel-max draw of ``sampling.gumbel_draw`` on
    y = z / T (weights w_v = exp(y_v)) with the DRAFT stream of (req, k);
  * greedy ties go to the lowest vocabulary index;
  * in greedy mode the reported log-normaliser is that of z itself (T = 1).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

from .rng import DRAFT, row_key
from .sampling import gumbel_draw


def decode_weights(w) -> np.ndarray:
    """fp32 / bf16 tensor (or ndarray) -> float64 ndarray; bf16 -> fp64 is exact."""
    if isinstance(w, torch.Tensor):
        return w.detach().to("cpu", torch.float64).numpy()
    return np.asarray(w, dtype=np.float64)


def _ints(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.asarray(x).astype(np.int64)


def markov_bias(W1: np.ndarray, W2: np.ndarray, prev: np.ndarray) -> np.ndarray:
    """B(v) = sum_i W1[prev, i] * W2col_v[i] for each previous token; [n, V].

    ``W1`` is [V][r] (row = token's rank-r vector), ``W2`` the r x V matrix
    stored column-major, i.e. an array [V][r] whose row v is column v.
    """
    H = W1[prev]          # gather h_{k-1} = W1[x_{k-1}]
    return H @ W2.T       # project back to the vocabulary


def logsumexp_rows(y: np.ndarray) -> np.ndarray:
    m = y.max(axis=-1, keepdims=True)
    return (m + np.log(np.exp(y - m).sum(axis=-1, keepdims=True)))[..., 0]


def top2_margin(key: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """key[idx] minus the largest key at any other index, per row."""
    rows = np.arange(key.shape[0])
    best = key[rows, idx]
    k2 = key.copy()
    k2[rows, idx] = -np.inf
    return best - k2.max(axis=-1)


@dataclasses.dataclass
class DraftResult:
    tokens: np.ndarray    # int64 [B, gamma]
    lse: np.ndarray       # float64 [B, gamma]: L_d = ln sum_v exp(y_v)
    ytok: np.ndarray      # float64 [B, gamma]: y at the drafted token
    margin: np.ndarray    # float64 [B, gamma]: top-2 gap of the greedy or Gumbel-max keys
    z: Optional[np.ndarray] = None   # float64 [B, gamma, V] when kept
    states: Optional[np.ndarray] = None   # GRU head: float64 [B, gamma, r], the state position k projected


def draft_markov(U, W1, W2, anchor, req_ids, temperature: float, seed: int, gamma: int,
                 keep_logits: bool = False) -> DraftResult:
    """Sample gamma draft tokens per request, position by position.

    U: [B][>=gamma][V] float32 (row k-1 = position k); W1, W2: [V][r];
    anchor, req_ids: [B].  Returns tokens, the draft log-normaliser and the
    (tempered) logit of each drafted token.
    """
    W1d = decode_weights(W1)
    W2d = decode_weights(W2)
    anc = _ints(anchor)
    req = _ints(req_ids) & 0xFFFFFFFF
    B = anc.shape[0]
    V = W1d.shape[0]
    T = float(temperature)
    tokens = np.zeros((B, gamma), dtype=np.int64)
    lse = np.zeros((B, gamma))
    ytok = np.zeros((B, gamma))
    margin = np.zeros((B, gamma))
    zs = np.zeros((B, gamma, V)) if keep_logits else None
    prev = anc.copy()
    for k in range(1, gamma + 1):
        Uk = U[:, k - 1, :]
        Uk = Uk.detach().to(torch.float64).numpy() if isinstance(Uk, torch.Tensor) \
            else np.asarray(Uk, dtype=np.float64)
        z = Uk + markov_bias(W1d, W2d, prev)
        y = z / T if T > 0 else z
        if T > 0:
            for b in range(B):
                x_b, m_b = gumbel_draw(y[b], row_key(seed, int(req[b]), k, DRAFT))
                tokens[b, k - 1] = x_b
                margin[b, k - 1] = m_b
            x = tokens[:, k - 1].copy()
        else:
            x = np.argmax(z, axis=-1)          # first maximum = lowest index on ties
            tokens[:, k - 1] = x
            margin[:, k - 1] = top2_margin(z, x)
        lse[:, k - 1] = logsumexp_rows(y)
        ytok[:, k - 1] = y[np.arange(B), x]
        if keep_logits:
            zs[:, k - 1, :] = z
        prev = x
    return DraftResult(tokens, lse, ytok, margin, zs)
