"""RNN (GRU) head semi-autoregressive draft, float64 (test oracle).

[blog] "RNN Head：长程依赖": instead of the previous token alone, the sequential
head keeps a GRU-style recurrent state s_k that starts from a learned vector
s_0 and absorbs every token sampled so far in the block; the bias B_k is that
state projected onto the vocabulary.  [summary] section 3 describes the same
alternative (a state vector compressing the whole draft prefix).  The pages
strip the update formula.

Readings:
  * the cell is the textbook GRU (Cho et al., 2014) in the gate order and
    bias placement of the common deep-learning libraries:
        r  = sigmoid(W_ir x + b_ir + W_hr s + b_hr)
        z  = sigmoid(W_iz x + b_iz + W_hz s + b_hz)
        n  = tanh(W_in x + b_in + r * (W_hn s + b_hn))
        s' = (1 - z) * n + z * s
    with W_ih = [W_ir; W_iz; W_in], W_hh likewise, state width r;
  * the cell's input is the sampled token's row W1[x_k] (the Markov head's
    token -> rank-r map), so s_k = GRU(s_{k-1}, W1[x_k]);
  * the bias at position k is B_k = s_{k-1} . W2 (W2 the r x V projection),
    so B_1 = s_0 . W2 for every request; the anchor token does not enter;
  * the state is carried at full precision; everything else (draft law,
    draws, greedy) is as for the Markov head.
"""
from __future__ import annotations

import numpy as np
import torch

from .markov import decode_weights, logsumexp_rows, top2_margin, _ints, DraftResult
from .rng import DRAFT, row_key
from .sampling import gumbel_draw


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def gru_cell(x: np.ndarray, s: np.ndarray, W_ih, W_hh, b_ih, b_hh) -> np.ndarray:
    """One GRU update for a batch: x [n, r_in], s [n, r] -> s' [n, r], float64."""
    r = s.shape[-1]
    gi = x @ W_ih.T + b_ih          # [n, 3r]: input contributions of the three gates
    gh = s @ W_hh.T + b_hh          # [n, 3r]: state contributions
    reset = _sigmoid(gi[:, :r] + gh[:, :r])
    update = _sigmoid(gi[:, r:2 * r] + gh[:, r:2 * r])
    new = np.tanh(gi[:, 2 * r:] + reset * gh[:, 2 * r:])
    return (1.0 - update) * new + update * s


def draft_rnn(U, W1, W2, gru: dict, req_ids, temperature: float, seed: int, gamma: int,
              keep_logits: bool = False) -> DraftResult:
    """Sample gamma draft tokens per request with the GRU head.

    U: [B][>=gamma][V]; W1, W2: [V][r]; gru: W_ih, W_hh [3r][r], b_ih, b_hh [3r],
    s0 [r].  Returns the tokens, log-normalisers, tempered logits at the tokens
    and (``states``) the state s_{k-1} that position k projected.
    """
    W1d = decode_weights(W1)
    W2d = decode_weights(W2)
    W_ih, W_hh = decode_weights(gru["W_ih"]), decode_weights(gru["W_hh"])
    b_ih, b_hh = decode_weights(gru["b_ih"]), decode_weights(gru["b_hh"])
    s0 = decode_weights(gru["s0"])
    req = _ints(req_ids) & 0xFFFFFFFF
    B = req.shape[0]
    V, r = W2d.shape
    T = float(temperature)
    tokens = np.zeros((B, gamma), dtype=np.int64)
    lse = np.zeros((B, gamma))
    ytok = np.zeros((B, gamma))
    margin = np.zeros((B, gamma))
    states = np.zeros((B, gamma, r))
    zs = np.zeros((B, gamma, V)) if keep_logits else None
    s = np.tile(s0, (B, 1))
    for k in range(1, gamma + 1):
        Uk = U[:, k - 1, :]
        Uk = Uk.detach().to(torch.float64).numpy() if isinstance(Uk, torch.Tensor) \
            else np.asarray(Uk, dtype=np.float64)
        states[:, k - 1, :] = s
        z = Uk + s @ W2d.T                      # B_k = s_{k-1} . W2
        y = z / T if T > 0 else z
        if T > 0:
            for b in range(B):
                x_b, m_b = gumbel_draw(y[b], row_key(seed, int(req[b]), k, DRAFT))
                tokens[b, k - 1] = x_b
                margin[b, k - 1] = m_b
            x = tokens[:, k - 1].copy()
        else:
            x = np.argmax(z, axis=-1)
            tokens[:, k - 1] = x
            margin[:, k - 1] = top2_margin(z, x)
        lse[:, k - 1] = logsumexp_rows(y)
        ytok[:, k - 1] = y[np.arange(B), x]
        if keep_logits:
            zs[:, k - 1, :] = z
        s = gru_cell(W1d[x], s, W_ih, W_hh, b_ih, b_hh)
    return DraftResult(tokens, lse, ytok, margin, zs, states)
