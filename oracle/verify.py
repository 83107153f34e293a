"""Lossless speculative accept/reject with residual resampling and bonus token.

[blog] "形式化定义": the target scores all drafted positions in one pass, the
positions are checked in order, everything after the first rejected position
is dropped and the target samples one compensation token there, so that the
output law is exactly the target's.  [summary] sections 1 and 4 state the same
lossless guarantee (accepted tokens are those the target would produce; a
rejected one is replaced by the target's own choice).

The accept/residual formulas are stripped from the pages; this follows the
standard lossless rule they describe (readings):
  * accept x_k iff u < p_t(x_k) / p_d(x_k) with u the ACCEPT uniform of (req, k);
  * at the first rejection draw from norm(max(0, p_t - p_d)) with the RESID
    stream (empty residual: draw from p_t with that stream);
  * if all K_b drafts are accepted, draw the bonus from target row K_b + 1
    with the BONUS stream;
  * every draw is the Gumbel-max draw of ``sampling.gumbel_draw``;
  * greedy (T = 0): accept iff x_k equals the lowest-index argmax of the
    target row; the compensation / bonus token is that argmax;
  * p_t = softmax(target / T), p_d = softmax((U + bias) / T), same T.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

from .markov import decode_weights, markov_bias, logsumexp_rows, _ints
from .rng import ACCEPT, RESID, BONUS, row_key, uniform_at
from .sampling import gumbel_draw


def _row(x, b, k) -> np.ndarray:
    r = x[b, k]
    if isinstance(r, torch.Tensor):
        return r.detach().to(torch.float64).numpy()
    return np.asarray(r, dtype=np.float64)


def target_logprobs(t_row: np.ndarray, T: float) -> np.ndarray:
    """ln p_t(v) = t_v / T - ln sum_w exp(t_w / T)."""
    tt = t_row / T
    return tt - logsumexp_rows(tt[None])[0]


def accept_ratio(log_pt_x: float, log_pd_x: float) -> float:
    """rho = p_t(x) / p_d(x); the draft x is kept iff u < rho."""
    return float(np.exp(log_pt_x - log_pd_x))


def residual_weights(log_pt: np.ndarray, log_pd: np.ndarray) -> np.ndarray:
    """Unnormalised residual law r_v = max(0, p_t(v) - p_d(v))."""
    return np.maximum(0.0, np.exp(log_pt) - np.exp(log_pd))


def _top2(key: np.ndarray, i: int) -> float:
    k2 = key.copy()
    k2[i] = -np.inf
    return float(key[i] - k2.max()) if k2.size > 1 else np.inf


@dataclasses.dataclass
class VerifyResult:
    accept_len: np.ndarray   # int64 [B]
    out_tokens: np.ndarray   # int64 [B, gamma+1], -1 after the emitted tokens
    margin: np.ndarray       # float64 [B, gamma]: margin of the accept decision at row k
    final_margin: np.ndarray  # float64 [B]: margin of the decision that chose the last token
    lse_t: np.ndarray        # float64 [B, gamma+1]: target log-normaliser per examined row
    resid_row: np.ndarray    # int64 [B]: 1-based row of the residual draw, 0 if none


def verify(target, tokens, lse_d, ytok, U, W1, W2, anchor, K, req_ids,
           temperature: float, seed: int, gamma: int, states=None) -> VerifyResult:
    """``states`` (GRU head, [B][gamma][r]): the residual's draft row uses the
    bias states[b, k-1] . W2 instead of the Markov bias W1[x_{k-1}] . W2."""
    tok = _ints(tokens)
    anc = _ints(anchor) if anchor is not None else None
    req = _ints(req_ids) & 0xFFFFFFFF
    lse_d = np.asarray(lse_d, dtype=np.float64)
    ytok = np.asarray(ytok, dtype=np.float64)
    B = tok.shape[0]
    Ks = np.full(B, gamma, dtype=np.int64) if K is None else _ints(K)
    T = float(temperature)
    greedy = T <= 0
    W1d = W2d = None
    acc = np.zeros(B, dtype=np.int64)
    out = np.full((B, gamma + 1), -1, dtype=np.int64)
    margin = np.full((B, gamma), np.inf)
    final_margin = np.full(B, np.inf)
    lse_t = np.full((B, gamma + 1), np.nan)
    resid_row = np.zeros(B, dtype=np.int64)
    for b in range(B):
        r_id = int(req[b])
        Kb = int(Ks[b])
        A = 0
        done = False
        for k in range(1, Kb + 1):
            t = _row(target, b, k - 1)
            x = int(tok[b, k - 1])
            if greedy:
                star = int(np.argmax(t))
                margin[b, k - 1] = _top2(t, star)
                lse_t[b, k - 1] = logsumexp_rows(t[None])[0]
                if x == star:
                    out[b, A] = x
                    A += 1
                    continue
                out[b, A] = star
                final_margin[b] = margin[b, k - 1]
                done = True
                break
            lpt = target_logprobs(t, T)
            lse_t[b, k - 1] = t[0] / T - lpt[0]
            rho = accept_ratio(lpt[x], ytok[b, k - 1] - lse_d[b, k - 1])
            u = uniform_at(row_key(seed, r_id, k, ACCEPT), 0)
            margin[b, k - 1] = abs(u - rho)
            if u < rho:
                out[b, A] = x
                A += 1
                continue
            # first rejection: residual draw from norm(max(0, p_t - p_d))
            if W2d is None:
                W1d = decode_weights(W1) if states is None else None
                W2d = decode_weights(W2)
            if states is None:
                prev = int(anc[b]) if k == 1 else int(tok[b, k - 2])
                bias = markov_bias(W1d, W2d, np.array([prev]))[0]
            else:
                bias = W2d @ np.asarray(states[b, k - 1], dtype=np.float64)
            z = _row(U, b, k - 1) + bias
            resid = residual_weights(lpt, z / T - lse_d[b, k - 1])
            rkey = row_key(seed, r_id, k, RESID)
            if np.any(resid > 0):
                with np.errstate(divide="ignore"):
                    xr, final_margin[b] = gumbel_draw(np.log(resid), rkey)
            else:
                xr, final_margin[b] = gumbel_draw(t / T, rkey)
            out[b, A] = xr
            resid_row[b] = k
            done = True
            break
        if not done:
            t = _row(target, b, Kb)   # row K_b + 1
            if greedy:
                star = int(np.argmax(t))
                final_margin[b] = _top2(t, star)
                lse_t[b, Kb] = logsumexp_rows(t[None])[0]
            else:
                star, final_margin[b] = gumbel_draw(t / T, row_key(seed, r_id, Kb + 1, BONUS))
                lse_t[b, Kb] = logsumexp_rows((t / T)[None])[0]
            out[b, A] = star
        acc[b] = A
    return VerifyResult(acc, out, margin, final_margin, lse_t, resid_row)


def accept_prob(target, tokens, lse_d, U, W1, W2, anchor, temperature: float, gamma: int,
                states=None) -> np.ndarray:
    """Per-position acceptance probability alpha[b, k-1] = sum_v min(p_d(v), p_t(v)).

    [summary] section 4 (the confidence head is trained toward the true
    acceptance rate, the total-variation distance between the draft and the
    target distributions) and [blog] "置信度头" (c_k targets P(accept k | all
    before accepted)): with the lossless rule, position k is kept with
    probability sum_v min(p_d, p_t) = 1 - TV(p_d, p_t) given its prefix.
    p_d is rebuilt from U and the bias of the given head (Markov: W1 of the
    previous drafted token, anchor at k = 1; GRU: ``states``); lse_d is the
    draft log-normaliser the draft returned.  Sampling temperatures only.
    """
    tok = _ints(tokens)
    anc = _ints(anchor) if anchor is not None else None
    lse_d = np.asarray(lse_d, dtype=np.float64)
    B = tok.shape[0]
    T = float(temperature)
    W1d = decode_weights(W1) if states is None else None
    W2d = decode_weights(W2)
    out = np.zeros((B, gamma))
    for b in range(B):
        for k in range(1, gamma + 1):
            if states is None:
                prev = int(anc[b]) if k == 1 else int(tok[b, k - 2])
                bias = markov_bias(W1d, W2d, np.array([prev]))[0]
            else:
                bias = W2d @ np.asarray(states[b, k - 1], dtype=np.float64)
            z = _row(U, b, k - 1) + bias
            lpd = z / T - lse_d[b, k - 1]
            lpt = target_logprobs(_row(target, b, k - 1), T)
            out[b, k - 1] = np.minimum(np.exp(lpd), np.exp(lpt)).sum()
    return out
