"""Hardware-aware prefix scheduler: greedy admission with early stop.

[blog] "硬件感知前缀调度器" (algorithm steps 1-4): form every (request r,
length j) candidate with its survival a_{r,j}, sort them from high to low,
admit candidates one at a time while tracking the objective
Theta = tau(B) * SPS(B), and stop once Theta no longer increases.
[summary] section 4: the expected throughput is the expected number of accepted
tokens times the steps-per-second of the resulting verify batch, read from a
table profiled at start-up; the early stop is what keeps the rule lossless.
[summary] section 5: the table is step-shaped with efficiency cliffs, so the
early stop can end in a local optimum (expected behaviour, kept as is).

Readings:
  * tau = sum_b (1 + sum of admitted a_{b,j}) -- each request always yields one
    target token besides its accepted drafts; N = B + n tokens after admitting n
    candidates; Theta_n = (B + S_n) * SPS[N - 1], Theta_0 = B * SPS[B - 1];
  * admission stops at the first n with Theta_n <= Theta_{n-1}, or when N would
    exceed the table;
  * sort key (a descending, request ascending, position ascending), so the
    admitted set of each request is a prefix.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .markov import decode_weights


@dataclasses.dataclass
class ScheduleResult:
    K: np.ndarray          # int64 [B]
    n_selected: int
    theta: float           # Theta at the admitted set
    min_rel_step: float    # min |Theta_n - Theta_{n-1}| / Theta_{n-1} over decisions taken
    cut_gap: float         # a of last admitted minus a of first refused (inf if none)


def schedule(surv, sps) -> ScheduleResult:
    a = decode_weights(surv)
    s = decode_weights(sps).reshape(-1)
    B, gamma = a.shape
    n_sps = s.shape[0]
    if B < 1 or B > n_sps:
        raise ValueError("need 1 <= B <= n_sps")
    cands = [(float(a[b, j]), b, j) for b in range(B) for j in range(gamma)]
    cands.sort(key=lambda e: (-e[0], e[1], e[2]))
    K = np.zeros(B, dtype=np.int64)
    theta_prev = B * s[B - 1]
    S = 0.0
    n_sel = 0
    min_rel = np.inf
    cut_gap = np.inf
    for n, (av, b, j) in enumerate(cands, start=1):
        N = B + n
        if N > n_sps:
            break
        theta = (B + (S + av)) * s[N - 1]
        min_rel = min(min_rel, abs(theta - theta_prev) / theta_prev)
        if theta <= theta_prev:
            cut_gap = (cands[n - 2][0] - av) if n >= 2 else np.inf
            break
        S += av
        theta_prev = theta
        K[b] += 1
        n_sel = n
    return ScheduleResult(K, n_sel, float(theta_prev), float(min_rel), float(cut_gap))


def schedule_async(surv, surv_hist, sps) -> ScheduleResult:
    """Asynchronous variant: capacity from history, order from the current step.

    [blog] "硬件感知前缀调度器" (the asynchronous mechanism: the verify
    length is estimated from confidences of earlier steps so the decision
    does not block the pipeline) and [summary] section 5 (the production
    rule: the truncation count comes from confidences two steps old, the
    candidates are still ranked by the latest confidences, and with the
    count fixed from history the early-stop break is dropped in favour of an
    unconstrained global search over the jagged throughput table).

    Readings:
      * surv_hist has the shape of surv (the same request slots two steps
        earlier); Theta_n = (B + S_n^hist) * SPS[B + n - 1] with S_n^hist the
        sum of the n largest historical survivals; the count n* is the first
        n attaining the maximum over 0 <= n <= min(B * gamma, n_sps - B);
      * the admitted set is the top n* candidates of the current survivals,
        ranked (a descending, request ascending, position ascending) as in
        the synchronous rule, so each request's set is a prefix;
      * theta is Theta_{n*} (the historical objective); min_rel_step is the
        relative gap between the maximum and the best other n (how clear the
        argmax is); cut_gap is the current survival of the last admitted
        candidate minus that of the first refused one.
    """
    a = decode_weights(surv)
    h = decode_weights(surv_hist)
    s = decode_weights(sps).reshape(-1)
    B, gamma = a.shape
    n_sps = s.shape[0]
    if h.shape != a.shape:
        raise ValueError("surv_hist must have the shape of surv")
    if B < 1 or B > n_sps:
        raise ValueError("need 1 <= B <= n_sps")
    old = sorted((float(h[b, j]) for b in range(B) for j in range(gamma)), reverse=True)
    n_max = min(B * gamma, n_sps - B)
    thetas = [B * s[B - 1]]
    S = 0.0
    for n in range(1, n_max + 1):
        S += old[n - 1]
        thetas.append((B + S) * s[B + n - 1])
    n_star = int(np.argmax(thetas))          # first maximum
    best = float(thetas[n_star])
    others = [t for i, t in enumerate(thetas) if i != n_star]
    min_rel = (best - max(others)) / best if others else np.inf
    cands = [(float(a[b, j]), b, j) for b in range(B) for j in range(gamma)]
    cands.sort(key=lambda e: (-e[0], e[1], e[2]))
    K = np.zeros(B, dtype=np.int64)
    for av, b, j in cands[:n_star]:
        K[b] += 1
    if 0 < n_star < len(cands):
        cut_gap = cands[n_star - 1][0] - cands[n_star][0]
    else:
        cut_gap = np.inf
    return ScheduleResult(K, n_star, best, float(min_rel), float(cut_gap))
