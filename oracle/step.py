"""One whole step: draft -> confidence -> [schedule] -> verify, float64.

[blog] "整体架构" and "硬件感知前缀调度器", [summary] sections 3-4: the parallel
backbone's outputs (U_k, h_k) enter a sequential head that drafts gamma tokens,
the confidence head scores them, the scheduler picks each request's verify
length K_b, and the target's scores decide acceptance.  Without a scheduler
every request verifies all gamma positions.

``rows`` restricts the computation to a subset of requests (all steps but the
scheduler are independent per request); it is refused when a scheduler runs,
since the scheduler needs every request's survival values.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

from .markov import draft_markov, DraftResult
from .rnn import draft_rnn
from .confidence import confidence, ConfidenceResult
from .schedule import schedule, ScheduleResult
from .verify import verify, VerifyResult


@dataclasses.dataclass
class StepResult:
    rows: np.ndarray
    draft: DraftResult
    conf: Optional[ConfidenceResult]
    sched: Optional[ScheduleResult]
    ver: VerifyResult


def step_lengths(inp: dict, tokens) -> tuple:
    """Confidence, survival and the scheduled verify lengths of drafted tokens.

    [blog] "置信度头" and "硬件感知前缀调度器", [summary] section 4: the
    confidence head scores every drafted position from its hidden state and
    the previous token, the survival products rank the candidates, and the
    synchronous greedy scheduler with early stop picks K_b.  Returns
    (ConfidenceResult or None, ScheduleResult or None); without a table every
    request verifies all gamma positions (K = None).
    """
    c = None
    if inp.get("h") is not None:
        c = confidence(inp["h"], inp["E"], inp["anchor"], tokens, inp["wc"], inp["bc"], inp.get("sts_T"))
    s = None
    if inp.get("sps") is not None:
        # the scheduler consumes the survival values as the fp32 the boundary carries
        s = schedule(c.surv.astype(np.float32), inp["sps"])
    return c, s


def run_step(inp: dict, seed: int, rows: Optional[Sequence[int]] = None) -> StepResult:
    wl = inp["wl"]
    B = inp["U"].shape[0]
    rows = np.arange(B) if rows is None else np.asarray(rows, dtype=np.int64)
    has_sched = inp.get("sps") is not None
    if has_sched and len(rows) != B:
        raise ValueError("a scheduled step needs every request")

    def sel(x):
        return x if len(rows) == B else x[rows]

    T = inp["temperature"]
    gru = inp.get("gru")
    if gru is None:
        d = draft_markov(sel(inp["U"]), inp["W1"], inp["W2"], sel(inp["anchor"]),
                         sel(inp["req_ids"]), T, seed, wl.gamma)
    else:
        d = draft_rnn(sel(inp["U"]), inp["W1"], inp["W2"], gru, sel(inp["req_ids"]), T, seed, wl.gamma)
    sub = dict(inp, h=sel(inp["h"]), anchor=sel(inp["anchor"])) if inp.get("h") is not None else inp
    c, s = step_lengths(sub, d.tokens)
    K = None if s is None else s.K
    v = verify(sel(inp["target"]), d.tokens, d.lse, d.ytok, sel(inp["U"]), inp["W1"], inp["W2"],
               sel(inp["anchor"]), K, sel(inp["req_ids"]), T, seed, wl.gamma, states=d.states)
    return StepResult(rows, d, c, s, v)
