"""Comparison of libdspark outputs with the CPU oracle.

Bar (from the method's definition as an exact sampler):
  * tokens, accept lengths and verify lengths equal exactly, except where the
    oracle's decision margin is below TIE (top-2 key gap of an arg-max, or
    |u - rho| of an accept test).  Such a near-tie is counted, and everything
    after it in that request is not compared (a flipped decision changes the
    rest of the request legitimately);
  * logits-derived values (log-normalisers, tempered logits, confidences,
    survivals) within RTOL relative (absolute floor FLOOR for |x| < 1).
"""
from __future__ import annotations

import dataclasses

import numpy as np

TIE = 1e-4
RTOL = 1e-3
FLOOR = 1e-3


@dataclasses.dataclass
class Report:
    compared: int = 0
    ties: int = 0
    max_rel: float = 0.0
    worst: str = ""
    problems: list = dataclasses.field(default_factory=list)

    def close(self, what, got, want):
        err = abs(float(got) - float(want)) / max(abs(float(want)), FLOOR)
        if err > self.max_rel:
            self.max_rel = err
            self.worst = f"{what} got {float(got)!r} want {float(want)!r}"
        if not err <= RTOL:
            self.problems.append(f"{what}: got {got!r} want {want!r} (rel {err:.2e})")

    def equal(self, what, got, want):
        self.compared += 1
        if int(got) != int(want):
            self.problems.append(f"{what}: got {int(got)} want {int(want)}")

    def ok(self):
        return not self.problems

    def summary(self):
        head = f"compared={self.compared} ties={self.ties} max_rel={self.max_rel:.2e} ({self.worst})"
        return head + ("" if self.ok() else "\n  " + "\n  ".join(self.problems[:20]))


def compare_draft(tok, lse, ytok, od, rows=None, rep=None):
    """GPU draft outputs (numpy) vs oracle DraftResult; returns (report, first tie position)."""
    rep = rep or Report()
    B, G = od.tokens.shape
    rows = np.arange(B) if rows is None else np.asarray(rows)
    taint = np.full(B, G + 1, dtype=np.int64)
    for i in range(B):
        g = rows[i]
        for k in range(1, G + 1):
            rep.close(f"lse[{g},{k}]", lse[g, k - 1], od.lse[i, k - 1])
            if od.margin[i, k - 1] < TIE:
                rep.ties += 1
                taint[i] = k
                if tok[g, k - 1] == od.tokens[i, k - 1]:
                    rep.close(f"ytok[{g},{k}]", ytok[g, k - 1], od.ytok[i, k - 1])
                break
            rep.equal(f"token[{g},{k}]", tok[g, k - 1], od.tokens[i, k - 1])
            if tok[g, k - 1] != od.tokens[i, k - 1]:
                taint[i] = k
                break
            rep.close(f"ytok[{g},{k}]", ytok[g, k - 1], od.ytok[i, k - 1])
    return rep, taint


def compare_states(states, od, taint, rows=None, rep=None):
    """GRU head: the state position k projected ([gamma][B][r] on the GPU,
    [B][gamma][r] in the oracle) is comparable while x_1 .. x_{k-1} agree."""
    rep = rep or Report()
    B, G, _ = od.states.shape
    rows = np.arange(B) if rows is None else np.asarray(rows)
    for i in range(B):
        g = rows[i]
        for k in range(1, min(G, int(taint[i])) + 1):
            got = np.asarray(states[k - 1, g], dtype=np.float64)
            want = od.states[i, k - 1]
            err = np.abs(got - want) / np.maximum(np.abs(want), FLOOR)
            j = int(np.argmax(err))
            rep.close(f"state[{k},{g},{j}]", got[j], want[j])
            rep.compared += 1
    return rep


def compare_confidence(conf, surv, oc, taint, rows=None, rep=None):
    """c_k and a_k are comparable while x_{k-1} agrees (k <= first tie position)."""
    rep = rep or Report()
    B, G = oc.conf.shape
    rows = np.arange(B) if rows is None else np.asarray(rows)
    for i in range(B):
        g = rows[i]
        for k in range(1, min(G, int(taint[i])) + 1):
            rep.close(f"conf[{g},{k}]", conf[g, k - 1], oc.conf[i, k - 1])
            rep.close(f"surv[{g},{k}]", surv[g, k - 1], oc.surv[i, k - 1])
            rep.compared += 1
    return rep


def compare_verify(acc, out, ov, taint, K, rows=None, rep=None):
    """accept lengths and emitted tokens; requests whose drafts differ are skipped."""
    rep = rep or Report()
    B = ov.accept_len.shape[0]
    G = out.shape[1] - 1
    rows = np.arange(B) if rows is None else np.asarray(rows)
    skipped = 0
    for i in range(B):
        g = rows[i]
        kb = G if K is None else int(K[i])
        if taint[i] <= kb:
            skipped += 1
            continue
        A = int(ov.accept_len[i])
        decided = min(A + 1, kb)
        tie_at = None
        for k in range(1, decided + 1):
            if ov.margin[i, k - 1] < TIE:
                tie_at = k
                break
        if tie_at is not None:
            rep.ties += 1
            for j in range(tie_at - 1):
                rep.equal(f"out[{g},{j}]", out[g, j], ov.out_tokens[i, j])
            continue
        rep.equal(f"accept_len[{g}]", acc[g], A)
        for j in range(A):
            rep.equal(f"out[{g},{j}]", out[g, j], ov.out_tokens[i, j])
        if ov.final_margin[i] < TIE:
            rep.ties += 1
        else:
            rep.equal(f"out[{g},{A}]", out[g, A], ov.out_tokens[i, A])
        for j in range(A + 1, G + 1):
            rep.equal(f"pad[{g},{j}]", out[g, j], -1)
    rep.skipped = skipped
    return rep
