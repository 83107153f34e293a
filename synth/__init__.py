"""Seeded synthetic inputs for the DSpark draft/verify step.

This module only draws random tensors of the right shapes, dtypes and
distributions.  It holds none of the method's arithmetic: no bias, softmax,
sampling, confidence, scheduling or verification.  Both the HIP path (through
its tests and ``bench.py``) and the CPU oracle read the identical bytes it
produces.

Workloads (the paper's pages, "DSpark" technical blog, sections on the Markov
head and the prefix scheduler, plus the long-form summary's deployment
section, describe the shapes; the value distributions are synthetic choices
of this package):

  tiny    B=4,   gamma=7, V=1024,   r=32,  fp32 weights ~N(0,0.1), U ~N(0,2),
          target = U + N(0,0.5), greedy.
  greedy  B=32,  gamma=7, V=151936, r=256, bf16 weights ~N(0,0.02), U ~N(0,3)
          with +8 at one random index per row, target = U + N(0,1), greedy.
  sample  B=128, gamma=7, V=151936, r=256, temperature 1, confidence head over
          [h (4096 bf16 ~N(0,1)); E[prev] (4096 bf16 ~N(0,1))], w_c ~N(0,0.02),
          b_c = 1.
  sched   B=512, gamma=7, V=129280, r=256, temperature 1, STS temperatures
          ~U[1,2], SPS table of 4096 entries, scheduled K_b.
  rnn     B=256, gamma=16, V=151936, r=256, the GRU head (state of width r,
          GRU weights, biases and learned s_0 bf16 ~N(0,0.05)), temperature 1,
          confidence with STS, scheduled K_b as for sched.
  rnn_tiny B=8, gamma=6, V=2048, r=32, fp32 W1/W2 ~N(0,0.1), the GRU head,
          temperature 1 (CPU-scale).

Layouts (row-major, contiguous):
  U, target : float32 [B][gamma+1][V]   (row k-1 holds draft position k)
  W1        : [V][r]  token -> rank-r vector (gathered by previous token)
  W2        : [V][r]  the r x V projection stored column-major, i.e. the
              r-vector of vocab entry v is contiguous (an LM-head layout)
  anchor    : int32 [B]
  req_ids   : int32 [B] (read as uint32)
  h         : bf16 [B][gamma][d_h]
  E         : bf16 [V][d_e]
  wc        : bf16 [d_h + d_e]
  sts_T     : float32 [gamma]
  sps       : float32 [n_sps]   (SPS[N-1] for a verify batch of N tokens)
  GRU head  : W_ih, W_hh bf16 [3r][r] (gate rows in the order reset, update,
              new), b_ih, b_hh bf16 [3r], s0 bf16 [r]

Calibration sets for fitting the per-position confidence temperatures
(``sts_calibration_set``): N held-out drafts of gamma positions.  The world
they come from: each position of each draft has a true acceptance
probability p ~ Beta(8 m_k, 8 (1 - m_k)) with m_k = max(0.85 - 0.03 (k - 1),
0.3) (p clipped to [1e-6, 1 - 1e-6]); the head reports the over-confident logit
T*_k * ln(p / (1 - p)), rounded to float32, with T*_k ~ U[1, 2] per position
(the spread of the STS temperatures above); acceptance events are
independent draws u < p in position order and the accepted length is the
number of leading accepted positions.  The candidate temperatures of the
grid search (``sts_grid``) are 0.5, 0.55, ... (64 values, float32).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    gamma: int
    V: int
    r: int
    wdtype: str            # "f32" or "bf16"
    u_std: float
    w_std: float
    noise_std: float
    peak: Optional[float]  # value added at one random index per row, or None
    temperature: float     # 0 => greedy
    conf: bool = False     # confidence head inputs
    d_h: int = 4096
    d_e: int = 4096
    wc_std: float = 0.02
    bc: float = 1.0
    sts: bool = False
    sched: bool = False
    n_sps: int = 4096
    head: str = "markov"   # "markov" or "gru"
    gru_std: float = 0.05
    seed: int = 1000

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", B=4, gamma=7, V=1024, r=32, wdtype="f32", u_std=2.0,
                     w_std=0.1, noise_std=0.5, peak=None, temperature=0.0, seed=1001),
    "greedy": Workload("greedy", B=32, gamma=7, V=151936, r=256, wdtype="bf16", u_std=3.0,
                       w_std=0.02, noise_std=1.0, peak=8.0, temperature=0.0, seed=1002),
    "sample": Workload("sample", B=128, gamma=7, V=151936, r=256, wdtype="bf16", u_std=3.0,
                       w_std=0.02, noise_std=1.0, peak=None, temperature=1.0, conf=True,
                       seed=1003),
    "sched": Workload("sched", B=512, gamma=7, V=129280, r=256, wdtype="bf16", u_std=3.0,
                      w_std=0.02, noise_std=1.0, peak=None, temperature=1.0, conf=True,
                      sts=True, sched=True, seed=1004),
    "rnn": Workload("rnn", B=256, gamma=16, V=151936, r=256, wdtype="bf16", u_std=3.0,
                    w_std=0.02, noise_std=1.0, peak=None, temperature=1.0, conf=True,
                    sts=True, sched=True, head="gru", seed=1005),
    "rnn_tiny": Workload("rnn_tiny", B=8, gamma=6, V=2048, r=32, wdtype="f32", u_std=2.0,
                         w_std=0.1, noise_std=0.5, peak=None, temperature=1.0, head="gru",
                         seed=1006),
}

# SPS table shape: a step every 64 tokens, slowly decreasing, with three cliffs.
SPS_STEP = 64
SPS_BASE = 1000.0
SPS_SLOPE = 2e-4
SPS_CLIFFS = (1536, 2560, 3584)
SPS_CLIFF_FACTOR = 0.9


def sps_table(n_sps: int = 4096) -> torch.Tensor:
    """Synthetic verify-throughput table: entry N-1 is the steps/s at N tokens."""
    out = torch.empty(n_sps, dtype=torch.float32)
    for n in range(1, n_sps + 1):
        val = SPS_BASE / (1.0 + SPS_SLOPE * math.ceil(n / SPS_STEP))
        for c in SPS_CLIFFS:
            if n >= c:
                val *= SPS_CLIFF_FACTOR
        out[n - 1] = val
    return out


def _randn(g: torch.Generator, shape, std: float) -> torch.Tensor:
    return torch.randn(shape, generator=g, dtype=torch.float32) * std


def make_inputs(wl: Workload, seed: Optional[int] = None, *, random_req_ids: bool = True) -> dict:
    """Draw every input of one step for workload ``wl`` (CPU tensors).

    Draw order is fixed: U, target noise, W1, W2, anchors, peaks, req_ids, h, E,
    wc, STS temperatures, then the GRU head's W_ih, W_hh, b_ih, b_hh, s0.  The
    SPS table is deterministic.
    """
    g = torch.Generator().manual_seed(wl.seed if seed is None else seed)
    B, G, V, r = wl.B, wl.gamma, wl.V, wl.r
    U = _randn(g, (B, G + 1, V), wl.u_std)
    noise = _randn(g, (B, G + 1, V), wl.noise_std)
    W1 = _randn(g, (V, r), wl.w_std)
    W2 = _randn(g, (V, r), wl.w_std)
    if wl.wdtype == "bf16":
        W1 = W1.to(torch.bfloat16)   # round-to-nearest-even
        W2 = W2.to(torch.bfloat16)
    elif wl.wdtype != "f32":
        raise ValueError(wl.wdtype)
    anchor = torch.randint(0, V, (B,), generator=g, dtype=torch.int64).to(torch.int32)
    if wl.peak is not None:
        pk = torch.randint(0, V, (B, G + 1), generator=g, dtype=torch.int64)
        U.scatter_add_(2, pk.unsqueeze(-1), torch.full((B, G + 1, 1), wl.peak))
    target = U + noise
    del noise
    if random_req_ids:
        req = torch.randint(0, 2**31 - 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)
    else:
        req = torch.arange(B, dtype=torch.int32)
    out = dict(wl=wl, U=U, target=target, W1=W1, W2=W2, anchor=anchor, req_ids=req,
               temperature=float(wl.temperature))
    if wl.conf:
        out["h"] = _randn(g, (B, G, wl.d_h), 1.0).to(torch.bfloat16)
        E = torch.empty((V, wl.d_e), dtype=torch.bfloat16)
        chunk = 8192
        for s in range(0, V, chunk):
            e = min(V, s + chunk)
            E[s:e] = _randn(g, (e - s, wl.d_e), 1.0).to(torch.bfloat16)
        out["E"] = E
        out["wc"] = _randn(g, (wl.d_h + wl.d_e,), wl.wc_std).to(torch.bfloat16)
        out["bc"] = float(wl.bc)
        if wl.sts:
            out["sts_T"] = 1.0 + torch.rand((G,), generator=g, dtype=torch.float32)
        else:
            out["sts_T"] = None
    if wl.sched:
        out["sps"] = sps_table(wl.n_sps)
    if wl.head == "gru":
        out["gru"] = dict(
            W_ih=_randn(g, (3 * r, r), wl.gru_std).to(torch.bfloat16),
            W_hh=_randn(g, (3 * r, r), wl.gru_std).to(torch.bfloat16),
            b_ih=_randn(g, (3 * r,), wl.gru_std).to(torch.bfloat16),
            b_hh=_randn(g, (3 * r,), wl.gru_std).to(torch.bfloat16),
            s0=_randn(g, (r,), wl.gru_std).to(torch.bfloat16))
    elif wl.head != "markov":
        raise ValueError(wl.head)
    return out


def survival_rows(B: int, gamma: int, seed: int, *, ties: bool = False) -> torch.Tensor:
    """Random non-increasing rows in (0,1] for exercising a scheduler alone.

    Each row is gamma uniforms sorted in descending order.  With ``ties`` the
    values are quantised to a coarse grid so that equal keys occur across rows.
    """
    g = torch.Generator().manual_seed(seed)
    x = torch.rand((B, gamma), generator=g, dtype=torch.float32)
    if ties:
        x = torch.ceil(x * 8.0) / 8.0
    x, _ = torch.sort(x, dim=1, descending=True)
    return x.contiguous()


def sts_calibration_set(N: int, gamma: int, seed: int, true_T=None) -> dict:
    """Held-out drafts with labels, drawn from the world stated in the module
    header.  Returns logit float32 [N][gamma], accept_len int32 [N] (0..gamma)
    and true_T float64 [gamma] (the over-confidence factors of the head)."""
    rs = np.random.default_rng(seed)
    if true_T is None:
        true_T = 1.0 + rs.random(gamma)
    else:
        true_T = np.asarray(true_T, dtype=np.float64).reshape(gamma)
    m = np.maximum(0.85 - 0.03 * np.arange(gamma), 0.3)
    p = np.clip(rs.beta(8.0 * m, 8.0 * (1.0 - m), size=(N, gamma)), 1e-6, 1.0 - 1e-6)
    u = rs.random((N, gamma))
    logit = (true_T[None, :] * np.log(p / (1.0 - p))).astype(np.float32)
    # accepted length: the leading run of accepted positions
    accept_len = np.cumprod(u < p, axis=1).sum(axis=1).astype(np.int32)
    return {"logit": torch.from_numpy(np.ascontiguousarray(logit)),
            "accept_len": torch.from_numpy(accept_len), "true_T": torch.from_numpy(true_T)}


def sts_grid(n: int = 64, lo: float = 0.5, step: float = 0.05) -> torch.Tensor:
    """Candidate temperatures lo, lo + step, ... as float32."""
    return (lo + step * torch.arange(n, dtype=torch.float64)).to(torch.float32)
