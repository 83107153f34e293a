"""GPU parity over a seeded spread of shapes: the whole step (draft,
confidence, verify with random verify lengths) against the oracle on every
request, for configurations drawn once from a fixed seed -- batch sizes on
both sides of the shared-tile and whole-draft thresholds, one to twelve
positions, ragged vocabularies (any multiple of 16), every supported rank,
both weight types, greedy and several temperatures, with and without the
confidence head.  bf16 cases with r = 256 and B <= 128 also run with the
whole-draft kernel forced on (DSPARK_PERSIST=2), so both draft paths meet
the same cases.  Cases with the confidence head also run the fused draft +
confidence call, which must give the two calls' outputs bit for bit (its
embedding rows of 1024 values keep every lane of a wave busy).
"""
import os

import numpy as np
import pytest
import torch

import synth
import semi_ar_draft_amd as dk
from test_gpu_parity import gpu_step, check_chain, to_dev

pytestmark = pytest.mark.gpu


def draw_cases(n=40, seed=20240611):
    rs = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        wdtype = "bf16" if rs.random() < 0.7 else "f32"
        r = int(rs.choice([32, 64, 128, 256] if wdtype == "f32" else [64, 128, 256, 256]))
        B = int(rs.choice([1, 3, 17, 33, 48, 64, 65, 96, 100, 128, 140]))
        G = int(rs.integers(1, 13))
        V = 16 * int(rs.integers(1, 400))
        T = float(rs.choice([0.0, 0.5, 1.0, 1.5]))
        conf = bool(rs.random() < 0.5)
        vary_k = bool(rs.random() < 0.5)
        cases.append((f"s{i}_{wdtype}_r{r}_B{B}_g{G}_V{V}_T{T}{'_conf' if conf else ''}{'_K' if vary_k else ''}",
                      dict(wdtype=wdtype, r=r, B=B, gamma=G, V=V, temperature=T, conf=conf), vary_k))
    return cases


CASES = draw_cases()


@pytest.fixture(scope="module")
def ctx():
    c = dk.Context(0)
    yield c
    c.close()


@pytest.fixture(scope="module")
def pctx():
    os.environ["DSPARK_PERSIST"] = "2"
    try:
        c = dk.Context(0)
    finally:
        del os.environ["DSPARK_PERSIST"]
    yield c
    c.close()


@pytest.mark.parametrize("name,over,vary_k", CASES, ids=[c[0] for c in CASES])
def test_shape(ctx, pctx, name, over, vary_k):
    base = "sample" if over["wdtype"] == "bf16" else "tiny"
    wl = synth.WORKLOADS[base].with_(**over, d_h=32, d_e=1024, peak=None,
                                      u_std=3.0 if over["wdtype"] == "bf16" else 2.0)
    inp = synth.make_inputs(wl, seed=wl.seed + 101)
    d = to_dev(inp)
    K = None
    if vary_k:
        rs = np.random.default_rng(len(name))
        K = rs.integers(0, wl.gamma + 1, size=wl.B).astype(np.int32)
    print(f"shape {name}", flush=True)
    Kd = None if K is None else torch.from_numpy(K).cuda()
    g = gpu_step(ctx, d, seed=555, K=Kd)
    check_chain(g, inp, 555, K=K)
    if wl.conf:
        f = ctx.draft_markov_conf(d["U"], d["W1"], d["W2"], d["anchor"], d["req_ids"], d["temperature"], 555,
                                  wl.gamma, d["h"], d["E"], d["wc"], d["bc"], d.get("sts_T"))
        ctx.check()
        for key, x in zip(("tok", "lse", "ytok", "conf", "surv"), f):
            assert np.array_equal(x.cpu().numpy(), g[key]), key
    if wl.wdtype == "bf16" and wl.r == 256 and wl.B <= 128 and wl.gamma > 1:
        g2 = gpu_step(pctx, d, seed=555, K=Kd)
        check_chain(g2, inp, 555, K=K)
