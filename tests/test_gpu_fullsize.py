"""GPU parity at the full sizes, on every request.

* The headline workload (B = 128, gamma = 7, V = 151936, r = 256, T = 1,
  confidence head d = 4096): the whole step -- draft, confidence and
  survival, verify with residual and bonus -- on all 128 requests against
  the oracle, through each draft path: the chained draft (the default at
  this size), the per-position sweeps and the whole-draft kernel.
* The scheduled workload (B = 512, gamma = 7, V = 129280, STS temperatures,
  the 4096-entry SPS table): GPU draft -> GPU confidence and STS -> GPU
  scheduler -> GPU verify with the scheduler's K, against the oracle's
  composed step (run_step) on all 512 requests.  K, n and Theta are compared
  when the oracle's early stop is clear of a near-tie; the draft and
  confidence outputs always; the verify outputs with the oracle's K.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
import semi_ar_draft_amd as dk
from parity import compare_draft, compare_confidence, compare_verify, TIE
from test_gpu_parity import gpu_step, to_dev

pytestmark = pytest.mark.gpu


def make_ctx(**env):
    old = {k: os.environ.get(k) for k in env}
    os.environ.update(env)
    try:
        return dk.Context(0)
    finally:
        for k, v in old.items():
            if v is None:
                del os.environ[k]
            else:
                os.environ[k] = v


SEED = 4711


@pytest.fixture(scope="module")
def headline():
    wl = synth.WORKLOADS["sample"]
    inp = synth.make_inputs(wl)
    print("oracle step on all 128 requests of the headline batch", flush=True)
    ref = oracle.run_step(inp, SEED)
    return inp, to_dev(inp), ref


PATHS = [("chained", {}), ("sweeps", dict(DSPARK_CHAIN="0")), ("whole_draft", dict(DSPARK_PERSIST="2"))]


@pytest.mark.parametrize("name,env", PATHS, ids=[p[0] for p in PATHS])
def test_headline_all_requests(headline, name, env):
    inp, d, ref = headline
    wl = inp["wl"]
    ctx = make_ctx(**env)
    try:
        print(f"headline batch through the {name} draft path", flush=True)
        g = gpu_step(ctx, d, seed=SEED)
    finally:
        ctx.close()
    rep, taint = compare_draft(g["tok"], g["lse"], g["ytok"], ref.draft)
    compare_confidence(g["conf"], g["surv"], ref.conf, taint, rep=rep)
    compare_verify(g["acc"], g["out"], ref.ver, taint, None, rep=rep)
    print(f"{name}: {rep.summary()}", flush=True)
    assert rep.ok(), rep.summary()
    # every request compared, up to its near-ties
    assert rep.compared >= wl.B * wl.gamma


def test_scheduled_workload_all_requests():
    wl = synth.WORKLOADS["sched"]
    inp = synth.make_inputs(wl)
    d = to_dev(inp)
    ctx = make_ctx()
    try:
        print(f"scheduled batch B={wl.B} V={wl.V} on the GPU", flush=True)
        g = gpu_step(ctx, d, seed=SEED, schedule=True)
    finally:
        ctx.close()
    print("oracle composed step (run_step) on all 512 requests", flush=True)
    ref = oracle.run_step(inp, SEED)
    rep, taint = compare_draft(g["tok"], g["lse"], g["ytok"], ref.draft)
    compare_confidence(g["conf"], g["surv"], ref.conf, taint, rep=rep)
    s = ref.sched
    clean = bool(np.all(taint > wl.gamma)) and s.min_rel_step > TIE
    print(f"schedule: oracle n={s.n_selected} gpu n={int(g['nsel'][0])} "
          f"min_rel_step={s.min_rel_step:.2e} clean={clean}", flush=True)
    assert 0 < s.n_selected < wl.B * wl.gamma          # the early stop did cut
    if clean:
        assert np.array_equal(g["K"], s.K)
        assert int(g["nsel"][0]) == s.n_selected
        assert abs(float(g["theta"][0]) - s.theta) <= 1e-6 * s.theta
        compare_verify(g["acc"], g["out"], ref.ver, taint, s.K, rep=rep)
    print(rep.summary(), flush=True)
    assert rep.ok(), rep.summary()
    assert rep.compared >= wl.B * wl.gamma
