"""GPU: dspark_draft_markov_conf -- the draft with its merge done by the
confidence launch -- against dspark_draft_markov then dspark_confidence:
tokens, lse, ytok, confidences and survivals bit for bit, through each draft
path (chained draft, per-position sweeps, whole-draft kernel), sampling and
greedy, with and without STS temperatures, gamma 1 and 32, one request,
rows of up to 4096 values (the headline width);
one launch fewer (no draft combine), and a second call on the same context
(the slot groups, the chained draft's counters and the per-request counters
are left at zero), also after a call with a larger batch."""
import os

import numpy as np
import pytest
import torch

import synth
import semi_ar_draft_amd as dk
from test_gpu_parity import to_dev

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


CASES = [
    ("chained_T1_sts", dict(), dict(B=128, gamma=7, V=40960, d_h=256, d_e=128, sts=True)),
    ("chained_greedy", dict(), dict(B=100, gamma=5, V=8192, d_h=64, d_e=64, temperature=0.0)),
    ("sweeps_T07", dict(DSPARK_CHAIN="0"), dict(B=128, gamma=9, V=8192, d_h=64, d_e=32, temperature=0.7)),
    ("sweeps_B140", dict(), dict(B=140, gamma=4, V=4096, d_h=32, d_e=32)),
    ("whole_draft_B32", dict(), dict(B=32, gamma=7, V=16384, d_h=64, d_e=64)),
    ("whole_draft_B96", dict(DSPARK_PERSIST="2"), dict(B=96, gamma=6, V=8192, d_h=64, d_e=64, sts=True)),
    ("fp32_weights", dict(), dict(B=48, gamma=3, V=2048, r=64, wdtype="f32", d_h=16, d_e=16)),
    ("gamma1", dict(), dict(B=64, gamma=1, V=4096, d_h=64, d_e=64)),
    ("gamma32_greedy", dict(), dict(B=24, gamma=32, V=2048, d_h=32, d_e=64, temperature=0.0, sts=True)),
    ("B1", dict(), dict(B=1, gamma=5, V=3008, d_h=8, d_e=8)),
    # rows of 4096 values: every lane of a wave reads part of the E row at x_k
    ("chained_d4096", dict(), dict(B=128, gamma=7, V=16384, d_h=4096, d_e=4096, sts=True)),
    ("sweeps_B512_d4096", dict(), dict(B=512, gamma=7, V=8192, d_h=4096, d_e=4096, sts=True)),
    ("whole_draft_d1024", dict(), dict(B=32, gamma=7, V=8192, d_h=1024, d_e=2048)),
]


@pytest.mark.parametrize("name,env,over", CASES, ids=[c[0] for c in CASES])
def test_fused_equals_separate_calls(name, env, over):
    wl = synth.WORKLOADS["sample"].with_(conf=True, **over)
    d = to_dev(synth.make_inputs(wl, seed=wl.seed + 41))
    T = wl.temperature
    sts = d.get("sts_T")
    ctx = make_ctx(**env)
    try:
        print(f"draft + confidence fused vs separate: {name}", flush=True)
        args = (d["U"], d["W1"], d["W2"], d["anchor"], d["req_ids"], T, 9, wl.gamma)
        tok, lse, ytok = ctx.draft_markov(*args)
        conf, surv = ctx.confidence(d["h"], d["E"], d["anchor"], tok, d["wc"], d["bc"], sts)
        torch.cuda.synchronize()
        ctx.check()
        ref = [x.cpu().numpy() for x in (tok, lse, ytok, conf, surv)]
        for rep in range(2):
            ctx.timing(True)
            ctx.read_timing()
            got = ctx.draft_markov_conf(*args, d["h"], d["E"], d["wc"], d["bc"], sts)
            torch.cuda.synchronize()
            tk = ctx.read_timing()
            ctx.timing(False)
            ctx.check()
            assert tk["conf_merge"][1] == 1 and tk["draft_combine"][1] == 0 and tk["confidence"][1] == 0
            for x, y in zip(got, ref):
                assert np.array_equal(x.cpu().numpy(), y), rep
    finally:
        ctx.close()


def test_fused_batch_sizes_in_turn():
    """Calls with growing and shrinking batches on one context: the counter
    block grows with the batch and every call leaves it at zero."""
    ctx = make_ctx()
    try:
        for i, B in enumerate((40, 200, 17, 200)):
            wl = synth.WORKLOADS["sample"].with_(conf=True, B=B, gamma=6, V=4096, d_h=32, d_e=32)
            d = to_dev(synth.make_inputs(wl, seed=100 + i))
            print(f"draft + confidence fused, B={B}", flush=True)
            args = (d["U"], d["W1"], d["W2"], d["anchor"], d["req_ids"], wl.temperature, 3 + i, wl.gamma)
            tok, lse, ytok = ctx.draft_markov(*args)
            conf, surv = ctx.confidence(d["h"], d["E"], d["anchor"], tok, d["wc"], d["bc"], None)
            ref = [x.cpu().numpy() for x in (tok, lse, ytok, conf, surv)]
            got = ctx.draft_markov_conf(*args, d["h"], d["E"], d["wc"], d["bc"], None)
            torch.cuda.synchronize()
            ctx.check()
            for x, y in zip(got, ref):
                assert np.array_equal(x.cpu().numpy(), y), B
    finally:
        ctx.close()
