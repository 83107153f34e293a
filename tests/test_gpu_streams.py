"""GPU: the library works on the caller's stream and keeps no state shared
between contexts.  The full step on a side stream equals the same step on
the default stream bit for bit; two contexts used in turn on one stream (the
whole-draft kernel, whose barrier counter is per context) equal one context;
two contexts running the per-position path on two streams at once equal the
same calls run one after the other, and so do two contexts running the fused
draft + confidence call (chained draft) on two streams at once.  (Two whole-draft launches at once are
not run: their workgroups may not all be resident together, which the
library documents.)"""
import os

import numpy as np
import pytest
import torch

import synth
import semi_ar_draft_amd as dk
from test_gpu_parity import gpu_step, to_dev

pytestmark = pytest.mark.gpu


def _ctx(**env):
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


def _equal(a, b):
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_step_on_a_side_stream_equals_default_stream():
    wl = synth.WORKLOADS["sample"].with_(B=70, V=4096, d_h=32, d_e=32, sts=True)
    inp = synth.make_inputs(wl, seed=61)
    d = to_dev(inp)
    ctx = _ctx()
    try:
        a = gpu_step(ctx, d, seed=5)
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            b = gpu_step(ctx, d, seed=5)
        s.synchronize()
    finally:
        ctx.close()
    _equal(a, b)


def test_two_contexts_in_turn_with_the_whole_draft_kernel():
    wl = synth.WORKLOADS["sample"].with_(B=16, V=8192, d_h=16, d_e=16)
    inp = synth.make_inputs(wl, seed=62)
    d = to_dev(inp)
    c1, c2 = _ctx(DSPARK_PERSIST="2"), _ctx(DSPARK_PERSIST="2")
    try:
        ref = gpu_step(c1, d, seed=9)
        outs = []
        for i in range(3):
            outs.append(gpu_step(c2 if i % 2 == 0 else c1, d, seed=9))
    finally:
        c1.close()
        c2.close()
    for o in outs:
        _equal(ref, o)


def test_two_contexts_on_two_streams_at_once():
    wl = synth.WORKLOADS["sample"].with_(B=96, V=6144, d_h=32, d_e=32)
    i1 = to_dev(synth.make_inputs(wl, seed=63))
    i2 = to_dev(synth.make_inputs(wl, seed=64))
    c1, c2 = _ctx(DSPARK_PERSIST="0"), _ctx(DSPARK_PERSIST="0")
    try:
        r1 = gpu_step(c1, i1, seed=11)
        r2 = gpu_step(c2, i2, seed=12)
        torch.cuda.synchronize()
        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        G = wl.gamma
        res = []
        for ctx, d, s, seed in ((c1, i1, s1, 11), (c2, i2, s2, 12)):
            with torch.cuda.stream(s):
                tok, lse, ytok = ctx.draft_markov(d["U"], d["W1"], d["W2"], d["anchor"], d["req_ids"],
                                                  d["temperature"], seed, G)
                conf, surv = ctx.confidence(d["h"], d["E"], d["anchor"], tok, d["wc"], d["bc"], d.get("sts_T"))
                acc, out = ctx.verify(d["target"], d["U"], d["W1"], d["W2"], d["anchor"], tok, lse, ytok, None,
                                      d["req_ids"], d["temperature"], seed)
            res.append(dict(tok=tok, lse=lse, ytok=ytok, conf=conf, surv=surv, acc=acc, out=out))
        s1.synchronize()
        s2.synchronize()
        c1.check(s1)
        c2.check(s2)
    finally:
        c1.close()
        c2.close()
    for want, got in ((r1, res[0]), (r2, res[1])):
        for k, v in got.items():
            assert np.array_equal(want[k], v.cpu().numpy()), k


def test_fused_call_on_two_streams_at_once():
    """The fused draft + confidence call of two contexts on two streams at
    once (each context has its own per-request counters) equals the two
    calls run one after the other on the default stream."""
    wl = synth.WORKLOADS["sample"].with_(B=100, V=6144, d_h=64, d_e=1024, sts=True)
    i1 = to_dev(synth.make_inputs(wl, seed=65))
    i2 = to_dev(synth.make_inputs(wl, seed=66))
    c1, c2 = _ctx(), _ctx()
    try:
        r1 = gpu_step(c1, i1, seed=13)
        r2 = gpu_step(c2, i2, seed=14)
        torch.cuda.synchronize()
        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        res = []
        for ctx, d, s, seed in ((c1, i1, s1, 13), (c2, i2, s2, 14)):
            with torch.cuda.stream(s):
                f = ctx.draft_markov_conf(d["U"], d["W1"], d["W2"], d["anchor"], d["req_ids"], d["temperature"], seed,
                                          wl.gamma, d["h"], d["E"], d["wc"], d["bc"], d.get("sts_T"))
            res.append(dict(zip(("tok", "lse", "ytok", "conf", "surv"), f)))
        s1.synchronize()
        s2.synchronize()
        c1.check(s1)
        c2.check(s2)
    finally:
        c1.close()
        c2.close()
    for want, got in ((r1, res[0]), (r2, res[1])):
        for k, v in got.items():
            assert np.array_equal(want[k], v.cpu().numpy()), k
