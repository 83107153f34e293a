"""GPU: a whole step (draft, confidence, verify) captured by the caller into
a HIP graph after one call of the same shape (so the context's workspace
exists) replays to the eager result, every replay, with other eager work
and synchronisations between replays (and two replays back to back) -- for
the per-position draft path, the chained draft and the whole-draft kernel
(plain launch; its default cooperative launch is not meant for capture),
with the draft and the confidence head as two calls or as the one fused
call (whose per-request counters every launch leaves at zero).  The library
records no memset into a graph: every clear it needs is a kernel."""
import os

import pytest
import torch

import synth
import semi_ar_draft_amd as dk
from test_gpu_parity import to_dev

pytestmark = pytest.mark.gpu


ENVS = [
    (70, dict(DSPARK_CHAIN="0")),                                 # per-position sweeps
    (70, {}),                                                     # chained draft (default at this size)
    (16, dict(DSPARK_PERSIST="2", DSPARK_PERSIST_COOP="0")),      # whole-draft kernel, plain launch
]


@pytest.mark.parametrize("fused", [False, True], ids=["two_calls", "fused"])
@pytest.mark.parametrize("B,env", ENVS, ids=["per_position", "chained", "whole_draft"])
def test_captured_step_replays_to_the_eager_result(B, env, fused):
    old = {k: os.environ.get(k) for k in env}
    os.environ.update(env)
    try:
        ctx = dk.Context(0)
    finally:
        for k, v in old.items():
            if v is None:
                del os.environ[k]
            else:
                os.environ[k] = v
    wl = synth.WORKLOADS["sample"].with_(B=B, V=4096, d_h=128 if fused else 32, d_e=1024 if fused else 32, sts=True)
    d = to_dev(synth.make_inputs(wl, seed=71))
    G = wl.gamma
    dev = "cuda"
    tok = torch.empty((B, G), dtype=torch.int32, device=dev)
    lse = torch.empty((B, G), device=dev)
    ytok = torch.empty((B, G), device=dev)
    conf = torch.empty((B, G), device=dev)
    surv = torch.empty((B, G), device=dev)
    acc = torch.empty((B,), dtype=torch.int32, device=dev)
    out = torch.empty((B, G + 1), dtype=torch.int32, device=dev)
    bufs = (tok, lse, ytok, conf, surv, acc, out)

    def step(seed):
        if fused:
            ctx.draft_markov_conf(d["U"], d["W1"], d["W2"], d["anchor"], d["req_ids"], 1.0, seed, G, d["h"], d["E"],
                                  d["wc"], d["bc"], d["sts_T"], out=(tok, lse, ytok, conf, surv))
        else:
            ctx.draft_markov(d["U"], d["W1"], d["W2"], d["anchor"], d["req_ids"], 1.0, seed, G,
                             out=(tok, lse, ytok))
            ctx.confidence(d["h"], d["E"], d["anchor"], tok, d["wc"], d["bc"], d["sts_T"], out=(conf, surv))
        ctx.verify(d["target"], d["U"], d["W1"], d["W2"], d["anchor"], tok, lse, ytok, None, d["req_ids"], 1.0,
                   seed, out=(acc, out))

    try:
        step(5)
        ctx.check()
        torch.cuda.synchronize()
        ref = [x.clone() for x in bufs]
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step(5)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        print(f"capturing the step, B={B}, env={env}, fused={fused}", flush=True)
        with torch.cuda.graph(g, stream=s):
            step(5)
        torch.cuda.synchronize()
        for rep in range(3):
            for x in bufs:
                x.zero_()
            step(6)                                      # other eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for name, a, b in zip(("tok", "lse", "ytok", "conf", "surv", "acc", "out"), ref, bufs):
                assert torch.equal(a, b), f"replay {rep}: {name}"
        for x in bufs:
            x.zero_()
        g.replay()                                      # two replays back to back
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("tok", "lse", "ytok", "conf", "surv", "acc", "out"), ref, bufs):
            assert torch.equal(a, b), f"back-to-back replay: {name}"
        ctx.check()
    finally:
        ctx.close()
