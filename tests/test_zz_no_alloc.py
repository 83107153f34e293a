"""GPU: the allocation-free draft entry point (dspark_draft_markov_static)
through the C ABI against dspark_draft_markov on the same inputs: two calls
in a row, the second with a smaller input (so the shared per-GPU scratch
holds the first call's contents when the second starts), on the chained
draft and on the per-position sweeps; a shape beyond the scratch's limit is
refused before anything is enqueued."""
import os

import numpy as np
import pytest
import torch

import synth
import semi_ar_draft_amd as dk
from test_gpu_parity import to_dev

pytestmark = pytest.mark.gpu


def _draft(ctx, d, wl, seed, static):
    out = ctx.draft_markov(d["U"], d["W1"], d["W2"], d["anchor"], d["req_ids"], wl.temperature, seed,
                           wl.gamma, static=static)
    torch.cuda.synchronize()
    ctx.check()
    return [x.cpu().numpy() for x in out]


CALLS = [
    # (workload, overrides): the first is the headline shape, the second smaller
    ("sample", dict(conf=False)),
    ("sample", dict(B=80, gamma=5, V=40960, conf=False, temperature=0.8)),
    ("greedy", dict(B=32, gamma=4, V=20480, peak=None)),     # per-position sweeps
]


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


def test_static_draft_matches_the_allocating_entry_point():
    """Bit-identical to dspark_draft_markov on a context that also avoids the
    whole-draft kernel; against the default context (which takes the
    whole-draft kernel at B = 32) tokens and ytok are identical and lse agrees
    to rounding (the same partials merged in a different chunking)."""
    ctx = _ctx()
    same = _ctx(DSPARK_PERSIST="0")
    try:
        for i, (base, over) in enumerate(CALLS):
            wl = synth.WORKLOADS[base].with_(**over)
            d = to_dev(synth.make_inputs(wl, seed=90 + i))
            print(f"static draft call {i}: B={wl.B} gamma={wl.gamma} V={wl.V} T={wl.temperature}", flush=True)
            got = _draft(ctx, d, wl, 300 + i, static=True)
            exact = _draft(same, d, wl, 300 + i, static=False)
            for name, a, b in zip(("tokens", "lse", "ytok"), exact, got):
                assert np.array_equal(a, b), (i, name)
            dflt = _draft(ctx, d, wl, 300 + i, static=False)
            assert np.array_equal(dflt[0], got[0]) and np.array_equal(dflt[2], got[2]), i
            assert np.allclose(dflt[1], got[1], rtol=1e-5, atol=1e-5), i
            del d
            torch.cuda.empty_cache()
    finally:
        ctx.close()
        same.close()


def test_static_draft_refuses_a_shape_beyond_its_scratch():
    wl = synth.WORKLOADS["sample"].with_(B=128, gamma=32, V=151936, conf=False)
    ctx = dk.Context(0)
    try:
        U = torch.zeros((wl.B, wl.gamma, wl.V), device="cuda")
        W = torch.zeros((wl.V, wl.r), dtype=torch.bfloat16, device="cuda")
        anchor = torch.zeros((wl.B,), dtype=torch.int32, device="cuda")
        with pytest.raises(dk.DSparkError, match="allocation-free draft"):
            ctx.draft_markov(U, W, W, anchor, None, 1.0, 1, wl.gamma, static=True)
    finally:
        ctx.close()
