"""GPU parity of the whole-draft kernel (Markov head, bf16 weights, r = 256,
B <= 128): every draft position in one launch of one workgroup per CU, W2
held in registers, positions separated by a grid barrier.

By default the library uses it for small batches only; the contexts here are
created with DSPARK_PERSIST=2, which selects it for every eligible batch, so
the same kernel is checked at the shapes the per-position sweeps are
checked at: against the oracle (small and ragged shapes, waves that own no
vocabulary tile, a long draft, the full-size sampling workload on sampled
requests), against the per-position sweeps (greedy full size: z at the
drafted token and the tokens are bit-identical, the MFMA sums being taken in
the same order), at the largest vocabulary it covers and one tile past it
(which falls back to the per-position sweeps), launched plainly (identical
results to the default cooperative launch), and with its barrier made to
time out from the host (the kernel still ends and the error is reported).
"""
import os

import numpy as np
import pytest
import torch

import synth
import semi_ar_draft_amd as dk
from test_gpu_parity import gpu_step, check_chain, to_dev

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


@pytest.fixture(scope="module")
def pctx():
    c = make_ctx(DSPARK_PERSIST="2")
    yield c
    c.close()


def draft_launches(ctx, d, T, seed, G):
    """Draft-sweep launches of one draft call (1 = the whole-draft kernel)."""
    ctx.timing(True)
    ctx.read_timing()
    out = ctx.draft_markov(d["U"], d["W1"], d["W2"], d["anchor"], d["req_ids"], T, seed, G)
    torch.cuda.synchronize()
    n = ctx.read_timing()["draft_sweep"][1]
    ctx.timing(False)
    ctx.check()
    return n, out


CASES = [
    # name, workload, overrides
    ("sample_B1_gamma2", "sample", dict(B=1, gamma=2, V=160, d_h=8, d_e=8)),
    ("greedy_B40_ragged", "greedy", dict(B=40, V=5008, peak=None)),
    ("sample_B70_T07", "sample", dict(B=70, V=3008, temperature=0.7, d_h=32, d_e=96, sts=True)),
    ("sample_B100_gamma16", "sample", dict(B=100, gamma=16, V=2064, d_h=32, d_e=32, sts=True)),
    # 2560 tiles: two or three per wave
    ("sample_B128_V40960", "sample", dict(B=128, gamma=3, V=40960, d_h=16, d_e=16)),
    # one tile in all: every wave but one owns none
    ("sample_B3_V16", "sample", dict(B=3, gamma=3, V=16, d_h=8, d_e=8)),
    # the longest draft: 31 barriers
    ("greedy_B8_gamma32", "greedy", dict(B=8, gamma=32, V=1040, peak=None)),
]


@pytest.mark.parametrize("name,base,over", CASES, ids=[c[0] for c in CASES])
def test_persist_chain(pctx, name, base, over):
    wl = synth.WORKLOADS[base].with_(**over)
    inp = synth.make_inputs(wl, seed=wl.seed + 23)
    d = to_dev(inp)
    print(f"persist {name}: B={wl.B} gamma={wl.gamma} V={wl.V} r={wl.r} T={wl.temperature}", flush=True)
    n, _ = draft_launches(pctx, d, wl.temperature, 1, wl.gamma)
    assert n == 1, f"whole-draft kernel not used ({n} sweep launches)"
    g = gpu_step(pctx, d, seed=4321)
    check_chain(g, inp, 4321)


def test_persist_full_sample_sampled(pctx):
    wl = synth.WORKLOADS["sample"]
    inp = synth.make_inputs(wl)
    d = to_dev(inp)
    rows = [0, 1, 15, 16, 63, 64, 100, 127]
    print(f"persist full sample B={wl.B} V={wl.V} rows={rows}", flush=True)
    n, _ = draft_launches(pctx, d, wl.temperature, 1, wl.gamma)
    assert n == 1
    g = gpu_step(pctx, d, seed=77)
    check_chain(g, inp, 77, rows=rows, min_compared=len(rows))
    # deterministic: the same seed gives the same draft
    g2 = gpu_step(pctx, d, seed=77)
    for k in g:
        assert np.array_equal(g[k], g2[k]), k


def test_persist_greedy_matches_sweeps(pctx):
    wl = synth.WORKLOADS["greedy"]
    inp = synth.make_inputs(wl)
    d = to_dev(inp)
    sctx = make_ctx(DSPARK_PERSIST="0")
    try:
        n_s, a = draft_launches(sctx, d, 0.0, 5, wl.gamma)
    finally:
        sctx.close()
    n_p, b = draft_launches(pctx, d, 0.0, 5, wl.gamma)
    print(f"greedy B={wl.B}: sweeps {n_s} launches, whole-draft {n_p}", flush=True)
    assert n_s == wl.gamma and n_p == 1
    ta, la, ya = (x.cpu().numpy() for x in a)
    tb, lb, yb = (x.cpu().numpy() for x in b)
    assert np.array_equal(ta, tb)
    assert np.array_equal(ya, yb)
    np.testing.assert_allclose(lb, la, rtol=2e-6, atol=2e-6)


def test_persist_vocabulary_limit(pctx):
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    vmax = 16 * 10 * 4 * cu                      # register tiles of every wave
    for V, whole in ((vmax, True), (vmax + 16, False)):
        wl = synth.WORKLOADS["greedy"].with_(B=8, gamma=3, V=V, peak=None)
        inp = synth.make_inputs(wl, seed=9)
        d = to_dev(inp)
        print(f"vocabulary limit: V={V} (max {vmax})", flush=True)
        n_p, b = draft_launches(pctx, d, 0.0, 2, wl.gamma)
        assert (n_p == 1) == whole
        sctx = make_ctx(DSPARK_PERSIST="0")
        try:
            _, a = draft_launches(sctx, d, 0.0, 2, wl.gamma)
        finally:
            sctx.close()
        assert np.array_equal(a[0].cpu().numpy(), b[0].cpu().numpy())
        assert np.array_equal(a[2].cpu().numpy(), b[2].cpu().numpy())


def test_persist_plain_launch_matches_cooperative(pctx):
    wl = synth.WORKLOADS["sample"].with_(B=24, gamma=5, V=20480, conf=False)
    inp = synth.make_inputs(wl, seed=13)
    d = to_dev(inp)
    pl = make_ctx(DSPARK_PERSIST="2", DSPARK_PERSIST_COOP="0")
    try:
        print("plain launch of the whole-draft kernel", flush=True)
        n_c, a = draft_launches(pl, d, 1.0, 8, wl.gamma)
    finally:
        pl.close()
    n_p, b = draft_launches(pctx, d, 1.0, 8, wl.gamma)
    assert n_c == 1 and n_p == 1
    for x, y in zip(a, b):
        assert np.array_equal(x.cpu().numpy(), y.cpu().numpy())


def test_persist_barrier_timeout_is_reported():
    wl = synth.WORKLOADS["sample"].with_(B=16, gamma=3, V=4096, conf=False)
    inp = synth.make_inputs(wl, seed=5)
    d = to_dev(inp)
    bctx = make_ctx(DSPARK_PERSIST="2", DSPARK_BARRIER_TEST="1")
    try:
        print("barrier made to time out from the host", flush=True)
        bctx.draft_markov(d["U"], d["W1"], d["W2"], d["anchor"], d["req_ids"], 1.0, 3, wl.gamma)
        with pytest.raises(dk.DSparkError, match="grid barrier"):
            bctx.check()
        # the next call on a healthy context is unaffected
    finally:
        bctx.close()
    ok = make_ctx(DSPARK_PERSIST="2")
    try:
        ok.draft_markov(d["U"], d["W1"], d["W2"], d["anchor"], d["req_ids"], 1.0, 3, wl.gamma)
        ok.check()
    finally:
        ok.close()
