"""GPU: the chained draft kernel (every position in one launch) and the safe
defaults under concurrent work.

The chained draft is the default for bf16 weights, r in {128, 256} and
65..128 requests.  Checked here: one draft-chain launch per call; the same
tokens as the per-position sweeps, with y at the token and the
log-normalisers equal to rounding (one vocabulary chunk per resident
workgroup instead of the sweeps' finer chunks), and bit-identical to them
when given the sweeps' chunks and layout; against the oracle at gamma = 1
(no wait), a long draft and r = 128; while a
long kernel runs on a second stream (its workgroups then cannot all be
resident, and items are claimed by whichever run); with every wait made to
give up from the host (the kernel still ends and the error is reported).

The small-batch whole-draft kernel is launched cooperatively by default; it
is checked while another stream keeps the device busy, and timed against
its plain launch and the per-position sweeps (printed).
"""
import os
import time

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
def ctx():
    c = make_ctx()
    yield c
    c.close()


@pytest.fixture(scope="module")
def sweeps():
    c = make_ctx(DSPARK_CHAIN="0")
    yield c
    c.close()


def draft(ctx, d, T, seed, G):
    out = ctx.draft_markov(d["U"], d["W1"], d["W2"], d["anchor"], d["req_ids"], T, seed, G)
    torch.cuda.synchronize()
    ctx.check()
    return [x.cpu().numpy() for x in out]


def launches(ctx, d, T, seed, G):
    ctx.timing(True)
    ctx.read_timing()
    draft(ctx, d, T, seed, G)
    tk = ctx.read_timing()
    ctx.timing(False)
    return tk["draft_chain"][1], tk["draft_sweep"][1]


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_chain_is_one_launch_and_equals_the_sweeps(ctx, sweeps, T):
    """The chained draft cuts the vocabulary into one chunk per resident
    workgroup, the sweeps into more: the same tokens, and y at the token and
    the log-normalisers to rounding (the same sums in another grouping); a
    chained draft whose chunks are the sweeps' is bit-identical."""
    wl = synth.WORKLOADS["sample"].with_(B=128, gamma=7, V=40960, conf=False, temperature=T)
    d = to_dev(synth.make_inputs(wl, seed=71))
    print(f"chain vs sweeps T={T}", flush=True)
    assert launches(ctx, d, T, 5, wl.gamma) == (1, 0)
    assert launches(sweeps, d, T, 5, wl.gamma) == (0, wl.gamma)
    a = draft(ctx, d, T, 5, wl.gamma)
    b = draft(sweeps, d, T, 5, wl.gamma)
    assert np.array_equal(a[0], b[0])
    assert np.allclose(a[1], b[1], rtol=1e-6, atol=1e-6) and np.allclose(a[2], b[2], rtol=1e-6, atol=1e-6)
    n_vc = sweeps_chunks(wl)
    same = make_ctx(DSPARK_CHAIN_SHAPE=f"4,32,1,{n_vc}")
    try:
        c = draft(same, d, T, 5, wl.gamma)
    finally:
        same.close()
    for x, y in zip(c, b):
        assert np.array_equal(x, y)


def sweeps_chunks(wl):
    """Vocabulary chunks of the per-position shared-tile sweep at this shape
    (the library aims at eight waves per CU: 2048 waves / (4 waves x one
    request quad), at most a chunk per four tiles)."""
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    return min(8 * cu // 4, (wl.V // 16) // 4)


CASES = [
    ("B65_gamma1", "sample", dict(B=65, gamma=1, V=3008, d_h=16, d_e=16)),
    ("B96_gamma16_sts", "sample", dict(B=96, gamma=16, V=2064, d_h=32, d_e=32, sts=True)),
    ("B128_r128_T07", "sample", dict(B=128, V=4096, r=128, temperature=0.7, d_h=16, d_e=16)),
    ("B80_greedy_gamma32", "greedy", dict(B=80, gamma=32, V=1040, peak=None)),
]


@pytest.mark.parametrize("name,base,over", CASES, ids=[c[0] for c in CASES])
def test_chain_against_the_oracle(ctx, name, base, over):
    wl = synth.WORKLOADS[base].with_(**over)
    inp = synth.make_inputs(wl, seed=wl.seed + 31)
    d = to_dev(inp)
    print(f"case {name}", flush=True)
    assert launches(ctx, d, wl.temperature, 3, wl.gamma)[0] == 1
    g = gpu_step(ctx, d, seed=777)
    check_chain(g, inp, 777, min_compared=wl.B)


def _busy_stream(seconds_hint=0.05):
    """Queue a few large matrix products on a second stream (bounded work)."""
    s = torch.cuda.Stream()
    a = torch.randn((4096, 4096), device="cuda")
    with torch.cuda.stream(s):
        for _ in range(12):
            a = torch.tanh(a @ a * 1e-3)
    return s, a


def test_chain_with_a_kernel_running_on_another_stream(ctx):
    wl = synth.WORKLOADS["sample"].with_(B=128, gamma=7, V=40960, conf=False)
    d = to_dev(synth.make_inputs(wl, seed=72))
    ref = draft(ctx, d, 1.0, 9, wl.gamma)
    torch.cuda.synchronize()
    print("chained draft beside a busy stream", flush=True)
    s, _ = _busy_stream()
    got = draft(ctx, d, 1.0, 9, wl.gamma)
    s.synchronize()
    for x, y in zip(ref, got):
        assert np.array_equal(x, y)


def test_chain_wait_timeout_is_reported():
    wl = synth.WORKLOADS["sample"].with_(B=96, gamma=3, V=4096, conf=False)
    d = to_dev(synth.make_inputs(wl, seed=5))
    bctx = make_ctx(DSPARK_BARRIER_TEST="1")
    try:
        print("chained-draft waits made to give up from the host", flush=True)
        bctx.draft_markov(d["U"], d["W1"], d["W2"], d["anchor"], d["req_ids"], 1.0, 3, wl.gamma)
        with pytest.raises(dk.DSparkError, match="grid barrier"):
            bctx.check()
    finally:
        bctx.close()
    ok = make_ctx()
    try:
        draft(ok, d, 1.0, 3, wl.gamma)
    finally:
        ok.close()


def test_small_batch_default_with_a_kernel_running_on_another_stream(ctx):
    """B = 32 uses the whole-draft kernel, launched cooperatively by default."""
    wl = synth.WORKLOADS["greedy"].with_(B=32, gamma=7, V=151936)
    inp = synth.make_inputs(wl, seed=73)
    d = to_dev(inp)
    ref = draft(ctx, d, 0.0, 0, wl.gamma)
    print("whole-draft kernel (default launch) beside a busy stream", flush=True)
    s, _ = _busy_stream()
    got = draft(ctx, d, 0.0, 0, wl.gamma)
    s.synchronize()
    for x, y in zip(ref, got):
        assert np.array_equal(x, y)
    # and it equals the per-position sweeps
    sw = make_ctx(DSPARK_PERSIST="0")
    try:
        alt = draft(sw, d, 0.0, 0, wl.gamma)
    finally:
        sw.close()
    assert np.array_equal(ref[0], alt[0]) and np.array_equal(ref[2], alt[2])


def test_small_batch_draft_times_per_mode():
    """Prints the B = 32 draft call time (greedy, gamma 7, V = 151936) of the
    cooperative (default) and plain launches of the whole-draft kernel and of
    the per-position sweeps; checks only that all three agree."""
    wl = synth.WORKLOADS["greedy"].with_(B=32, gamma=7, V=151936)
    d = to_dev(synth.make_inputs(wl, seed=74))
    res, times = {}, {}
    for name, env in (("cooperative", {}), ("plain", dict(DSPARK_PERSIST_COOP="0")),
                      ("sweeps", dict(DSPARK_PERSIST="0"))):
        c = make_ctx(**env)
        try:
            for i in range(5):
                draft(c, d, 0.0, i, wl.gamma)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(20):
                c.draft_markov(d["U"], d["W1"], d["W2"], d["anchor"], d["req_ids"], 0.0, i, wl.gamma)
            e1.record()
            torch.cuda.synchronize()
            c.check()
            times[name] = 1e3 * e0.elapsed_time(e1) / 20
            res[name] = draft(c, d, 0.0, 3, wl.gamma)
        finally:
            c.close()
    print("B=32 greedy draft call, us: " + ", ".join(f"{k} {v:.1f}" for k, v in times.items()), flush=True)
    for name in ("plain", "sweeps"):
        assert np.array_equal(res["cooperative"][0], res[name][0])
