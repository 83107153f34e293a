"""GPU: the verify chain (every needed target row in one launch, each
request's rows decided one after another inside it) against the window
passes and the oracle.

The chain merges a row's chunk partials in the order the window path's
decision kernel uses, so its outputs are bit-identical to the windows'; they
are checked so on greedy and sampling batches with random verify lengths
(including 0 and gamma), fewer requests than partitions, the packed target
layout and the GRU head's states, and against the oracle on the headline
batch (every request).  Also: while a long kernel runs on a second stream,
replayed from a captured HIP graph, and with every wait for a row made to
give up from the host (the kernel still ends and the error is reported).
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
import semi_ar_draft_amd as dk
from parity import compare_draft, compare_verify
from test_gpu_packed import pack
from test_gpu_parity import to_dev
from test_gpu_rnn import to_dev as to_dev_rnn

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
def chain():
    c = make_ctx(DSPARK_VERIFY_CHAIN="1")
    yield c
    c.close()


@pytest.fixture(scope="module")
def windows():
    c = make_ctx(DSPARK_VERIFY_CHAIN="0")
    yield c
    c.close()


def launches(ctx, fn):
    ctx.timing(True)
    ctx.read_timing()
    out = fn()
    torch.cuda.synchronize()
    tk = ctx.read_timing()
    ctx.timing(False)
    return out, tk


def draft(ctx, d, seed):
    return ctx.draft_markov(d["U"], d["W1"], d["W2"], d["anchor"], d["req_ids"], d["temperature"], seed,
                            d["wl"].gamma)


def verify(ctx, d, dr, K, seed):
    tok, lse, ytok = dr
    acc, out = ctx.verify(d["target"], d["U"], d["W1"], d["W2"], d["anchor"], tok, lse, ytok, K, d["req_ids"],
                          d["temperature"], seed)
    torch.cuda.synchronize()
    ctx.check()
    return acc.cpu().numpy(), out.cpu().numpy()


CASES = [
    ("sample_B128_V40960", "sample", dict(B=128, gamma=7, V=40960, conf=False)),
    ("sample_T07_B96_g12", "sample", dict(B=96, gamma=12, V=8192, temperature=0.7, conf=False)),
    ("greedy_B80_g32", "greedy", dict(B=80, gamma=32, V=1040, peak=None)),
    ("greedy_peaked_B32", "greedy", dict(B=32, gamma=7, V=16384)),
    ("sample_B5_g3", "sample", dict(B=5, gamma=3, V=2064, conf=False)),
    ("sample_B1_g1", "sample", dict(B=1, gamma=1, V=3008, conf=False)),
    ("sample_B140_r128", "sample", dict(B=140, gamma=9, V=6144, r=128, conf=False)),
]


@pytest.mark.parametrize("name,base,over", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("Kmode", ["full", "random"])
def test_chain_equals_windows(chain, windows, name, base, over, Kmode):
    wl = synth.WORKLOADS[base].with_(**over)
    inp = synth.make_inputs(wl, seed=wl.seed + 17)
    d = to_dev(inp)
    rs = np.random.default_rng(len(name) * 7 + wl.B)
    K = None if Kmode == "full" else torch.from_numpy(rs.integers(0, wl.gamma + 1, wl.B).astype(np.int32)).cuda()
    print(f"verify chain vs windows {name} K={Kmode}", flush=True)
    dr = draft(windows, d, 11)
    (a1, o1), tk = launches(chain, lambda: verify(chain, d, dr, K, 12))
    assert tk["verify_chain"][1] == 1 and tk["verify_rows"][1] == 0 and tk["verify_decide"][1] == 0
    a2, o2 = verify(windows, d, dr, K, 12)
    assert np.array_equal(a1, a2)
    assert np.array_equal(o1, o2)
    # and a second call on the same context (the counter block is left at zero)
    a3, o3 = verify(chain, d, dr, K, 12)
    assert np.array_equal(a1, a3) and np.array_equal(o1, o3)


def test_chain_headline_batch_against_the_oracle(chain):
    wl = synth.WORKLOADS["sample"]
    inp = synth.make_inputs(wl)
    d = to_dev(inp)
    seed = 4711
    print("headline batch: GPU draft, verify chain; oracle on all 128 requests", flush=True)
    tok, lse, ytok = draft(chain, d, seed)
    acc, out = chain.verify(d["target"], d["U"], d["W1"], d["W2"], d["anchor"], tok, lse, ytok, None, d["req_ids"],
                            1.0, seed)
    chain.check()
    ref = oracle.run_step(dict(inp, h=None), seed)
    rep, taint = compare_draft(tok.cpu().numpy(), lse.cpu().numpy(), ytok.cpu().numpy(), ref.draft)
    compare_verify(acc.cpu().numpy(), out.cpu().numpy(), ref.ver, taint, None, rep=rep)
    print(rep.summary(), flush=True)
    assert rep.ok(), rep.summary()
    assert rep.compared >= wl.B * wl.gamma


def test_chain_packed_layout(chain, windows):
    wl = synth.WORKLOADS["sample"].with_(B=48, V=4096, d_h=16, d_e=16, conf=False)
    inp = synth.make_inputs(wl, seed=5)
    d = to_dev(inp)
    rs = np.random.default_rng(3)
    K = rs.integers(0, wl.gamma + 1, wl.B).astype(np.int32)
    packed, offs = pack(inp["target"], K, order=list(rs.permutation(wl.B)))
    tok, lse, ytok = draft(windows, d, 5)
    Kd = torch.from_numpy(K).cuda()
    res = []
    for c in (chain, windows):
        a, o = c.verify_packed(packed.cuda(), torch.from_numpy(offs).cuda(), d["U"], d["W1"], d["W2"], d["anchor"],
                               tok, lse, ytok, Kd, d["req_ids"], wl.temperature, 5)
        c.check()
        res.append((a.cpu().numpy(), o.cpu().numpy()))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])


def test_chain_gru_states(chain, windows):
    wl = synth.WORKLOADS["rnn"].with_(B=40, gamma=8, V=2048, r=128, conf=False, sts=False, sched=False)
    inp = synth.make_inputs(wl, seed=7)
    d = to_dev_rnn(inp)
    tok, lse, ytok, states = windows.draft_rnn(d["U"], d["W1"], d["W2"], d["gru"], d["req_ids"], wl.temperature, 7,
                                               wl.gamma)
    res = []
    for c in (chain, windows):
        a, o = c.verify(d["target"], d["U"], None, d["W2"], None, tok, lse, ytok, None, d["req_ids"],
                        wl.temperature, 7, states=states)
        c.check()
        res.append((a.cpu().numpy(), o.cpu().numpy()))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])


def _busy_stream():
    s = torch.cuda.Stream()
    a = torch.randn((4096, 4096), device="cuda")
    with torch.cuda.stream(s):
        for _ in range(12):
            a = torch.tanh(a @ a * 1e-3)
    return s, a


def test_chain_with_a_kernel_running_on_another_stream(chain):
    wl = synth.WORKLOADS["sample"].with_(B=128, gamma=7, V=40960, conf=False)
    d = to_dev(synth.make_inputs(wl, seed=72))
    dr = draft(chain, d, 9)
    ref = verify(chain, d, dr, None, 9)
    print("verify chain beside a busy stream", flush=True)
    s, _ = _busy_stream()
    got = verify(chain, d, dr, None, 9)
    s.synchronize()
    assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1])


def test_chain_graph_replays(chain):
    wl = synth.WORKLOADS["sample"].with_(B=96, gamma=7, V=8192, conf=False)
    d = to_dev(synth.make_inputs(wl, seed=31))
    tok, lse, ytok = draft(chain, d, 3)
    K = torch.full((wl.B,), wl.gamma, dtype=torch.int32, device="cuda")
    acc = torch.empty((wl.B,), dtype=torch.int32, device="cuda")
    out = torch.empty((wl.B, wl.gamma + 1), dtype=torch.int32, device="cuda")
    args = (d["target"], d["U"], d["W1"], d["W2"], d["anchor"], tok, lse, ytok, K, d["req_ids"], 1.0, 3)
    chain.verify(*args, out=(acc, out))                  # sizes the workspace outside the capture
    chain.check()
    ref = (acc.cpu().numpy().copy(), out.cpu().numpy().copy())
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        chain.verify(*args, out=(acc, out), stream=s)
    other = synth.WORKLOADS["sample"].with_(B=70, gamma=4, V=4096, conf=False)
    d2 = to_dev(synth.make_inputs(other, seed=2))
    dr2 = draft(chain, d2, 4)
    for i in range(3):
        acc.fill_(-7)
        out.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        chain.check()
        assert np.array_equal(acc.cpu().numpy(), ref[0]) and np.array_equal(out.cpu().numpy(), ref[1]), i
        verify(chain, d2, dr2, None, 4)                   # eager work of another shape between replays


def test_chain_wait_timeout_is_reported(windows):
    wl = synth.WORKLOADS["greedy"].with_(B=96, gamma=5, V=4096, peak=None)
    d = to_dev(synth.make_inputs(wl, seed=5))
    dr = draft(windows, d, 3)
    bctx = make_ctx(DSPARK_VERIFY_CHAIN="1", DSPARK_BARRIER_TEST="1")
    try:
        print("verify-chain waits made to give up from the host", flush=True)
        bctx.verify(d["target"], d["U"], d["W1"], d["W2"], d["anchor"], *dr, None, d["req_ids"], 0.0, 3)
        with pytest.raises(dk.DSparkError, match="grid barrier"):
            bctx.check()
    finally:
        bctx.close()
    ok = make_ctx(DSPARK_VERIFY_CHAIN="1")
    try:
        a1, o1 = verify(ok, d, dr, None, 3)
    finally:
        ok.close()
    a2, o2 = verify(windows, d, dr, None, 3)
    assert np.array_equal(a1, a2) and np.array_equal(o1, o2)
