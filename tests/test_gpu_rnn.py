"""GPU parity of the GRU (RNN) head path: libdspark through its C ABI against
the CPU oracle (draft with states, confidence, schedule, verify whose
residual projects the states)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import semi_ar_draft_amd as dk
from parity import Report, compare_draft, compare_states, compare_confidence, compare_verify, TIE

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    c = dk.Context(0)
    yield c
    c.close()


def to_dev(inp):
    out = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    out["gru"] = {k: v.cuda() for k, v in inp["gru"].items()}
    return out


def gpu_step(ctx, d, seed, K=None, schedule=False):
    G = d["wl"].gamma
    tok, lse, ytok, states = ctx.draft_rnn(d["U"], d["W1"], d["W2"], d["gru"], d["req_ids"],
                                           d["temperature"], seed, G)
    res = dict(tok=tok, lse=lse, ytok=ytok, states=states)
    if d.get("h") is not None:
        res["conf"], res["surv"] = ctx.confidence(d["h"], d["E"], d["anchor"], tok, d["wc"], d["bc"],
                                                  d.get("sts_T"))
    if schedule:
        res["K"], res["nsel"], res["theta"] = ctx.schedule(res["surv"], d["sps"])
        K = res["K"]
    res["acc"], res["out"] = ctx.verify(d["target"], d["U"], None, d["W2"], None, tok, lse, ytok, K,
                                        d["req_ids"], d["temperature"], seed, states=states)
    ctx.check()
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in res.items()}


def oracle_draft(inp, seed, rows=None):
    sel = (lambda x: x) if rows is None else (lambda x: x[rows])
    d = oracle.draft_rnn(sel(inp["U"]), inp["W1"], inp["W2"], inp["gru"], sel(inp["req_ids"]),
                         inp["temperature"], seed, inp["wl"].gamma)
    c = None
    if inp.get("h") is not None:
        c = oracle.confidence(sel(inp["h"]), inp["E"], sel(inp["anchor"]), d.tokens, inp["wc"], inp["bc"],
                              inp.get("sts_T"))
    return d, c


def oracle_verify(inp, d, seed, rows=None, K=None):
    sel = (lambda x: x) if rows is None else (lambda x: x[rows])
    return oracle.verify(sel(inp["target"]), d.tokens, d.lse, d.ytok, sel(inp["U"]), None, inp["W2"], None, K,
                         sel(inp["req_ids"]), inp["temperature"], seed, inp["wl"].gamma, states=d.states)


def check(g, inp, seed, rows=None, K=None, min_compared=1):
    d, c = oracle_draft(inp, seed, rows)
    rep, taint = compare_draft(g["tok"], g["lse"], g["ytok"], d, rows)
    compare_states(g["states"], d, taint, rows, rep)
    if c is not None:
        compare_confidence(g["conf"], g["surv"], c, taint, rows, rep)
    v = oracle_verify(inp, d, seed, rows, K)
    compare_verify(g["acc"], g["out"], v, taint, K, rows, rep)
    print(rep.summary(), flush=True)
    assert rep.ok(), rep.summary()
    assert rep.compared >= min_compared
    return rep, taint, v


SMALL = [
    ("tiny_f32_sample", "rnn_tiny", {}),
    ("tiny_f32_greedy", "rnn_tiny", dict(temperature=0.0)),
    ("tiny_f32_r64_T08", "rnn_tiny", dict(r=64, B=5, gamma=4, temperature=0.8)),
    ("bf16_shared_r128", "rnn", dict(B=96, gamma=5, V=4096, r=128, d_h=32, d_e=32, sts=False, sched=False)),
    ("bf16_shared_r256_conf", "rnn", dict(B=70, gamma=6, V=3008, d_h=64, d_e=64, sched=False)),
    ("bf16_private_r256", "rnn", dict(B=20, gamma=7, V=2048, conf=False, sts=False, sched=False)),
]


@pytest.mark.parametrize("name,base,over", SMALL, ids=[s[0] for s in SMALL])
def test_small_rnn_chain(ctx, name, base, over):
    wl = synth.WORKLOADS[base].with_(**over)
    inp = synth.make_inputs(wl, seed=wl.seed + 23)
    print(f"rnn case {name}: B={wl.B} gamma={wl.gamma} V={wl.V} r={wl.r} T={wl.temperature}", flush=True)
    g = gpu_step(ctx, to_dev(inp), seed=4321)
    check(g, inp, 4321, min_compared=wl.B)


def test_rnn_variable_K(ctx):
    wl = synth.WORKLOADS["rnn"].with_(B=48, gamma=8, V=2048, r=128, d_h=16, d_e=16, sched=False)
    inp = synth.make_inputs(wl, seed=31)
    K = np.random.default_rng(3).integers(0, wl.gamma + 1, size=wl.B).astype(np.int32)
    K[:3] = [0, wl.gamma, 1]
    print(f"rnn variable K: {K[:10]}", flush=True)
    g = gpu_step(ctx, to_dev(inp), seed=8, K=torch.from_numpy(K).cuda())
    check(g, inp, 8, K=K)


def test_rnn_scheduled_chain(ctx):
    wl = synth.WORKLOADS["rnn"].with_(B=64, gamma=16, V=2048, r=64, d_h=32, d_e=32, n_sps=1024)
    inp = synth.make_inputs(wl, seed=41)
    print(f"rnn scheduled chain B={wl.B} gamma={wl.gamma} n_sps={wl.n_sps}", flush=True)
    g = gpu_step(ctx, to_dev(inp), seed=6, schedule=True)
    d, c = oracle_draft(inp, 6)
    rep, taint = compare_draft(g["tok"], g["lse"], g["ytok"], d)
    compare_states(g["states"], d, taint, rep=rep)
    compare_confidence(g["conf"], g["surv"], c, taint, rep=rep)
    s = oracle.schedule(c.surv.astype(np.float32), inp["sps"])
    clean = bool(np.all(taint > wl.gamma)) and s.min_rel_step > TIE
    print(f"schedule: oracle n={s.n_selected} gpu n={int(g['nsel'][0])} clean={clean}", flush=True)
    if clean:
        assert np.array_equal(g["K"], s.K)
        v = oracle_verify(inp, d, 6, K=s.K)
        compare_verify(g["acc"], g["out"], v, taint, s.K, rep=rep)
    print(rep.summary(), flush=True)
    assert rep.ok(), rep.summary()


def test_full_rnn_shape_sampled(ctx):
    """The GRU head's headline shape (B=256, gamma=16, V=151936, r=256) in the
    benchmark's launch configuration; sampled requests, a seeded K."""
    wl = synth.WORKLOADS["rnn"]
    inp = synth.make_inputs(wl)
    d = to_dev(inp)
    rows = [0, 37, 128, 255]
    K = np.random.default_rng(9).integers(0, wl.gamma + 1, size=wl.B).astype(np.int32)
    K[rows[0]] = wl.gamma
    print(f"full rnn shape B={wl.B} gamma={wl.gamma} V={wl.V} rows={rows}", flush=True)
    g = gpu_step(ctx, d, seed=11, K=torch.from_numpy(K).cuda())
    del d
    check(g, inp, 11, rows=rows, K=K[rows], min_compared=len(rows))


def test_rnn_is_deterministic(ctx):
    wl = synth.WORKLOADS["rnn"].with_(B=96, gamma=5, V=4096, r=128, d_h=32, d_e=32, sts=False, sched=False)
    d = to_dev(synth.make_inputs(wl, seed=5))
    a = gpu_step(ctx, d, seed=3)
    b = gpu_step(ctx, d, seed=3)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def draw_rnn_cases(n=16, seed=77031):
    """GRU-head shapes drawn once from a fixed seed: batch sizes on both sides
    of the shared-tile threshold, one to ten positions, ragged vocabularies,
    every rank, both W1 types, greedy and several temperatures, random K."""
    rs = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        wdtype = "bf16" if rs.random() < 0.7 else "f32"
        r = int(rs.choice([32, 64, 128, 256]))
        B = int(rs.choice([1, 5, 31, 33, 64, 96, 129, 160]))
        G = int(rs.integers(1, 11))
        V = 16 * int(rs.integers(1, 300))
        T = float(rs.choice([0.0, 0.7, 1.0, 1.3]))
        cases.append((f"g{i}_{wdtype}_r{r}_B{B}_g{G}_V{V}_T{T}",
                      dict(wdtype=wdtype, r=r, B=B, gamma=G, V=V, temperature=T)))
    return cases


RNN_CASES = draw_rnn_cases()


@pytest.mark.parametrize("name,over", RNN_CASES, ids=[c[0] for c in RNN_CASES])
def test_rnn_shape(ctx, name, over):
    wl = synth.WORKLOADS["rnn"].with_(**over, conf=False, sts=False, sched=False,
                                      u_std=3.0 if over["wdtype"] == "bf16" else 2.0)
    inp = synth.make_inputs(wl, seed=wl.seed + 211)
    rs = np.random.default_rng(len(name))
    K = rs.integers(0, wl.gamma + 1, size=wl.B).astype(np.int32)
    print(f"rnn shape {name}", flush=True)
    g = gpu_step(ctx, to_dev(inp), seed=808, K=torch.from_numpy(K).cuda())
    check(g, inp, 808, K=K)
