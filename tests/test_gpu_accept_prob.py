"""GPU parity of the diagnostic pass dspark_accept_prob: the acceptance
probability sum_v min(p_d, p_t) of every drafted position, for the Markov and
the GRU heads, against the CPU oracle.

The drafted tokens, draft log-normalisers and GRU states fed to both sides
come from the oracle's own draft (inputs may flow from the oracle to the GPU,
never back), except in the full-size case, which runs the whole batch through
the GPU draft and compares the sampled rows whose drafts agree.

Tolerance: alpha is a sum of V probabilities, each off by a few fp32 ulps of
its exponent (the logits reach |z/T| ~ 20, so about 2e-6 relative) plus the
fp32 partial sums; ATOL = 5e-5 absolute covers that with a wide margin and is
still far below the spread of alpha between positions (~1e-1).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import semi_ar_draft_amd as dk
from parity import compare_draft

pytestmark = pytest.mark.gpu

ATOL = 5e-5


@pytest.fixture(scope="module")
def ctx():
    c = dk.Context(0)
    yield c
    c.close()


def _check(got, want, what):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == want.shape
    assert np.all(got >= -ATOL) and np.all(got <= 1.0 + ATOL), what
    err = np.abs(got - want)
    i = np.unravel_index(np.argmax(err), err.shape)
    print(f"{what}: max |err| {err.max():.2e} at {i} (got {got[i]:.6f} want {want[i]:.6f})", flush=True)
    assert err.max() <= ATOL, what


@pytest.mark.parametrize("name,wl", [
    ("markov_f32", synth.WORKLOADS["tiny"].with_(B=6, V=4112, temperature=1.0)),
    ("markov_bf16", synth.WORKLOADS["sample"].with_(B=5, gamma=5, V=8240, conf=False)),
    ("markov_hot", synth.WORKLOADS["tiny"].with_(B=4, V=2048, temperature=0.7, u_std=6.0)),
])
def test_accept_prob_markov(ctx, name, wl):
    seed = 31
    inp = synth.make_inputs(wl, seed=wl.seed + 11)
    T = wl.temperature
    print(f"accept_prob {name}: B={wl.B} gamma={wl.gamma} V={wl.V} r={wl.r} T={T}", flush=True)
    od = oracle.draft_markov(inp["U"], inp["W1"], inp["W2"], inp["anchor"], inp["req_ids"], T, seed, wl.gamma)
    want = oracle.accept_prob(inp["target"], od.tokens, od.lse, inp["U"], inp["W1"], inp["W2"], inp["anchor"],
                              T, wl.gamma)
    tok = torch.from_numpy(np.ascontiguousarray(od.tokens, dtype=np.int32)).cuda()
    lse = torch.from_numpy(np.ascontiguousarray(od.lse, dtype=np.float32)).cuda()
    got = ctx.accept_prob(inp["target"].cuda(), inp["U"].cuda(), inp["W1"].cuda(), inp["W2"].cuda(),
                          inp["anchor"].cuda(), tok, lse, T)
    ctx.check()
    _check(got.cpu().numpy(), want, name)


def test_accept_prob_gru(ctx):
    wl = synth.WORKLOADS["rnn_tiny"].with_(B=5, V=4112)
    seed = 32
    inp = synth.make_inputs(wl, seed=wl.seed + 11)
    print(f"accept_prob gru: B={wl.B} gamma={wl.gamma} V={wl.V} r={wl.r}", flush=True)
    od = oracle.draft_rnn(inp["U"], inp["W1"], inp["W2"], inp["gru"], inp["req_ids"], 1.0, seed, wl.gamma)
    want = oracle.accept_prob(inp["target"], od.tokens, od.lse, inp["U"], None, inp["W2"], None, 1.0, wl.gamma,
                              states=od.states)
    tok = torch.from_numpy(np.ascontiguousarray(od.tokens, dtype=np.int32)).cuda()
    lse = torch.from_numpy(np.ascontiguousarray(od.lse, dtype=np.float32)).cuda()
    # oracle states are [B][gamma][r]; the library takes [gamma][B][r]
    states = torch.from_numpy(np.ascontiguousarray(od.states.transpose(1, 0, 2), dtype=np.float32)).cuda()
    got = ctx.accept_prob(inp["target"].cuda(), inp["U"].cuda(), None, inp["W2"].cuda(), None, tok, lse, 1.0,
                          states=states)
    ctx.check()
    _check(got.cpu().numpy(), want, "gru")


def test_accept_prob_full_size_sampled(ctx):
    """The 128-request, 151936-token sampling workload: GPU draft, GPU alpha;
    oracle alpha on sampled rows whose drafted tokens match the oracle's."""
    wl = synth.WORKLOADS["sample"]
    seed = 33
    inp = synth.make_inputs(wl, seed=wl.seed + 11)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    print(f"accept_prob full: B={wl.B} gamma={wl.gamma} V={wl.V}", flush=True)
    tok, lse, ytok = ctx.draft_markov(d["U"], d["W1"], d["W2"], d["anchor"], d["req_ids"], 1.0, seed, wl.gamma)
    got = ctx.accept_prob(d["target"], d["U"], d["W1"], d["W2"], d["anchor"], tok, lse, 1.0)
    ctx.check()
    got = got.cpu().numpy()
    assert np.all(got >= -ATOL) and np.all(got <= 1.0 + ATOL)
    rows = [0, 1, 77, 127]
    sel = lambda x: x[rows]
    od = oracle.draft_markov(sel(inp["U"]), inp["W1"], inp["W2"], sel(inp["anchor"]), sel(inp["req_ids"]), 1.0,
                             seed, wl.gamma)
    rep, taint = compare_draft(tok.cpu().numpy(), lse.cpu().numpy(), ytok.cpu().numpy(), od, rows)
    assert rep.ok(), rep.summary()
    want = oracle.accept_prob(sel(inp["target"]), od.tokens, od.lse, sel(inp["U"]), inp["W1"], inp["W2"],
                              sel(inp["anchor"]), 1.0, wl.gamma)
    # position k depends on tokens 1..k-1 (its bias) and the log-normaliser at k
    for i, g in enumerate(rows):
        n = min(wl.gamma, int(taint[i]))
        _check(got[g, :n], want[i, :n], f"full row {g}")


def test_accept_prob_rejects_greedy(ctx):
    wl = synth.WORKLOADS["tiny"].with_(B=2, gamma=2, V=256)
    inp = synth.make_inputs(wl)
    tok = torch.zeros((2, 2), dtype=torch.int32, device="cuda")
    lse = torch.zeros((2, 2), dtype=torch.float32, device="cuda")
    with pytest.raises(dk.DSparkError):
        ctx.accept_prob(inp["target"].cuda(), inp["U"].cuda(), inp["W1"].cuda(), inp["W2"].cuda(),
                        inp["anchor"].cuda(), tok, lse, 0.0)


def draw_alpha_cases(n=8, seed=9091):
    """Markov-head shapes drawn once from a fixed seed for the diagnostic
    pass: batch sizes on both sides of the shared-tile threshold, ragged
    vocabularies, ranks, both weight types, several temperatures."""
    rs = np.random.default_rng(seed)
    out = []
    for i in range(n):
        wdtype = "bf16" if rs.random() < 0.7 else "f32"
        r = int(rs.choice([32, 64, 128, 256]) if wdtype == "f32" else rs.choice([64, 128, 256]))
        B = int(rs.choice([1, 7, 40, 96, 130]))
        G = int(rs.integers(1, 9))
        V = 16 * int(rs.integers(1, 300))
        T = float(rs.choice([0.7, 1.0, 1.4]))
        out.append((f"a{i}_{wdtype}_r{r}_B{B}_g{G}_V{V}_T{T}", dict(wdtype=wdtype, r=r, B=B, gamma=G, V=V,
                                                                   temperature=T)))
    return out


ALPHA_CASES = draw_alpha_cases()


@pytest.mark.parametrize("name,over", ALPHA_CASES, ids=[c[0] for c in ALPHA_CASES])
def test_accept_prob_shape(ctx, name, over):
    wl = synth.WORKLOADS["sample"].with_(**over, conf=False, peak=None,
                                         u_std=3.0 if over["wdtype"] == "bf16" else 2.0)
    inp = synth.make_inputs(wl, seed=wl.seed + 19)
    T, seed = wl.temperature, 41
    print(f"accept_prob shape {name}", flush=True)
    od = oracle.draft_markov(inp["U"], inp["W1"], inp["W2"], inp["anchor"], inp["req_ids"], T, seed, wl.gamma)
    want = oracle.accept_prob(inp["target"], od.tokens, od.lse, inp["U"], inp["W1"], inp["W2"], inp["anchor"],
                              T, wl.gamma)
    tok = torch.from_numpy(np.ascontiguousarray(od.tokens, dtype=np.int32)).cuda()
    lse = torch.from_numpy(np.ascontiguousarray(od.lse, dtype=np.float32)).cuda()
    got = ctx.accept_prob(inp["target"].cuda(), inp["U"].cuda(), inp["W1"].cuda(), inp["W2"].cuda(),
                          inp["anchor"].cuda(), tok, lse, T)
    ctx.check()
    _check(got.cpu().numpy(), want, name)
