"""GPU: verification over a flattened (packed) target -- request b's rows
1 .. K_b + 1 laid end to end with per-request row offsets -- is bit-identical
to the padded layout and matches the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
import semi_ar_draft_amd as dk
from parity import compare_draft, compare_verify

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    c = dk.Context(0)
    yield c
    c.close()


def pack(target: torch.Tensor, K: np.ndarray, order):
    """Rows 1..K_b+1 of every request, requests in the given order; returns
    (packed [n_rows][V], offsets [B])."""
    B = target.shape[0]
    offs = np.zeros(B, dtype=np.int32)
    parts, row = [], 0
    for b in order:
        offs[b] = row
        parts.append(target[b, :int(K[b]) + 1])
        row += int(K[b]) + 1
    return torch.cat(parts, 0).contiguous(), offs


def _case(name):
    if name == "markov_small":
        return synth.WORKLOADS["sample"].with_(B=48, V=4096, d_h=16, d_e=16), 5
    if name == "markov_full":
        return synth.WORKLOADS["sample"], 6
    if name == "gru_small":
        return synth.WORKLOADS["rnn"].with_(B=40, gamma=8, V=2048, r=128, conf=False, sts=False, sched=False), 7
    raise KeyError(name)


@pytest.mark.parametrize("name", ["markov_small", "gru_small", "markov_full"])
def test_packed_equals_padded_and_oracle(ctx, name):
    wl, seed = _case(name)
    inp = synth.make_inputs(wl, seed=wl.seed + 3)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    K = np.random.default_rng(seed).integers(0, wl.gamma + 1, size=wl.B).astype(np.int32)
    K[:2] = [0, wl.gamma]
    Kd = torch.from_numpy(K).cuda()
    packed, offs = pack(inp["target"], K, order=list(range(wl.B))[::-1])
    print(f"packed verify {name}: B={wl.B} gamma={wl.gamma} V={wl.V} rows={packed.shape[0]}", flush=True)
    gru = inp.get("gru")
    if gru is None:
        tok, lse, ytok = ctx.draft_markov(d["U"], d["W1"], d["W2"], d["anchor"], d["req_ids"], 1.0, seed, wl.gamma)
        states = None
    else:
        tok, lse, ytok, states = ctx.draft_rnn(d["U"], d["W1"], d["W2"], {k: v.cuda() for k, v in gru.items()},
                                               d["req_ids"], 1.0, seed, wl.gamma)
    a1, o1 = ctx.verify(d["target"], d["U"], d["W1"], d["W2"], d["anchor"], tok, lse, ytok, Kd, d["req_ids"],
                        1.0, seed, states=states)
    a2, o2 = ctx.verify_packed(packed.cuda(), torch.from_numpy(offs).cuda(), d["U"], d["W1"], d["W2"], d["anchor"],
                               tok, lse, ytok, Kd, d["req_ids"], 1.0, seed, states=states)
    ctx.check()
    assert torch.equal(a1, a2) and torch.equal(o1, o2)
    rows = list(range(wl.B)) if wl.B <= 64 else [0, 1, 2, 64, 127]
    sel = lambda x: x[rows]
    if gru is None:
        od = oracle.draft_markov(sel(inp["U"]), inp["W1"], inp["W2"], sel(inp["anchor"]), sel(inp["req_ids"]),
                                 1.0, seed, wl.gamma)
    else:
        od = oracle.draft_rnn(sel(inp["U"]), inp["W1"], inp["W2"], gru, sel(inp["req_ids"]), 1.0, seed, wl.gamma)
    rep, taint = compare_draft(tok.cpu().numpy(), lse.cpu().numpy(), ytok.cpu().numpy(), od, rows)
    ov = oracle.verify(sel(inp["target"]), od.tokens, od.lse, od.ytok, sel(inp["U"]), inp["W1"], inp["W2"],
                       sel(inp["anchor"]), K[rows], sel(inp["req_ids"]), 1.0, seed, wl.gamma, states=od.states)
    compare_verify(a2.cpu().numpy(), o2.cpu().numpy(), ov, taint, K[rows], rows, rep)
    print(rep.summary(), flush=True)
    assert rep.ok(), rep.summary()


def test_packed_row_out_of_range_is_flagged(ctx):
    wl = synth.WORKLOADS["sample"].with_(B=8, V=1024, d_h=8, d_e=8)
    inp = synth.make_inputs(wl, seed=3)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    K = np.full(wl.B, 2, dtype=np.int32)
    packed, offs = pack(inp["target"], K, order=range(wl.B))
    offs[5] = packed.shape[0] - 1          # rows 2 and 3 of request 5 fall past the end
    tok, lse, ytok = ctx.draft_markov(d["U"], d["W1"], d["W2"], d["anchor"], d["req_ids"], 1.0, 1, wl.gamma)
    ctx.verify_packed(packed.cuda(), torch.from_numpy(offs).cuda(), d["U"], d["W1"], d["W2"], d["anchor"],
                      tok, lse, ytok, torch.from_numpy(K).cuda(), d["req_ids"], 1.0, 1)
    with pytest.raises(dk.DSparkError) as e:
        ctx.check()
    assert e.value.code == dk.DSPARK_EDEVICE and "packed" in str(e.value)
    ctx.check()   # the flag is cleared


def draw_packed_cases(n=10, seed=5150):
    """Markov-head shapes drawn once from a fixed seed for the packed layout:
    batch sizes on both sides of the shared-tile threshold, ragged
    vocabularies, ranks, both weight types, greedy and sampling."""
    rs = np.random.default_rng(seed)
    out = []
    for i in range(n):
        wdtype = "bf16" if rs.random() < 0.7 else "f32"
        r = int(rs.choice([64, 128, 256]))
        B = int(rs.choice([1, 9, 33, 70, 100, 128]))
        G = int(rs.integers(1, 10))
        V = 16 * int(rs.integers(1, 300))
        T = float(rs.choice([0.0, 0.8, 1.0]))
        out.append((f"p{i}_{wdtype}_r{r}_B{B}_g{G}_V{V}_T{T}", dict(wdtype=wdtype, r=r, B=B, gamma=G, V=V,
                                                                   temperature=T)))
    return out


PACKED_CASES = draw_packed_cases()


@pytest.mark.parametrize("name,over", PACKED_CASES, ids=[c[0] for c in PACKED_CASES])
def test_packed_shape(ctx, name, over):
    wl = synth.WORKLOADS["sample"].with_(**over, conf=False, peak=None,
                                         u_std=3.0 if over["wdtype"] == "bf16" else 2.0)
    inp = synth.make_inputs(wl, seed=wl.seed + 71)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    rs = np.random.default_rng(len(name))
    K = rs.integers(0, wl.gamma + 1, size=wl.B).astype(np.int32)
    Kd = torch.from_numpy(K).cuda()
    packed, offs = pack(inp["target"], K, order=list(rs.permutation(wl.B)))
    T, seed = wl.temperature, 606
    print(f"packed shape {name}: rows={packed.shape[0]}", flush=True)
    tok, lse, ytok = ctx.draft_markov(d["U"], d["W1"], d["W2"], d["anchor"], d["req_ids"], T, seed, wl.gamma)
    a1, o1 = ctx.verify(d["target"], d["U"], d["W1"], d["W2"], d["anchor"], tok, lse, ytok, Kd, d["req_ids"],
                        T, seed)
    a2, o2 = ctx.verify_packed(packed.cuda(), torch.from_numpy(offs).cuda(), d["U"], d["W1"], d["W2"], d["anchor"],
                               tok, lse, ytok, Kd, d["req_ids"], T, seed)
    ctx.check()
    assert torch.equal(a1, a2) and torch.equal(o1, o2)
    od = oracle.draft_markov(inp["U"], inp["W1"], inp["W2"], inp["anchor"], inp["req_ids"], T, seed, wl.gamma)
    rep, taint = compare_draft(tok.cpu().numpy(), lse.cpu().numpy(), ytok.cpu().numpy(), od)
    ov = oracle.verify(inp["target"], od.tokens, od.lse, od.ytok, inp["U"], inp["W1"], inp["W2"], inp["anchor"], K,
                       inp["req_ids"], T, seed, wl.gamma)
    compare_verify(a2.cpu().numpy(), o2.cpu().numpy(), ov, taint, K, None, rep)
    print(rep.summary(), flush=True)
    assert rep.ok(), rep.summary()
