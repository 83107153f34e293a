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
