"""GPU: the whole-draft kernel's cooperative launch (the default for small
batches) when the runtime refuses it -- as it does while another process on
the device holds the cooperative-launch resource.  The library then runs
that call on the per-position sweeps: the draft still completes, with the
whole-draft kernel's tokens.  Here a parent process keeps a context that
has made cooperative launches while a child process drafts the same batch;
the child's greedy tokens and y at the token equal the parent's bit for
bit (the two paths agree exactly on greedy drafts), and its sampled draft
and verification equal the oracle.  Which path the child took is printed:
the outcome must not depend on it."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
import semi_ar_draft_amd as dk
from parity import compare_draft, compare_verify
from test_gpu_parity import to_dev

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import sys, numpy as np, torch
sys.path.insert(0, "tests")
import synth, semi_ar_draft_amd as dk
from test_gpu_parity import to_dev
out = {}
with dk.Context(0) as ctx:
    for T in (0.0, 1.0):
        wl = synth.WORKLOADS["sample"].with_(B=24, V=8192, conf=False, temperature=T)
        d = to_dev(synth.make_inputs(wl, seed=12))
        ctx.timing(True); ctx.read_timing()
        tok, lse, ytok = ctx.draft_markov(d["U"], d["W1"], d["W2"], d["anchor"], d["req_ids"], T, 6, wl.gamma)
        acc, o = ctx.verify(d["target"], d["U"], d["W1"], d["W2"], d["anchor"], tok, lse, ytok, None,
                            d["req_ids"], T, 6)
        torch.cuda.synchronize(); ctx.check()
        tk = ctx.read_timing(); ctx.timing(False)
        print(f"child T={T}: draft sweep launches {tk['draft_sweep'][1]}", flush=True)
        out[f"T{T}"] = [x.cpu().numpy() for x in (tok, lse, ytok, acc, o)]
np.savez(sys.argv[1], **{f"{k}_{i}": v for k, vs in out.items() for i, v in enumerate(vs)})
print("child done", flush=True)
'''


def test_draft_completes_when_the_cooperative_launch_is_refused(tmp_path):
    wl = synth.WORKLOADS["sample"].with_(B=24, V=8192, conf=False, temperature=0.0)
    inp = synth.make_inputs(wl, seed=12)
    d = to_dev(inp)
    with dk.Context(0) as ctx:
        ctx.timing(True)
        ctx.read_timing()
        tok, lse, ytok = ctx.draft_markov(d["U"], d["W1"], d["W2"], d["anchor"], d["req_ids"], 0.0, 6, wl.gamma)
        torch.cuda.synchronize()
        ctx.check()
        tk = ctx.read_timing()
        ctx.timing(False)
        print(f"parent: draft sweep launches {tk['draft_sweep'][1]}", flush=True)
        ref_tok, ref_y = tok.cpu().numpy(), ytok.cpu().numpy()
        # the child drafts while this context (and its cooperative launches) is alive
        path = str(tmp_path / "child.npz")
        p = subprocess.run([sys.executable, "-c", CHILD, path], cwd=ROOT, capture_output=True, text=True,
                           timeout=240)
        print(p.stdout, flush=True)
        assert p.returncode == 0, p.stdout + p.stderr
    got = np.load(path)
    assert np.array_equal(got["T0.0_0"], ref_tok)
    assert np.array_equal(got["T0.0_2"], ref_y)
    # the sampled draft and its verification against the oracle
    wl1 = synth.WORKLOADS["sample"].with_(B=24, V=8192, conf=False, temperature=1.0)
    inp1 = synth.make_inputs(wl1, seed=12)
    od = oracle.draft_markov(inp1["U"], inp1["W1"], inp1["W2"], inp1["anchor"], inp1["req_ids"], 1.0, 6,
                             wl1.gamma)
    ov = oracle.verify(inp1["target"], od.tokens, od.lse, od.ytok, inp1["U"], inp1["W1"], inp1["W2"],
                       inp1["anchor"], None, inp1["req_ids"], 1.0, 6, wl1.gamma)
    rep, taint = compare_draft(got["T1.0_0"], got["T1.0_1"], got["T1.0_2"], od)
    compare_verify(got["T1.0_3"], got["T1.0_4"], ov, taint, None, rep=rep)
    print(rep.summary(), flush=True)
    assert rep.ok(), rep.summary()
