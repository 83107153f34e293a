"""GPU: the host trace ranges.  With DSPARK_ROCTX=1 the library loads the
roctx API and wraps every call in a named range; the results are those of a
run without tracing, bit for bit.  Run in a child process so that the
switch, read once per process, does not leak into the other tests."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import sys, torch
sys.path.insert(0, "tests")
import synth, semi_ar_draft_amd as dk
from test_gpu_parity import to_dev
wl = synth.WORKLOADS["sample"].with_(B=64, V=4096, d_h=64, d_e=256)   # not the cooperative path
d = to_dev(synth.make_inputs(wl, seed=3))
with dk.Context(0) as ctx:
    tok, lse, ytok, conf, surv = ctx.draft_markov_conf(d["U"], d["W1"], d["W2"], d["anchor"], d["req_ids"],
                                                       1.0, 5, wl.gamma, d["h"], d["E"], d["wc"], d["bc"])
    acc, out = ctx.verify(d["target"], d["U"], d["W1"], d["W2"], d["anchor"], tok, lse, ytok, None,
                          d["req_ids"], 1.0, 5)
    ctx.check()
torch.save([x.cpu() for x in (tok, lse, ytok, conf, surv, acc, out)], sys.argv[1])
print("child done", flush=True)
'''


def run(env_extra, path):
    env = dict(os.environ, **env_extra)
    p = subprocess.run([sys.executable, "-c", CHILD, path], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=240)
    assert p.returncode == 0, p.stdout + p.stderr
    assert "child done" in p.stdout


def test_traced_calls_give_the_untraced_results(tmp_path):
    import torch
    print("a step with and without DSPARK_ROCTX=1, each in a child process", flush=True)
    run({"DSPARK_ROCTX": "1"}, str(tmp_path / "on.pt"))
    run({"DSPARK_ROCTX": "0"}, str(tmp_path / "off.pt"))
    a = torch.load(tmp_path / "on.pt")
    b = torch.load(tmp_path / "off.pt")
    for x, y in zip(a, b):
        assert torch.equal(x, y)
