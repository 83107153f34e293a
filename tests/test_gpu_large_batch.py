"""GPU: a large ragged batch (1030 requests: eight full 128-row quads and a
ragged ninth) through the per-position sweeps, the confidence head (two
calls, and the fused call bit for bit) and the verify windows, against the
oracle on every request, with random verify lengths including 0 and gamma.
The batch sizes elsewhere stop at 512; this one exercises the row-quad
indexing, the slot groups and the pending lists well past them."""
import numpy as np
import pytest
import torch

import synth
import semi_ar_draft_amd as dk
from test_gpu_parity import gpu_step, check_chain, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_batch_of_1030_requests(T):
    wl = synth.WORKLOADS["sample"].with_(B=1030, gamma=3, V=2048, r=256, temperature=T, d_h=64, d_e=512,
                                          sts=True)
    inp = synth.make_inputs(wl, seed=77)
    d = to_dev(inp)
    K = np.random.default_rng(5).integers(0, wl.gamma + 1, size=wl.B).astype(np.int32)
    print(f"B={wl.B} T={T}: GPU step with random K, oracle on every request", flush=True)
    with dk.Context(0) as ctx:
        g = gpu_step(ctx, d, seed=91, K=torch.from_numpy(K).cuda())
        f = ctx.draft_markov_conf(d["U"], d["W1"], d["W2"], d["anchor"], d["req_ids"], T, 91, wl.gamma,
                                  d["h"], d["E"], d["wc"], d["bc"], d["sts_T"])
        ctx.check()
        for key, x in zip(("tok", "lse", "ytok", "conf", "surv"), f):
            assert np.array_equal(x.cpu().numpy(), g[key]), key
    check_chain(g, inp, 91, K=K, min_compared=wl.B)
