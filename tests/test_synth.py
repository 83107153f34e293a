"""The seeded input generator that feeds both the oracle and the GPU path:
identical bytes for identical seeds, the shapes, types and ranges each
workload promises, and the stated recipe (target = U + N(0, noise_std),
weights rounded to bf16, one planted peak per row where asked)."""
import math

import numpy as np
import pytest
import torch

import synth


def small(name, **kw):
    return synth.WORKLOADS[name].with_(**kw)


CASES = [
    small("tiny"),
    small("sample", B=6, V=2048, d_h=16, d_e=24, sts=True),
    small("greedy", B=5, V=1024),
    small("sched", B=7, V=512, d_h=8, d_e=8, n_sps=64),
    small("rnn", B=4, gamma=5, V=768, r=64, d_h=8, d_e=8, n_sps=64),
]


def _flat(d):
    out = {}
    for k, v in d.items():
        if isinstance(v, dict):
            for kk, vv in v.items():
                out[f"{k}.{kk}"] = vv
        else:
            out[k] = v
    return out


@pytest.mark.parametrize("wl", CASES, ids=[w.name for w in CASES])
def test_same_seed_same_bytes(wl):
    a = _flat(synth.make_inputs(wl, seed=123))
    b = _flat(synth.make_inputs(wl, seed=123))
    c = _flat(synth.make_inputs(wl, seed=124))
    assert a.keys() == b.keys()
    for k in a:
        if isinstance(a[k], torch.Tensor):
            assert torch.equal(a[k], b[k]), k
        else:
            assert a[k] == b[k] or (a[k] is None and b[k] is None), k
    assert not torch.equal(a["U"], c["U"])


@pytest.mark.parametrize("wl", CASES, ids=[w.name for w in CASES])
def test_shapes_types_and_ranges(wl):
    d = synth.make_inputs(wl, seed=7)
    B, G, V, r = wl.B, wl.gamma, wl.V, wl.r
    wt = torch.bfloat16 if wl.wdtype == "bf16" else torch.float32
    assert d["U"].shape == (B, G + 1, V) and d["U"].dtype == torch.float32
    assert d["target"].shape == (B, G + 1, V) and d["target"].dtype == torch.float32
    assert d["W1"].shape == (V, r) and d["W1"].dtype == wt
    assert d["W2"].shape == (V, r) and d["W2"].dtype == wt
    assert d["anchor"].dtype == torch.int32 and d["anchor"].shape == (B,)
    assert int(d["anchor"].min()) >= 0 and int(d["anchor"].max()) < V
    assert d["req_ids"].dtype == torch.int32 and int(d["req_ids"].min()) >= 0
    assert d["temperature"] == wl.temperature
    if wl.conf:
        assert d["h"].shape == (B, G, wl.d_h) and d["h"].dtype == torch.bfloat16
        assert d["E"].shape == (V, wl.d_e) and d["E"].dtype == torch.bfloat16
        assert d["wc"].shape == (wl.d_h + wl.d_e,)
        if wl.sts:
            assert d["sts_T"].shape == (G,)
            assert float(d["sts_T"].min()) >= 1.0 and float(d["sts_T"].max()) <= 2.0
        else:
            assert d["sts_T"] is None
    else:
        assert "h" not in d
    if wl.sched:
        assert torch.equal(d["sps"], synth.sps_table(wl.n_sps))
    if wl.head == "gru":
        g = d["gru"]
        assert g["W_ih"].shape == (3 * r, r) and g["W_hh"].shape == (3 * r, r)
        assert g["b_ih"].shape == (3 * r,) and g["b_hh"].shape == (3 * r,) and g["s0"].shape == (r,)
        assert all(v.dtype == torch.bfloat16 for v in g.values())


def test_target_is_u_plus_noise_of_the_stated_spread():
    wl = small("sample", B=8, V=8192, conf=False)
    d = synth.make_inputs(wl, seed=3)
    noise = (d["target"] - d["U"]).double()
    n = noise.numel()
    # sample standard deviation within 5 standard errors of noise_std
    se = wl.noise_std / math.sqrt(2 * n)
    assert abs(float(noise.std()) - wl.noise_std) < 5 * se
    assert abs(float(noise.mean())) < 5 * wl.noise_std / math.sqrt(n)
    assert abs(float(d["U"].double().std()) - wl.u_std) < 5 * wl.u_std / math.sqrt(2 * n)


def test_bf16_weights_are_exactly_representable():
    wl = small("sample", B=2, V=512, conf=False)
    d = synth.make_inputs(wl, seed=5)
    for k in ("W1", "W2"):
        w = d[k]
        assert torch.equal(w.float().to(torch.bfloat16), w)


def test_greedy_workload_plants_one_peak_per_row():
    # U is drawn first, so the same seed without the peak gives the same base
    # logits: the difference is exactly one +peak per row, also in the target
    wl = small("greedy", B=6, V=4096)
    a = synth.make_inputs(wl, seed=9)
    b = synth.make_inputs(wl.with_(peak=None), seed=9)
    diff = (a["U"] - b["U"]).numpy()
    nz = np.count_nonzero(diff, axis=-1)
    assert (nz == 1).all()
    assert np.allclose(diff.max(axis=-1), wl.peak, atol=1e-5)
    tdiff = (a["target"] - a["U"]).numpy() - (b["target"] - b["U"]).numpy()
    assert np.abs(tdiff).max() < 1e-5


def test_sequential_request_ids_on_request():
    wl = small("tiny")
    d = synth.make_inputs(wl, seed=1, random_req_ids=False)
    assert torch.equal(d["req_ids"], torch.arange(wl.B, dtype=torch.int32))


def test_survival_rows_are_non_increasing_in_unit_interval():
    x = synth.survival_rows(9, 6, seed=2)
    assert x.shape == (9, 6)
    assert float(x.min()) > 0.0 and float(x.max()) <= 1.0
    assert bool((x[:, 1:] <= x[:, :-1]).all())
    t = synth.survival_rows(9, 6, seed=2, ties=True)
    assert bool(((t * 8.0) == torch.round(t * 8.0)).all())
