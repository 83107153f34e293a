"""GPU parity of the temperature fit (dspark_sts_fit) against the oracle
(oracle/sts_fit.py) on synthetic calibration sets (synth.sts_calibration_set).

The GPU scores in fp32; the oracle in fp64.  A score within the fp32 error
bound delta of a bin edge may land in the neighbouring bin, which moves at
most 2 |y - S| / N of ECE, so every ECE entry must agree within
    tol = sum over such near-edge samples of 2 |y - S| / N + delta + 2^-22
(2^-22: the fixed-point sums).  Position k of the oracle is scored with the
temperatures the GPU fitted at positions < k, so the check follows the GPU's
own sequence.  The GPU's choice must be a minimiser within the tolerances,
and identical to the oracle's wherever the oracle's best candidate leads by
more than them.  Mid-size cases check every candidate; the full-size set
(2^20 drafts, gamma 7, 64 candidates, 15 bins: the timed workload) checks
the chosen candidate, its neighbours and fixed samples one by one, and the
recovery of the head's known over-confidence.
"""
import numpy as np
import pytest
import torch

import synth
import semi_ar_draft_amd as dk
from oracle.sts_fit import ece as o_ece, labels as o_labels, candidate_scores

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    c = dk.Context(0)
    yield c
    c.close()


def run_gpu(ctx, logit, accept_len, grid, n_bins, stride_pad=0):
    N, G = logit.shape
    if stride_pad:
        wide = torch.zeros((N, G + stride_pad), dtype=torch.float32)
        wide[:, :G] = logit
        ld = wide.cuda()[:, :G]
    else:
        ld = logit.cuda()
    T, idx, ece = ctx.sts_fit(ld, accept_len.cuda(), grid.cuda(), n_bins)
    torch.cuda.synchronize()
    ctx.check()
    return T.cpu().numpy(), idx.cpu().numpy(), ece.cpu().numpy()


def delta_of(k):
    # fp32 error bound of a score: k scaled sigmoids (exponential, reciprocal,
    # products), a few ulps each
    return (6 * k + 4) * 2.0 ** -23


def oracle_entries(l, a, k, T_prev, temps, n_bins):
    """Oracle ECE of each candidate temperature at 1-based position k, and
    its tolerance."""
    S_all = candidate_scores(l, k, T_prev, temps)
    y = o_labels(a, k)
    N = y.size
    d = delta_of(k)
    out = []
    for S in S_all:
        e = o_ece(S, y, n_bins)
        if N == 0:
            out.append((e, 1e-15))
            continue
        x = S * n_bins
        r = np.round(x)
        near = (np.abs(x - r) < d * n_bins) & (r >= 1) & (r <= n_bins - 1)
        tol = float(np.sum(2.0 * np.abs(y[near] - S[near]))) / N + d + 2.0 ** -22
        out.append((e, tol))
    return out


def check_fit(l, a, grid, n_bins, T, idx, ece, cands=None):
    N, G = l.shape
    gr = grid.numpy().astype(np.float64)
    n_grid = gr.size
    assert ece.shape == (G, n_grid)
    for k in range(1, G + 1):
        # the GPU's own outputs agree with each other exactly
        assert 0 <= idx[k - 1] < n_grid
        assert T[k - 1] == grid.numpy()[idx[k - 1]]
        assert idx[k - 1] == int(np.argmin(ece[k - 1]))
        T_prev = T[:k - 1].astype(np.float64)
        gs = range(n_grid) if cands is None else sorted(set(cands(idx[k - 1], n_grid)))
        want, tol = {}, {}
        for g, (e, t) in zip(gs, oracle_entries(l, a, k, T_prev, gr[list(gs)], n_bins)):
            want[g], tol[g] = e, t
        for g in gs:
            assert abs(ece[k - 1, g] - want[g]) <= tol[g], (k, g, ece[k - 1, g], want[g], tol[g])
        c = int(idx[k - 1])
        assert c in want
        for g in gs:
            assert want[c] <= want[g] + tol[c] + tol[g], (k, c, g, want[c], want[g])
        if cands is None:
            best = min(gs, key=lambda g: (want[g], g))
            runner = [g for g in gs if g != best]
            if not runner or all(want[g] - want[best] > tol[g] + tol[best] for g in runner):
                assert c == best, (k, c, best)


CASES = [
    # name, N, gamma, grid (n, lo, step), n_bins, stride padding, seed
    ("N1000_g7_c64_b15", 1000, 7, (64, 0.5, 0.05), 15, 0, 1),
    ("N33333_g7_c64_b15_ragged", 33333, 7, (64, 0.5, 0.05), 15, 0, 2),
    ("N5000_g16_c130_b10", 5000, 16, (130, 0.3, 0.03), 10, 0, 3),
    ("N777_g3_c256_b16_maxcells", 777, 3, (256, 0.25, 0.02), 16, 0, 4),
    ("N64_g1_c1_b1", 64, 1, (1, 1.5, 0.0), 1, 0, 5),
    ("N1_g2_c7_b64", 1, 2, (7, 0.5, 0.5), 64, 0, 6),
    ("N20000_g32_c65_b15", 20000, 32, (65, 0.5, 0.05), 15, 0, 7),
    ("N4097_g5_c40_b12_strided", 4097, 5, (40, 0.6, 0.07), 12, 5, 8),
    # the remaining (candidate slices, table size) instantiations of the pass
    ("N999_g2_c64_b64_slices1_big", 999, 2, (64, 0.5, 0.05), 64, 0, 9),
    ("N2500_g6_c100_b20_slices2_big", 2500, 6, (100, 0.4, 0.03), 20, 0, 10),
    ("N1500_g3_c150_b6_slices3_small", 1500, 3, (150, 0.3, 0.02), 6, 0, 11),
    ("N3000_g4_c256_b4_slices4_small", 3000, 4, (256, 0.3, 0.012), 4, 0, 12),
]


@pytest.mark.parametrize("name,N,G,gspec,M,pad,seed", CASES, ids=[c[0] for c in CASES])
def test_sts_fit_matches_oracle(ctx, name, N, G, gspec, M, pad, seed):
    d = synth.sts_calibration_set(N, G, seed=100 + seed)
    grid = synth.sts_grid(*gspec)
    print(f"sts fit {name}", flush=True)
    T, idx, ece = run_gpu(ctx, d["logit"], d["accept_len"], grid, M, stride_pad=pad)
    check_fit(d["logit"].numpy(), d["accept_len"].numpy(), grid, M, T, idx, ece)


def test_sts_fit_empty_set(ctx):
    grid = synth.sts_grid(10, 0.5, 0.1)
    logit = torch.zeros((0, 4), dtype=torch.float32)
    a = torch.zeros(0, dtype=torch.int32)
    T, idx, ece = run_gpu(ctx, logit, a, grid, 15)
    assert list(idx) == [0, 0, 0, 0] and np.all(T == grid.numpy()[0]) and not ece.any()


def test_sts_fit_full_size_sampled_and_deterministic(ctx):
    N, G = 1 << 20, 7
    d = synth.sts_calibration_set(N, G, seed=2024)
    grid = synth.sts_grid()
    print(f"sts fit full size N={N} gamma={G} candidates={grid.numel()} bins=15", flush=True)
    T, idx, ece = run_gpu(ctx, d["logit"], d["accept_len"], grid, 15)
    T2, idx2, ece2 = run_gpu(ctx, d["logit"], d["accept_len"], grid, 15)
    assert np.array_equal(ece, ece2) and np.array_equal(idx, idx2) and np.array_equal(T, T2)
    sample = lambda c, n: [g for g in (c - 2, c - 1, c, c + 1, c + 2, 0, 10, 31, n - 1) if 0 <= g < n]
    check_fit(d["logit"].numpy(), d["accept_len"].numpy(), grid, 15, T, idx, ece, cands=sample)
    # sigmoid(l / T*) is the true acceptance probability: the fit lands near T*
    assert np.all(np.abs(T - d["true_T"].numpy()) <= 0.1 + 1e-6), (T, d["true_T"])


def test_sts_fit_flags_bad_candidates_and_lengths(ctx):
    d = synth.sts_calibration_set(300, 3, seed=9)
    grid = synth.sts_grid(8, 0.5, 0.25).clone()
    grid[3] = 0.0
    ld, ad = d["logit"].cuda(), d["accept_len"].cuda()
    ctx.sts_fit(ld, ad, grid.cuda(), 10)
    with pytest.raises(dk.DSparkError, match="candidate temperature"):
        ctx.check()
    bad = d["accept_len"].clone()
    bad[5], bad[7] = -1, 4
    ctx.sts_fit(ld, bad.cuda(), synth.sts_grid(8, 0.5, 0.25).cuda(), 10)
    with pytest.raises(dk.DSparkError, match="accepted length"):
        ctx.check()
    ctx.check()


def test_sts_fit_rejects_bad_shapes(ctx):
    d = synth.sts_calibration_set(10, 3, seed=1)
    ld, ad = d["logit"].cuda(), d["accept_len"].cuda()
    with pytest.raises(dk.DSparkError, match="n_grid"):
        ctx.sts_fit(ld, ad, synth.sts_grid(257).cuda(), 10)
    with pytest.raises(dk.DSparkError, match="n_grid"):
        ctx.sts_fit(ld, ad, synth.sts_grid(100).cuda(), 41)
    with pytest.raises(dk.DSparkError, match="n_grid"):
        ctx.sts_fit(ld, ad, synth.sts_grid(10).cuda(), 0)
    wide = torch.zeros((10, 40), dtype=torch.float32, device="cuda")
    with pytest.raises(dk.DSparkError, match="gamma"):
        ctx.sts_fit(wide, ad, synth.sts_grid(10).cuda(), 10)


def test_sts_fit_graph_capture_replays(ctx):
    # the per-pass counter and sums are left zeroed by every pass, so a
    # captured fit replays to the eager result, also with eager fits of
    # another shape in between
    d = synth.sts_calibration_set(20000, 5, seed=31)
    e = synth.sts_calibration_set(3000, 7, seed=32)
    grid = synth.sts_grid(48, 0.6, 0.05).cuda()
    l, a = d["logit"].cuda(), d["accept_len"].cuda()
    l2, a2 = e["logit"].cuda(), e["accept_len"].cuda()
    out = (torch.empty(5, device="cuda"), torch.empty(5, dtype=torch.int32, device="cuda"),
           torch.empty((5, 48), dtype=torch.float64, device="cuda"))
    ctx.sts_fit(l, a, grid, 15, out=out)
    ctx.check()
    ref = [x.clone() for x in out]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ctx.sts_fit(l, a, grid, 15, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    print("capturing a temperature fit", flush=True)
    with torch.cuda.graph(g, stream=s):
        ctx.sts_fit(l, a, grid, 15, out=out)
    torch.cuda.synchronize()
    for rep in range(3):
        for x in out:
            x.zero_()
        ctx.sts_fit(l2, a2, grid, 12)                   # other eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, want, got in zip(("T", "index", "ece"), ref, out):
            assert torch.equal(want, got), f"replay {rep}: {name}"
    ctx.check()


def test_sts_fit_two_contexts_on_two_streams():
    d1 = synth.sts_calibration_set(50000, 7, seed=41)
    d2 = synth.sts_calibration_set(40000, 4, seed=42)
    grid = synth.sts_grid().cuda()
    c1, c2 = dk.Context(0), dk.Context(0)
    try:
        i1 = (d1["logit"].cuda(), d1["accept_len"].cuda())
        i2 = (d2["logit"].cuda(), d2["accept_len"].cuda())
        r1 = [x.cpu() for x in c1.sts_fit(*i1, grid, 15)]
        r2 = [x.cpu() for x in c2.sts_fit(*i2, grid, 10)]
        torch.cuda.synchronize()
        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        s1.wait_stream(torch.cuda.current_stream())
        s2.wait_stream(torch.cuda.current_stream())
        print("two temperature fits on two streams", flush=True)
        with torch.cuda.stream(s1):
            o1 = c1.sts_fit(*i1, grid, 15, stream=s1)
        with torch.cuda.stream(s2):
            o2 = c2.sts_fit(*i2, grid, 10, stream=s2)
        s1.synchronize()
        s2.synchronize()
        c1.check(s1)
        c2.check(s2)
        for want, got in zip(r1, o1):
            assert torch.equal(want, got.cpu())
        for want, got in zip(r2, o2):
            assert torch.equal(want, got.cpu())
    finally:
        c1.close()
        c2.close()


def test_sts_fit_rejects_sample_counts_from_two_to_the_33():
    """N < 2^33 keeps every cell's fixed-point sum (2^-30 units) below 2^63;
    the limit is checked on the host before anything is enqueued (so the
    small buffers passed here are never read)."""
    c = dk.Context(0)
    try:
        d = synth.sts_calibration_set(10, 3, seed=1)
        ld, ad = d["logit"].cuda(), d["accept_len"].cuda()
        grid = synth.sts_grid(8).cuda()
        T = torch.empty((3,), dtype=torch.float32, device="cuda")
        idx = torch.empty((3,), dtype=torch.int32, device="cuda")
        ece = torch.empty((3, 8), dtype=torch.float64, device="cuda")
        for N in (1 << 33, 1 << 40):
            rc = c.lib.dspark_sts_fit(c._h, None, N, 3, ld.data_ptr(), 3, ad.data_ptr(), grid.data_ptr(), 8, 10,
                                      T.data_ptr(), idx.data_ptr(), ece.data_ptr())
            assert rc == dk.DSPARK_EINVAL
            assert b"2^33" in c.lib.dspark_last_error(c._h)
    finally:
        c.close()
