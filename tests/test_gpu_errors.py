"""Argument checks and device error reporting through the C ABI (GPU)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import semi_ar_draft_amd as dk

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    c = dk.Context(0)
    yield c
    c.close()


@pytest.fixture(scope="module")
def small():
    wl = synth.WORKLOADS["sample"].with_(B=8, V=512, r=32, d_h=16, d_e=16)
    inp = synth.make_inputs(wl, seed=3)
    return wl, {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def _code(excinfo):
    return excinfo.value.code


def test_shape_and_pointer_checks(ctx, small):
    wl, d = small
    G = wl.gamma
    with pytest.raises(dk.DSparkError) as e:   # V not a multiple of 16
        ctx.draft_markov(d["U"][:, :, :500], d["W1"][:500], d["W2"][:500], d["anchor"], None, 1.0, 0, G)
    assert _code(e) == dk.DSPARK_EINVAL
    with pytest.raises(dk.DSparkError) as e:   # unsupported rank
        ctx.draft_markov(d["U"], d["W1"][:, :16].contiguous(), d["W2"][:, :16].contiguous(),
                         d["anchor"], None, 1.0, 0, G)
    assert _code(e) == dk.DSPARK_EINVAL
    with pytest.raises(dk.DSparkError) as e:   # negative temperature
        ctx.draft_markov(d["U"], d["W1"], d["W2"], d["anchor"], None, -1.0, 0, G)
    assert _code(e) == dk.DSPARK_EINVAL
    with pytest.raises(ValueError):            # gamma beyond the rows of U (binding check)
        ctx.draft_markov(d["U"], d["W1"], d["W2"], d["anchor"], None, 1.0, 0, G + 2)
    # the library's own stride check for the same mistake
    lib = dk.load_library()
    B, R, V = d["U"].shape
    out = torch.empty((B, G + 2), dtype=torch.int32, device="cuda")
    outf = torch.empty((B, G + 2), device="cuda")
    rc = lib.dspark_draft_markov(ctx._h, None, B, G + 2, V, wl.r, dk.DSPARK_BF16, d["U"].data_ptr(),
                                 R * V, V, d["W1"].data_ptr(), d["W2"].data_ptr(), d["anchor"].data_ptr(),
                                 None, 1.0, 0, out.data_ptr(), outf.data_ptr(), outf.data_ptr())
    assert rc == dk.DSPARK_EINVAL
    with pytest.raises(dk.DSparkError) as e:   # misaligned logits
        Uo = torch.empty(d["U"].numel() + 1, device="cuda")[1:].view_as(d["U"])
        ctx.draft_markov(Uo, d["W1"], d["W2"], d["anchor"], None, 1.0, 0, G)
    assert _code(e) == dk.DSPARK_EINVAL
    with pytest.raises(dk.DSparkError) as e:   # too many scheduler keys
        ctx.schedule(torch.rand(1024, 5, device="cuda"), torch.ones(4096, device="cuda"))
    assert _code(e) == dk.DSPARK_EINVAL
    with pytest.raises(dk.DSparkError) as e:   # table shorter than the batch
        ctx.schedule(torch.rand(64, 5, device="cuda"), torch.ones(32, device="cuda"))
    assert _code(e) == dk.DSPARK_EINVAL
    with pytest.raises(dk.DSparkError) as e:   # hidden width not a multiple of 8
        tok = torch.zeros((wl.B, G), dtype=torch.int32, device="cuda")
        h = torch.zeros((wl.B, G, 12), dtype=torch.bfloat16, device="cuda")
        wc = torch.zeros(12 + wl.d_e, dtype=torch.bfloat16, device="cuda")
        ctx.confidence(h, d["E"], d["anchor"], tok, wc, 0.0)
    assert _code(e) == dk.DSPARK_EINVAL
    ctx.check()   # nothing was enqueued by the refused calls


def test_out_of_range_token_is_flagged(ctx, small):
    wl, d = small
    bad = d["anchor"].clone()
    bad[3] = wl.V + 5
    ctx.draft_markov(d["U"], d["W1"], d["W2"], bad, None, 1.0, 0, wl.gamma)
    with pytest.raises(dk.DSparkError) as e:
        ctx.check()
    assert _code(e) == dk.DSPARK_EDEVICE
    ctx.check()   # the flag was cleared


def test_out_of_range_verify_length_is_flagged(ctx, small):
    wl, d = small
    tok, lse, ytok = ctx.draft_markov(d["U"], d["W1"], d["W2"], d["anchor"], None, 1.0, 0, wl.gamma)
    K = torch.full((wl.B,), wl.gamma, dtype=torch.int32, device="cuda")
    K[2] = wl.gamma + 3
    ctx.verify(d["target"], d["U"], d["W1"], d["W2"], d["anchor"], tok, lse, ytok, K, None, 1.0, 0)
    with pytest.raises(dk.DSparkError) as e:
        ctx.check()
    assert _code(e) == dk.DSPARK_EDEVICE


def test_smallest_vocabulary_single_tile(ctx):
    wl = synth.WORKLOADS["sample"].with_(B=3, gamma=4, V=16, r=32, conf=False)
    inp = synth.make_inputs(wl, seed=8)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    tok, lse, ytok = ctx.draft_markov(d["U"], d["W1"], d["W2"], d["anchor"], d["req_ids"], 1.0, 4, 4)
    acc, out = ctx.verify(d["target"], d["U"], d["W1"], d["W2"], d["anchor"], tok, lse, ytok, None,
                          d["req_ids"], 1.0, 4)
    ctx.check()
    od = oracle.draft_markov(inp["U"], inp["W1"], inp["W2"], inp["anchor"], inp["req_ids"], 1.0, 4, 4)
    if od.margin.min() > 1e-4:
        assert np.array_equal(tok.cpu().numpy(), od.tokens)
        ov = oracle.verify(inp["target"], od.tokens, od.lse, od.ytok, inp["U"], inp["W1"], inp["W2"],
                           inp["anchor"], None, inp["req_ids"], 1.0, 4, 4)
        if ov.margin.min() > 1e-4 and ov.final_margin.min() > 1e-4:
            assert np.array_equal(acc.cpu().numpy(), ov.accept_len)
            assert np.array_equal(out.cpu().numpy(), ov.out_tokens)


def test_empty_batch_and_gamma_out_of_range_are_refused(ctx, small):
    """An empty batch (B = 0) and gamma outside 1..32 are argument errors of
    every call, refused on the host before anything is enqueued."""
    wl, d = small
    lib = dk.load_library()
    B, R, V = d["U"].shape
    G = wl.gamma
    i32 = torch.zeros((B, 33), dtype=torch.int32, device="cuda")
    f32 = torch.zeros((B, 33), device="cuda")
    draft_args = lambda b, g: (ctx._h, None, b, g, V, wl.r, dk.DSPARK_BF16, d["U"].data_ptr(), R * V, V,
                               d["W1"].data_ptr(), d["W2"].data_ptr(), d["anchor"].data_ptr(), None, 1.0, 0)
    for b, g in ((0, G), (B, 0), (B, 33), (-1, G)):
        assert lib.dspark_draft_markov(*draft_args(b, g), i32.data_ptr(), f32.data_ptr(),
                                       f32.data_ptr()) == dk.DSPARK_EINVAL, (b, g)
        assert lib.dspark_draft_markov_static(*draft_args(b, g), i32.data_ptr(), f32.data_ptr(),
                                              f32.data_ptr()) == dk.DSPARK_EINVAL, (b, g)
    h = torch.zeros((B, G, 16), dtype=torch.bfloat16, device="cuda")
    E = torch.zeros((V, 16), dtype=torch.bfloat16, device="cuda")
    wc = torch.zeros(32, dtype=torch.bfloat16, device="cuda")
    for b, g in ((0, G), (B, 0), (B, 33)):
        assert lib.dspark_confidence(ctx._h, None, b, g, V, 16, 16, h.data_ptr(), E.data_ptr(),
                                     d["anchor"].data_ptr(), i32.data_ptr(), wc.data_ptr(), 0.0, None,
                                     f32.data_ptr(), f32.data_ptr()) == dk.DSPARK_EINVAL, (b, g)
        assert lib.dspark_draft_markov_conf(*draft_args(b, g), 16, 16, h.data_ptr(), E.data_ptr(),
                                            wc.data_ptr(), 0.0, None, i32.data_ptr(), f32.data_ptr(),
                                            f32.data_ptr(), f32.data_ptr(), f32.data_ptr()) == dk.DSPARK_EINVAL
        assert lib.dspark_verify(ctx._h, None, b, g, V, wl.r, dk.DSPARK_BF16, d["target"].data_ptr(),
                                 d["target"].stride(0), d["target"].stride(1), d["U"].data_ptr(), R * V, V,
                                 d["W1"].data_ptr(), d["W2"].data_ptr(), d["anchor"].data_ptr(),
                                 i32.data_ptr(), f32.data_ptr(), f32.data_ptr(), None, None, None, 1.0, 0,
                                 i32.data_ptr(), i32.data_ptr()) == dk.DSPARK_EINVAL, (b, g)
    sps = torch.ones(4096, device="cuda")
    K = torch.zeros(B, dtype=torch.int32, device="cuda")
    n = torch.zeros(1, dtype=torch.int32, device="cuda")
    th = torch.zeros(1, dtype=torch.float64, device="cuda")
    for b, g in ((0, G), (B, 0), (B, 33)):
        assert lib.dspark_schedule(ctx._h, None, b, g, f32.data_ptr(), sps.data_ptr(), 4096, K.data_ptr(),
                                   n.data_ptr(), th.data_ptr()) == dk.DSPARK_EINVAL, (b, g)
    ctx.check()   # nothing was enqueued
