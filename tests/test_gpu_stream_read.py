"""GPU: the streaming-read calibration (dspark_stream_read) sums what it
reads: against a float64 sum on the host for sizes with and without a
ragged tail of fewer than four floats, an empty input, bit-identical on
repeated calls; a misaligned pointer is refused before anything runs."""
import numpy as np
import pytest
import torch

import semi_ar_draft_amd as dk

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    c = dk.Context(0)
    yield c
    c.close()


@pytest.mark.parametrize("n", [0, 1, 3, 4, 5, 1023, 65536, 256 * 2048 * 4 + 7, (1 << 24) + 1])
def test_sum_matches_the_host(ctx, n):
    g = torch.Generator().manual_seed(n + 11)
    x = torch.rand(n, generator=g, dtype=torch.float32) - 0.25
    print(f"stream read n={n}", flush=True)
    xd = x.cuda()
    a = ctx.stream_read(xd).cpu().item()
    b = ctx.stream_read(xd).cpu().item()
    ctx.check()
    want = float(x.double().sum())
    # float32 accumulation: per-thread chains, then fixed trees
    tol = 1e-6 + 1e-5 * float(x.double().abs().sum())
    assert abs(a - want) <= tol, (a, want)
    assert np.float32(a).tobytes() == np.float32(b).tobytes()


def test_misaligned_pointer_is_refused(ctx):
    x = torch.ones(1025, dtype=torch.float32, device="cuda")
    with pytest.raises(dk.DSparkError):
        ctx.stream_read(x[1:])
    ctx.check()


def test_host_checks_through_the_c_abi(ctx):
    lib = ctx.lib
    out = torch.empty((1,), dtype=torch.float32, device="cuda")
    x = torch.ones(64, dtype=torch.float32, device="cuda")
    assert lib.dspark_stream_read(ctx._h, None, x.data_ptr(), -1, out.data_ptr()) == dk.DSPARK_EINVAL
    assert lib.dspark_stream_read(ctx._h, None, x.data_ptr(), 64, None) == dk.DSPARK_EINVAL
    assert lib.dspark_stream_read(ctx._h, None, None, 64, out.data_ptr()) == dk.DSPARK_EINVAL
    assert lib.dspark_stream_read(None, None, x.data_ptr(), 64, out.data_ptr()) == dk.DSPARK_EINVAL
    # n = 0 with no buffer writes 0
    out.fill_(7.0)
    assert lib.dspark_stream_read(ctx._h, None, None, 0, out.data_ptr()) == dk.DSPARK_OK
    ctx.check()
    assert out.item() == 0.0
