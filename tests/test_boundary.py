"""C-ABI boundary checks that need no GPU."""
import ctypes
import os
import re
import subprocess

import pytest

import semi_ar_draft_amd as dk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dspark.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dspark_\w+)\s*\(", src)))


def test_header_declares_the_four_calls_and_helpers():
    names = _declared()
    for n in ("dspark_draft_markov", "dspark_confidence", "dspark_schedule", "dspark_verify",
              "dspark_create", "dspark_destroy", "dspark_last_error", "dspark_check",
              "dspark_version"):
        assert n in names
    assert set(names) == set(dk.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = dk.load_library()
    for n in _declared():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", dk.LIB_PATH], capture_output=True, text=True)
    exported = set(re.findall(r"\bT (dspark_\w+)", out.stdout))
    assert set(_declared()) <= exported


def test_library_embeds_gfx950_device_code():
    # the offload bundle of our own build names its target triple
    blob = open(dk.LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob


def test_timing_classes_match_the_header():
    import re
    with open(HEADER) as f:
        h = f.read()
    n = int(re.search(r"DSPARK_K_COUNT\s*=\s*(\d+)", h).group(1))
    assert n == len(dk.KERNEL_CLASSES)
    ids = [int(v) for v in re.findall(r"DSPARK_K_[A-Z_]+\s*=\s*(\d+),", h)]
    assert ids == list(range(n))


def test_version():
    assert dk.load_library().dspark_version() == 101


def test_null_context_is_rejected_everywhere():
    lib = dk.load_library()
    assert lib.dspark_create(None, 0) == dk.DSPARK_EINVAL
    assert lib.dspark_check(None, None) == dk.DSPARK_EINVAL
    assert lib.dspark_last_error(None) == b"null context"
    lib.dspark_destroy(None)
    assert lib.dspark_draft_markov(None, None, 1, 1, 16, 32, 1, None, 16, 16, None, None, None,
                                   None, 0.0, 0, None, None, None) == dk.DSPARK_EINVAL
    assert lib.dspark_confidence(None, None, 1, 1, 1, 8, 8, None, None, None, None, None, 0.0,
                                 None, None, None) == dk.DSPARK_EINVAL
    assert lib.dspark_schedule(None, None, 1, 1, None, None, 1, None, None, None) == dk.DSPARK_EINVAL
    assert lib.dspark_schedule_async(None, None, 1, 1, None, None, None, 1, None, None, None) == dk.DSPARK_EINVAL
    assert lib.dspark_verify(None, None, 1, 1, 16, 32, 1, None, 32, 16, None, 16, 16, None, None,
                             None, None, None, None, None, None, None, 0.0, 0, None, None) == dk.DSPARK_EINVAL
    assert lib.dspark_verify_packed(None, None, 1, 1, 16, 32, 1, None, 16, None, 1, None, 16, 16, None, None,
                                    None, None, None, None, None, None, None, 0.0, 0, None, None) == dk.DSPARK_EINVAL
    assert lib.dspark_accept_prob(None, None, 1, 1, 16, 32, 1, None, 16, 16, None, 16, 16, None, None, None,
                                  None, None, None, 1.0, None) == dk.DSPARK_EINVAL
    assert lib.dspark_draft_rnn(None, None, 1, 1, 16, 32, 1, None, 16, 16, None, None, None, None, None,
                                None, None, None, 0.0, 0, None, None, None, None) == dk.DSPARK_EINVAL
    assert lib.dspark_sts_fit(None, None, 1, 1, None, 1, None, None, 1, 1, None, None, None) == dk.DSPARK_EINVAL
    assert lib.dspark_stream_read(None, None, None, 0, None) == dk.DSPARK_EINVAL
    assert lib.dspark_draft_markov_static(None, None, 1, 1, 16, 32, 1, None, 16, 16, None, None, None,
                                          None, 0.0, 0, None, None, None) == dk.DSPARK_EINVAL
    assert lib.dspark_draft_markov_conf(None, None, 1, 1, 16, 32, 1, None, 16, 16, None, None, None, None, 0.0, 0,
                                        8, 8, None, None, None, 0.0, None, None, None, None, None,
                                        None) == dk.DSPARK_EINVAL


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU device node is present")
def test_create_fails_cleanly_without_a_device():
    lib = dk.load_library()
    h = ctypes.c_void_p(12345)
    rc = lib.dspark_create(ctypes.byref(h), 0)
    assert rc == dk.DSPARK_EHIP
    assert h.value is None


def test_binding_refuses_missing_library(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        dk.load_library(str(tmp_path / "missing.so"))
