"""Python binding of libdspark: argument marshalling only.

Every computation happens in the HIP kernels of ``libdspark.so``; this module
checks tensor placement, dtypes and layouts, allocates outputs with PyTorch
(device memory is PyTorch's), and passes raw pointers, sizes and the current
HIP stream across the C ABI declared in ``include/dspark.h``.  There is no
fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdspark.so")

DSPARK_OK, DSPARK_EINVAL, DSPARK_EHIP, DSPARK_ENOMEM, DSPARK_EDEVICE = 0, 1, 2, 3, 4
DSPARK_F32, DSPARK_BF16 = 0, 1

EXPORTS = (
    "dspark_version", "dspark_create", "dspark_destroy", "dspark_last_error", "dspark_check",
    "dspark_draft_markov", "dspark_draft_markov_static", "dspark_draft_markov_conf", "dspark_draft_rnn",
    "dspark_confidence", "dspark_schedule", "dspark_schedule_async", "dspark_verify",
    "dspark_verify_packed", "dspark_accept_prob", "dspark_sts_fit", "dspark_stream_read",
    "dspark_timing_enable", "dspark_timing_read",
)
KERNEL_CLASSES = ("draft_sweep", "draft_combine", "confidence", "survival", "schedule",
                  "verify_rows", "verify_decide", "resid_sweep", "resid_combine", "gru", "diag", "sts_fit",
                  "draft_chain", "verify_chain", "conf_merge")

_lib = None
_vp, _i32, _i64, _u64, _f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float


class DSparkError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libdspark error {code}: {msg}")
        self.code = code


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libdspark.so (built in-tree by ``semi_ar_draft_amd.build``)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built; run `python -m semi_ar_draft_amd.build`")
    lib = ctypes.CDLL(p)
    lib.dspark_version.restype = _i32
    lib.dspark_version.argtypes = []
    lib.dspark_create.restype = _i32
    lib.dspark_create.argtypes = [ctypes.POINTER(_vp), _i32]
    lib.dspark_destroy.restype = None
    lib.dspark_destroy.argtypes = [_vp]
    lib.dspark_last_error.restype = ctypes.c_char_p
    lib.dspark_last_error.argtypes = [_vp]
    lib.dspark_check.restype = _i32
    lib.dspark_check.argtypes = [_vp, _vp]
    lib.dspark_timing_enable.restype = _i32
    lib.dspark_timing_enable.argtypes = [_vp, _i32]
    lib.dspark_timing_read.restype = _i32
    lib.dspark_timing_read.argtypes = [_vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i32)]
    lib.dspark_draft_markov.restype = _i32
    lib.dspark_draft_markov.argtypes = [
        _vp, _vp, _i32, _i32, _i32, _i32, _i32,
        _vp, _i64, _i64, _vp, _vp, _vp, _vp, _f32, _u64, _vp, _vp, _vp]
    lib.dspark_draft_markov_static.restype = _i32
    lib.dspark_draft_markov_static.argtypes = lib.dspark_draft_markov.argtypes
    lib.dspark_draft_markov_conf.restype = _i32
    lib.dspark_draft_markov_conf.argtypes = [
        _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _f32, _u64,
        _i32, _i32, _vp, _vp, _vp, _f32, _vp, _vp, _vp, _vp, _vp, _vp]
    lib.dspark_draft_rnn.restype = _i32
    lib.dspark_draft_rnn.argtypes = [
        _vp, _vp, _i32, _i32, _i32, _i32, _i32,
        _vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _u64, _vp, _vp, _vp, _vp]
    lib.dspark_confidence.restype = _i32
    lib.dspark_confidence.argtypes = [
        _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _vp, _vp]
    lib.dspark_schedule.restype = _i32
    lib.dspark_schedule.argtypes = [_vp, _vp, _i32, _i32, _vp, _vp, _i32, _vp, _vp, _vp]
    lib.dspark_schedule_async.restype = _i32
    lib.dspark_schedule_async.argtypes = [_vp, _vp, _i32, _i32, _vp, _vp, _vp, _i32, _vp, _vp, _vp]
    lib.dspark_verify.restype = _i32
    lib.dspark_verify.argtypes = [
        _vp, _vp, _i32, _i32, _i32, _i32, _i32,
        _vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _vp,
        _vp, _vp, _vp, _vp, _vp, _vp, _f32, _u64, _vp, _vp]
    lib.dspark_verify_packed.restype = _i32
    lib.dspark_verify_packed.argtypes = [
        _vp, _vp, _i32, _i32, _i32, _i32, _i32,
        _vp, _i64, _vp, _i32, _vp, _i64, _i64, _vp, _vp, _vp,
        _vp, _vp, _vp, _vp, _vp, _vp, _f32, _u64, _vp, _vp]
    lib.dspark_accept_prob.restype = _i32
    lib.dspark_accept_prob.argtypes = [
        _vp, _vp, _i32, _i32, _i32, _i32, _i32,
        _vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _vp]
    lib.dspark_sts_fit.restype = _i32
    lib.dspark_sts_fit.argtypes = [
        _vp, _vp, _i64, _i32, _vp, _i64, _vp, _vp, _i32, _i32, _vp, _vp, _vp]
    lib.dspark_stream_read.restype = _i32
    lib.dspark_stream_read.argtypes = [_vp, _vp, _vp, _i64, _vp]
    if path is None:
        _lib = lib
    return lib


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _wdtype(w: torch.Tensor) -> int:
    if w.dtype == torch.bfloat16:
        return DSPARK_BF16
    if w.dtype == torch.float32:
        return DSPARK_F32
    raise TypeError(f"Markov weights must be bf16 or fp32, got {w.dtype}")


def _need(t: torch.Tensor, name: str, dtype, device, ndim=None, contiguous=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _len(t: torch.Tensor, n: int, name: str):
    if t.shape[0] != n:
        raise ValueError(f"{name} must have {n} entries, got {t.shape[0]}")


def _logits3(t: torch.Tensor, name: str, device):
    _need(t, name, torch.float32, device, 3, contiguous=False)
    if t.stride(2) != 1:
        raise ValueError(f"{name} rows must be contiguous over the vocabulary")
    return t.stride(0), t.stride(1)


class Context:
    """One libdspark context on one GPU (owns workspace, graph cache, error flag)."""

    def __init__(self, device: int = 0):
        self.lib = load_library()
        self.device = torch.device("cuda", device)
        h = _vp()
        rc = self.lib.dspark_create(ctypes.byref(h), device)
        if rc != DSPARK_OK:
            raise DSparkError(rc, f"dspark_create(device={device}) failed")
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            self.lib.dspark_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def _rc(self, rc: int):
        if rc != DSPARK_OK:
            raise DSparkError(rc, self.lib.dspark_last_error(self._h).decode())

    def check(self, stream=None):
        """Synchronise the stream and raise if a kernel flagged bad data."""
        self._rc(self.lib.dspark_check(self._h, _stream(self.device, stream)))

    # -- kernel timing ------------------------------------------------------
    def timing(self, enable: bool):
        self._rc(self.lib.dspark_timing_enable(self._h, 1 if enable else 0))

    def read_timing(self) -> dict:
        """{kernel class: (total ms, launches)} since the last read."""
        n = len(KERNEL_CLASSES)
        ms = (ctypes.c_double * n)()
        cnt = (_i32 * n)()
        self._rc(self.lib.dspark_timing_read(self._h, ms, cnt))
        return {name: (ms[i], cnt[i]) for i, name in enumerate(KERNEL_CLASSES)}

    # -- dspark_draft_markov ------------------------------------------------
    def draft_markov(self, U, W1, W2, anchor, req_ids, temperature: float, seed: int, gamma: int,
                     out=None, stream=None, static: bool = False):
        """dspark_draft_markov, or with static=True dspark_draft_markov_static
        (the allocation-free variant: its scratch is a fixed per-GPU array)."""
        dev = self.device
        sb, sk = _logits3(U, "U", dev)
        B, rows, V = U.shape
        if rows < gamma:
            raise ValueError(f"U has {rows} positions, gamma is {gamma}")
        _need(W1, "W1", None, dev, 2)
        _need(W2, "W2", W1.dtype, dev, 2)
        r = W1.shape[1]
        if W1.shape != (V, r) or W2.shape != (V, r):
            raise ValueError("W1 and W2 must both be [V][r]")
        _need(anchor, "anchor", torch.int32, dev, 1)
        _len(anchor, B, "anchor")
        if req_ids is not None:
            _need(req_ids, "req_ids", torch.int32, dev, 1)
            _len(req_ids, B, "req_ids")
        if out is None:
            out = (torch.empty((B, gamma), dtype=torch.int32, device=dev),
                   torch.empty((B, gamma), dtype=torch.float32, device=dev),
                   torch.empty((B, gamma), dtype=torch.float32, device=dev))
        tokens, lse, ytok = out
        fn = self.lib.dspark_draft_markov_static if static else self.lib.dspark_draft_markov
        self._rc(fn(
            self._h, _stream(dev, stream), B, gamma, V, r, _wdtype(W1),
            U.data_ptr(), sb, sk, W1.data_ptr(), W2.data_ptr(), anchor.data_ptr(),
            _ptr(req_ids), float(temperature), int(seed) & 0xFFFFFFFFFFFFFFFF,
            tokens.data_ptr(), lse.data_ptr(), ytok.data_ptr()))
        return tokens, lse, ytok

    # -- dspark_draft_markov_conf ---------------------------------------------
    def draft_markov_conf(self, U, W1, W2, anchor, req_ids, temperature: float, seed: int, gamma: int,
                          h, E, wc, bc: float, sts_T=None, out=None, stream=None):
        """dspark_draft_markov then dspark_confidence on its tokens, with the
        draft's merge done by the confidence launch.  Returns tokens, lse,
        ytok, conf, surv."""
        dev = self.device
        sb, sk = _logits3(U, "U", dev)
        B, rows, V = U.shape
        if rows < gamma:
            raise ValueError(f"U has {rows} positions, gamma is {gamma}")
        _need(W1, "W1", None, dev, 2)
        _need(W2, "W2", W1.dtype, dev, 2)
        r = W1.shape[1]
        if W1.shape != (V, r) or W2.shape != (V, r):
            raise ValueError("W1 and W2 must both be [V][r]")
        _need(anchor, "anchor", torch.int32, dev, 1)
        _len(anchor, B, "anchor")
        if req_ids is not None:
            _need(req_ids, "req_ids", torch.int32, dev, 1)
            _len(req_ids, B, "req_ids")
        _need(h, "h", torch.bfloat16, dev, 3)
        _need(E, "E", torch.bfloat16, dev, 2)
        _need(wc, "wc", torch.bfloat16, dev, 1)
        if tuple(h.shape[:2]) != (B, gamma):
            raise ValueError("h must be [B][gamma][d_h]")
        d_h = h.shape[2]
        if E.shape[0] != V:
            raise ValueError("E must be [V][d_e]")
        d_e = E.shape[1]
        if wc.shape[0] != d_h + d_e:
            raise ValueError("wc must have d_h + d_e entries")
        if sts_T is not None:
            _need(sts_T, "sts_T", torch.float32, dev, 1)
            _len(sts_T, gamma, "sts_T")
        if out is None:
            out = (torch.empty((B, gamma), dtype=torch.int32, device=dev),
                   torch.empty((B, gamma), dtype=torch.float32, device=dev),
                   torch.empty((B, gamma), dtype=torch.float32, device=dev),
                   torch.empty((B, gamma), dtype=torch.float32, device=dev),
                   torch.empty((B, gamma), dtype=torch.float32, device=dev))
        tokens, lse, ytok, conf, surv = out
        self._rc(self.lib.dspark_draft_markov_conf(
            self._h, _stream(dev, stream), B, gamma, V, r, _wdtype(W1),
            U.data_ptr(), sb, sk, W1.data_ptr(), W2.data_ptr(), anchor.data_ptr(),
            _ptr(req_ids), float(temperature), int(seed) & 0xFFFFFFFFFFFFFFFF,
            d_h, d_e, h.data_ptr(), E.data_ptr(), wc.data_ptr(), float(bc), _ptr(sts_T),
            tokens.data_ptr(), lse.data_ptr(), ytok.data_ptr(), conf.data_ptr(), surv.data_ptr()))
        return tokens, lse, ytok, conf, surv

    # -- dspark_draft_rnn ------------------------------------------------------
    def draft_rnn(self, U, W1, W2, gru: dict, req_ids, temperature: float, seed: int, gamma: int,
                  out=None, stream=None):
        """GRU head; ``gru`` holds W_ih, W_hh [3r][r], b_ih, b_hh [3r], s0 [r] (bf16).
        Returns tokens, lse, ytok and the fp32 states [gamma][B][r]."""
        dev = self.device
        sb, sk = _logits3(U, "U", dev)
        B, rows, V = U.shape
        if rows < gamma:
            raise ValueError(f"U has {rows} positions, gamma is {gamma}")
        _need(W1, "W1", None, dev, 2)
        _need(W2, "W2", W1.dtype, dev, 2)
        r = W1.shape[1]
        if W1.shape != (V, r) or W2.shape != (V, r):
            raise ValueError("W1 and W2 must both be [V][r]")
        for nm, shape in (("W_ih", (3 * r, r)), ("W_hh", (3 * r, r)), ("b_ih", (3 * r,)),
                          ("b_hh", (3 * r,)), ("s0", (r,))):
            _need(gru[nm], nm, torch.bfloat16, dev, len(shape))
            if tuple(gru[nm].shape) != shape:
                raise ValueError(f"{nm} must be {list(shape)}")
        if req_ids is not None:
            _need(req_ids, "req_ids", torch.int32, dev, 1)
            _len(req_ids, B, "req_ids")
        if out is None:
            out = (torch.empty((B, gamma), dtype=torch.int32, device=dev),
                   torch.empty((B, gamma), dtype=torch.float32, device=dev),
                   torch.empty((B, gamma), dtype=torch.float32, device=dev),
                   torch.empty((gamma, B, r), dtype=torch.float32, device=dev))
        tokens, lse, ytok, states = out
        self._rc(self.lib.dspark_draft_rnn(
            self._h, _stream(dev, stream), B, gamma, V, r, _wdtype(W1),
            U.data_ptr(), sb, sk, W1.data_ptr(), W2.data_ptr(), gru["W_ih"].data_ptr(),
            gru["W_hh"].data_ptr(), gru["b_ih"].data_ptr(), gru["b_hh"].data_ptr(), gru["s0"].data_ptr(),
            _ptr(req_ids), float(temperature), int(seed) & 0xFFFFFFFFFFFFFFFF,
            tokens.data_ptr(), lse.data_ptr(), ytok.data_ptr(), states.data_ptr()))
        return tokens, lse, ytok, states

    # -- dspark_confidence ----------------------------------------------------
    def confidence(self, h, E, anchor, tokens, wc, bc: float, sts_T=None, out=None, stream=None):
        dev = self.device
        _need(h, "h", torch.bfloat16, dev, 3)
        _need(E, "E", torch.bfloat16, dev, 2)
        _need(wc, "wc", torch.bfloat16, dev, 1)
        _need(anchor, "anchor", torch.int32, dev, 1)
        _need(tokens, "tokens", torch.int32, dev, 2)
        B, gamma, d_h = h.shape
        V, d_e = E.shape
        if wc.shape[0] != d_h + d_e:
            raise ValueError("wc must have d_h + d_e entries")
        _len(anchor, B, "anchor")
        if tuple(tokens.shape) != (B, gamma):
            raise ValueError("tokens must be [B][gamma]")
        if sts_T is not None:
            _need(sts_T, "sts_T", torch.float32, dev, 1)
            _len(sts_T, gamma, "sts_T")
        if out is None:
            out = (torch.empty((B, gamma), dtype=torch.float32, device=dev),
                   torch.empty((B, gamma), dtype=torch.float32, device=dev))
        conf, surv = out
        self._rc(self.lib.dspark_confidence(
            self._h, _stream(dev, stream), B, gamma, V, d_h, d_e, h.data_ptr(), E.data_ptr(),
            anchor.data_ptr(), tokens.data_ptr(), wc.data_ptr(), float(bc), _ptr(sts_T),
            conf.data_ptr(), surv.data_ptr()))
        return conf, surv

    # -- dspark_schedule --------------------------------------------------------
    def schedule(self, surv, sps, out=None, stream=None):
        dev = self.device
        _need(surv, "surv", torch.float32, dev, 2)
        _need(sps, "sps", torch.float32, dev, 1)
        B, gamma = surv.shape
        if out is None:
            out = (torch.empty((B,), dtype=torch.int32, device=dev),
                   torch.empty((1,), dtype=torch.int32, device=dev),
                   torch.empty((1,), dtype=torch.float64, device=dev))
        K, n_sel, theta = out
        self._rc(self.lib.dspark_schedule(
            self._h, _stream(dev, stream), B, gamma, surv.data_ptr(), sps.data_ptr(), sps.shape[0],
            K.data_ptr(), n_sel.data_ptr(), theta.data_ptr()))
        return K, n_sel, theta

    # -- dspark_schedule_async ------------------------------------------------------
    def schedule_async(self, surv, surv_hist, sps, out=None, stream=None):
        """Capacity from ``surv_hist`` (two steps earlier), order from ``surv``."""
        dev = self.device
        _need(surv, "surv", torch.float32, dev, 2)
        _need(surv_hist, "surv_hist", torch.float32, dev, 2)
        _need(sps, "sps", torch.float32, dev, 1)
        B, gamma = surv.shape
        if tuple(surv_hist.shape) != (B, gamma):
            raise ValueError("surv_hist must have the shape of surv")
        if out is None:
            out = (torch.empty((B,), dtype=torch.int32, device=dev),
                   torch.empty((1,), dtype=torch.int32, device=dev),
                   torch.empty((1,), dtype=torch.float64, device=dev))
        K, n_sel, theta = out
        self._rc(self.lib.dspark_schedule_async(
            self._h, _stream(dev, stream), B, gamma, surv.data_ptr(), surv_hist.data_ptr(), sps.data_ptr(),
            sps.shape[0], K.data_ptr(), n_sel.data_ptr(), theta.data_ptr()))
        return K, n_sel, theta

    # -- dspark_verify ------------------------------------------------------------
    def verify(self, target, U, W1, W2, anchor, tokens, lse, ytok, K, req_ids,
               temperature: float, seed: int, out=None, stream=None, states=None):
        """Markov head: W1 and anchor; GRU head: ``states`` from draft_rnn (W1 and
        anchor may then be None)."""
        dev = self.device
        tsb, tsk = _logits3(target, "target", dev)
        usb, usk = _logits3(U, "U", dev)
        B, trows, V = target.shape
        _need(tokens, "tokens", torch.int32, dev, 2)
        gamma = tokens.shape[1]
        if trows < gamma + 1 or U.shape[0] != B or U.shape[1] < gamma or U.shape[2] != V:
            raise ValueError("target must be [B][>=gamma+1][V] and U [B][>=gamma][V]")
        _need(W2, "W2", None, dev, 2)
        r = W2.shape[1]
        if W2.shape != (V, r):
            raise ValueError("W2 must be [V][r]")
        if states is None or W1 is not None:
            _need(W1, "W1", W2.dtype, dev, 2)
            if W1.shape != (V, r):
                raise ValueError("W1 and W2 must both be [V][r]")
        if states is None or anchor is not None:
            _need(anchor, "anchor", torch.int32, dev, 1)
            _len(anchor, B, "anchor")
        if states is not None:
            _need(states, "states", torch.float32, dev, 3)
            if tuple(states.shape) != (gamma, B, r):
                raise ValueError("states must be [gamma][B][r]")
        _need(lse, "lse", torch.float32, dev, 2)
        _need(ytok, "ytok", torch.float32, dev, 2)
        for t, nm in ((tokens, "tokens"), (lse, "lse"), (ytok, "ytok")):
            if tuple(t.shape) != (B, gamma):
                raise ValueError(f"{nm} must be [B][gamma]")
        if K is not None:
            _need(K, "K", torch.int32, dev, 1)
            _len(K, B, "K")
        if req_ids is not None:
            _need(req_ids, "req_ids", torch.int32, dev, 1)
            _len(req_ids, B, "req_ids")
        if out is None:
            out = (torch.empty((B,), dtype=torch.int32, device=dev),
                   torch.empty((B, gamma + 1), dtype=torch.int32, device=dev))
        acc, toks = out
        self._rc(self.lib.dspark_verify(
            self._h, _stream(dev, stream), B, gamma, V, r, _wdtype(W2),
            target.data_ptr(), tsb, tsk, U.data_ptr(), usb, usk, _ptr(W1), W2.data_ptr(),
            _ptr(anchor), tokens.data_ptr(), lse.data_ptr(), ytok.data_ptr(), _ptr(states), _ptr(K),
            _ptr(req_ids), float(temperature), int(seed) & 0xFFFFFFFFFFFFFFFF,
            acc.data_ptr(), toks.data_ptr()))
        return acc, toks


    # -- dspark_verify_packed -------------------------------------------------------
    def verify_packed(self, target, t_offsets, U, W1, W2, anchor, tokens, lse, ytok, K, req_ids,
                      temperature: float, seed: int, out=None, stream=None, states=None):
        """``target`` [n_rows][V] packed: request b's rows 1 .. K[b]+1 start at
        row t_offsets[b]."""
        dev = self.device
        _need(target, "target", torch.float32, dev, 2, contiguous=False)
        if target.stride(1) != 1:
            raise ValueError("target rows must be contiguous over the vocabulary")
        n_rows, V = target.shape
        usb, usk = _logits3(U, "U", dev)
        B = U.shape[0]
        _need(tokens, "tokens", torch.int32, dev, 2)
        gamma = tokens.shape[1]
        _need(t_offsets, "t_offsets", torch.int32, dev, 1)
        _len(t_offsets, B, "t_offsets")
        _need(K, "K", torch.int32, dev, 1)
        _len(K, B, "K")
        _need(W2, "W2", None, dev, 2)
        r = W2.shape[1]
        if W2.shape != (V, r):
            raise ValueError("W2 must be [V][r]")
        if states is None or W1 is not None:
            _need(W1, "W1", W2.dtype, dev, 2)
        if states is None or anchor is not None:
            _need(anchor, "anchor", torch.int32, dev, 1)
        if states is not None:
            _need(states, "states", torch.float32, dev, 3)
            if tuple(states.shape) != (gamma, B, r):
                raise ValueError("states must be [gamma][B][r]")
        for t, nm in ((tokens, "tokens"), (lse, "lse"), (ytok, "ytok")):
            if tuple(t.shape) != (B, gamma):
                raise ValueError(f"{nm} must be [B][gamma]")
        if req_ids is not None:
            _need(req_ids, "req_ids", torch.int32, dev, 1)
            _len(req_ids, B, "req_ids")
        if out is None:
            out = (torch.empty((B,), dtype=torch.int32, device=dev),
                   torch.empty((B, gamma + 1), dtype=torch.int32, device=dev))
        acc, toks = out
        self._rc(self.lib.dspark_verify_packed(
            self._h, _stream(dev, stream), B, gamma, V, r, _wdtype(W2),
            target.data_ptr(), target.stride(0), t_offsets.data_ptr(), n_rows, U.data_ptr(), usb, usk,
            _ptr(W1), W2.data_ptr(), _ptr(anchor), tokens.data_ptr(), lse.data_ptr(), ytok.data_ptr(),
            _ptr(states), K.data_ptr(), _ptr(req_ids), float(temperature), int(seed) & 0xFFFFFFFFFFFFFFFF,
            acc.data_ptr(), toks.data_ptr()))
        return acc, toks


    # -- dspark_accept_prob ---------------------------------------------------------
    def accept_prob(self, target, U, W1, W2, anchor, tokens, lse, temperature: float, states=None,
                    out=None, stream=None):
        """alpha[b][k-1] = sum_v min(p_d, p_t): the acceptance probability of every drafted position."""
        dev = self.device
        tsb, tsk = _logits3(target, "target", dev)
        usb, usk = _logits3(U, "U", dev)
        B, _, V = target.shape
        _need(tokens, "tokens", torch.int32, dev, 2)
        gamma = tokens.shape[1]
        _need(W2, "W2", None, dev, 2)
        r = W2.shape[1]
        _need(lse, "lse", torch.float32, dev, 2)
        if states is None:
            _need(W1, "W1", W2.dtype, dev, 2)
            _need(anchor, "anchor", torch.int32, dev, 1)
        else:
            _need(states, "states", torch.float32, dev, 3)
        if out is None:
            out = torch.empty((B, gamma), dtype=torch.float32, device=dev)
        self._rc(self.lib.dspark_accept_prob(
            self._h, _stream(dev, stream), B, gamma, V, r, _wdtype(W2), target.data_ptr(), tsb, tsk,
            U.data_ptr(), usb, usk, _ptr(W1), W2.data_ptr(), _ptr(anchor), tokens.data_ptr(), lse.data_ptr(),
            _ptr(states), float(temperature), out.data_ptr()))
        return out

    # -- dspark_sts_fit ---------------------------------------------------------------
    def sts_fit(self, logit, accept_len, grid, n_bins: int, out=None, stream=None):
        """Per-position temperatures by ECE grid search on held-out drafts.

        logit: float32 [N][gamma] (row stride >= gamma); accept_len: int32 [N];
        grid: float32 [n_grid] candidates.  Returns (T float32 [gamma],
        index int32 [gamma], ece float64 [gamma][n_grid])."""
        dev = self.device
        _need(logit, "logit", torch.float32, dev, 2, contiguous=False)
        if logit.stride(1) != 1:
            raise ValueError("logit rows must be contiguous over positions")
        N, gamma = logit.shape
        _need(accept_len, "accept_len", torch.int32, dev, 1)
        _len(accept_len, N, "accept_len")
        _need(grid, "grid", torch.float32, dev, 1)
        n_grid = grid.shape[0]
        if out is None:
            out = (torch.empty((gamma,), dtype=torch.float32, device=dev),
                   torch.empty((gamma,), dtype=torch.int32, device=dev),
                   torch.empty((gamma, n_grid), dtype=torch.float64, device=dev))
        T, idx, ece = out
        stride = logit.stride(0) if N > 0 else gamma
        self._rc(self.lib.dspark_sts_fit(
            self._h, _stream(dev, stream), N, gamma, logit.data_ptr() if N > 0 else None, stride,
            accept_len.data_ptr() if N > 0 else None, grid.data_ptr(), n_grid, int(n_bins),
            T.data_ptr(), idx.data_ptr(), ece.data_ptr()))
        return T, idx, ece

    # -- dspark_stream_read (measurement support) -----------------------------------
    def stream_read(self, x, out=None, stream=None):
        """The float32 sum of a contiguous float32 tensor, every element read
        once: the streaming-read calibration.  Returns out (float32 [1])."""
        dev = self.device
        _need(x, "x", torch.float32, dev)
        if out is None:
            out = torch.empty((1,), dtype=torch.float32, device=dev)
        _need(out, "out", torch.float32, dev, 1)
        n = x.numel()
        self._rc(self.lib.dspark_stream_read(self._h, _stream(dev, stream), x.data_ptr() if n > 0 else None, n,
                                             out.data_ptr()))
        return out


__all__ = ["Context", "DSparkError", "load_library", "LIB_PATH", "EXPORTS", "KERNEL_CLASSES",
           "DSPARK_OK", "DSPARK_EINVAL", "DSPARK_EHIP", "DSPARK_ENOMEM", "DSPARK_EDEVICE",
           "DSPARK_F32", "DSPARK_BF16"]
