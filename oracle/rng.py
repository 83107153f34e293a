"""Counter-based random numbers keyed on (seed, request, position, purpose).

The pages fix no generator; the method only needs independent uniforms for
the Gumbel-max draws, the accept test, the residual draw and the bonus draw.
This is the oracle's own implementation, written from the published
definitions of its two building blocks:

* ``mix64`` -- the output function of SplitMix64 (G. Steele, D. Lea,
  C. Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014;
  the constants of S. Vigna's reference splitmix64.c).
* ``fmix32`` -- the 32-bit finalizer of MurmurHash3 (A. Appleby).

Definition (shared by contract with the HIP side, which implements it
separately):

  row key  K = mix64(mix64(mix64(seed + 0x9E3779B97F4A7C15) ^ req) ^ ((pos << 8) | purpose))
  element  h = fmix32(((K mod 2^32) ^ (v * 0x9E3779B9 mod 2^32)) + (K >> 32)  mod 2^32)
  uniform  u = (2 * (h >> 9) + 1) * 2^-24          in (0, 1), exact in fp32
  Gumbel   g = -ln(-ln u)

``pos`` is the 1-based draft position (K_b + 1 for the bonus row), ``purpose``
one of DRAFT, ACCEPT, RESID, BONUS.  The accept test of position k uses the
element v = 0 of its ACCEPT row.
"""
from __future__ import annotations

import numpy as np

DRAFT, ACCEPT, RESID, BONUS = 1, 2, 3, 4

_M64 = (1 << 64) - 1
_M32 = (1 << 32) - 1
_GOLDEN64 = 0x9E3779B97F4A7C15
_GOLDEN32 = 0x9E3779B9


def mix64(z: int) -> int:
    """SplitMix64 output mixing function on a Python int (mod 2^64)."""
    z &= _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def splitmix64_next(state: int) -> tuple[int, int]:
    """One SplitMix64 step: returns (new_state, output)."""
    state = (state + _GOLDEN64) & _M64
    return state, mix64(state)


def fmix32(h):
    """MurmurHash3 32-bit finalizer; works on Python ints and uint32 arrays."""
    if isinstance(h, np.ndarray):
        h = h.astype(np.uint32, copy=True)
        h ^= h >> np.uint32(16)
        h *= np.uint32(0x85EBCA6B)
        h ^= h >> np.uint32(13)
        h *= np.uint32(0xC2B2AE35)
        h ^= h >> np.uint32(16)
        return h
    h &= _M32
    h ^= h >> 16
    h = (h * 0x85EBCA6B) & _M32
    h ^= h >> 13
    h = (h * 0xC2B2AE35) & _M32
    h ^= h >> 16
    return h


def row_key(seed: int, req: int, pos: int, purpose: int) -> int:
    """64-bit key of one (seed, request, position, purpose) row."""
    k = mix64((seed + _GOLDEN64) & _M64)
    k = mix64(k ^ (req & _M32))
    return mix64(k ^ ((pos << 8) | purpose))


def _hash_elements(key: int, v: np.ndarray) -> np.ndarray:
    lo = np.uint32(key & _M32)
    hi = np.uint32(key >> 32)
    x = (v.astype(np.uint32) * np.uint32(_GOLDEN32)) ^ lo
    x = x + hi
    return fmix32(x)


def uniforms(key: int, n: int) -> np.ndarray:
    """Uniforms u_v, v = 0..n-1, of one row as float64 (each exact in fp32)."""
    h = _hash_elements(key, np.arange(n, dtype=np.uint32))
    return (2.0 * (h >> np.uint32(9)).astype(np.float64) + 1.0) * 2.0 ** -24


def uniform_at(key: int, v: int) -> float:
    """Single uniform of element v of a row (scalar path, Python ints only)."""
    x = (((v * _GOLDEN32) & _M32) ^ (key & _M32))
    x = (x + (key >> 32)) & _M32
    h = fmix32(x)
    return (2.0 * (h >> 9) + 1.0) * 2.0 ** -24


def gumbels(key: int, n: int) -> np.ndarray:
    """Standard Gumbel variates g_v = -ln(-ln u_v) of one row, float64."""
    return -np.log(-np.log(uniforms(key, n)))
