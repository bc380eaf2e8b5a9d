"""Seeded synthetic inputs shared by the HIP path, the tests and the oracle.

This module only draws numbers; it holds none of the transformer block's
arithmetic.  Every tensor is a pure function of (workload seed, tensor name,
element index), so any element can be regenerated on its own and the CPU
oracle and the GPU path always see bit-identical inputs.

Generator (counter-based, so no state is carried between tensors):

* sub-seed  s = splitmix64_mix(seed ^ fnv1a64(name))
* raw word  w_i = splitmix64_mix(s + (i + 1) * 0x9E3779B97F4A7C15)   (mod 2**64)
  -- this is the i-th output of Steele, Lea and Flood's SplitMix64 generator
  started from state s (the published splitmix64 finaliser with the golden
  gamma increment).
* uniform   u_i = (w_i >> 11) * 2**-53                                in [0, 1)
* normal    n_i = sqrt(-2 ln(1 - u_{2i})) * cos(2 pi u_{2i+1})      (Box-Muller,
  cosine branch only, so element i needs counters 2i and 2i+1 and nothing else)
* fp32 values are the double draw rounded to nearest even; bf16 values are the
  fp32 value rounded to nearest even on the upper 16 bits.
* integer ids are floor(u_i * V).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22


def _mix(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output finaliser on a uint64 array (wrapping arithmetic)."""
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _mix_int(x: int) -> int:
    m = (1 << 64) - 1
    z = x & m
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & m
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & m
    return z ^ (z >> 31)


def fnv1a64(name: str) -> int:
    h = 0xCBF29CE484222325
    for b in name.encode():
        h ^= b
        h = (h * 0x100000001B3) & ((1 << 64) - 1)
    return h


def subseed(seed: int, name: str) -> int:
    return _mix_int((seed ^ fnv1a64(name)) & ((1 << 64) - 1))


def _words(s: int, start: int, n: int) -> np.ndarray:
    with np.errstate(over="ignore"):
        ctr = np.arange(start + 1, start + n + 1, dtype=np.uint64)
        return _mix(np.uint64(s) + ctr * _GOLDEN)


def _uniform_words(s: int, start: int, n: int) -> np.ndarray:
    return (_words(s, start, n) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def uniform(seed: int, name: str, n: int, start: int = 0) -> np.ndarray:
    """n uniform doubles in [0, 1) for elements start .. start+n-1."""
    s = subseed(seed, name)
    out = np.empty(n, dtype=np.float64)
    for c0 in range(0, n, _CHUNK):
        c1 = min(n, c0 + _CHUNK)
        out[c0:c1] = _uniform_words(s, start + c0, c1 - c0)
    return out


def _threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def normal(seed: int, name: str, n: int, start: int = 0) -> np.ndarray:
    """n standard normal doubles for elements start .. start+n-1."""
    s = subseed(seed, name)
    out = np.empty(n, dtype=np.float64)

    def fill(c0):
        c1 = min(n, c0 + _CHUNK)
        i0 = start + c0
        m = c1 - c0
        u = _uniform_words(s, 2 * i0, 2 * m)
        u1, u2 = u[0::2], u[1::2]
        out[c0:c1] = np.sqrt(-2.0 * np.log1p(-u1)) * np.cos(2.0 * np.pi * u2)

    starts = range(0, n, _CHUNK)
    if n > 2 * _CHUNK:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, starts))
    else:
        for c0 in starts:
            fill(c0)
    return out


def round_bf16(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even), returned as fp32 values."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    b = x32.view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = ((b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32)


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Upper 16 bits of fp32 values that are already bf16-representable."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    return (x32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def tensor(seed: int, name: str, shape, std: float = 1.0, mean: float = 0.0,
           dtype: str = "f32") -> np.ndarray:
    """A seeded N(mean, std^2) tensor as fp32 values (bf16-representable if
    dtype == 'bf16')."""
    n = int(np.prod(shape)) if len(shape) else 1
    v = (mean + std * normal(seed, name, n)).astype(np.float32)
    if dtype == "bf16":
        v = round_bf16(v)
    return v.reshape(shape)


def const(shape, value: float) -> np.ndarray:
    return np.full(shape, value, dtype=np.float32)


def ids(seed: int, name: str, n: int, vocab: int) -> np.ndarray:
    u = uniform(seed, name, n)
    return np.minimum((u * vocab).astype(np.int64), vocab - 1).astype(np.int32)


def rows(seed: int, name: str, row_ids: np.ndarray, width: int, std: float,
         dtype: str = "f32") -> np.ndarray:
    """Rows row_ids of the seeded [*, width] N(0, std^2) matrix `name`, drawn
    element by element without generating the rest of the matrix."""
    row_ids = np.asarray(row_ids, dtype=np.int64)
    out = np.empty((row_ids.size, width), dtype=np.float32)
    uniq, inv = np.unique(row_ids, return_inverse=True)
    cache = np.empty((uniq.size, width), dtype=np.float32)
    for k, r in enumerate(uniq):
        cache[k] = (std * normal(seed, name, width, start=int(r) * width)).astype(np.float32)
    out[:] = cache[inv]
    if dtype == "bf16":
        out = round_bf16(out)
    return out
