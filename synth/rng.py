"""Counter-based, row-addressable random numbers for the synthetic workloads.

Every value is a pure function of (seed, element index), so any row range of a
tensor can be regenerated on its own, in any order, on any thread.

Generator: the SplitMix64 output function (Steele, Lea and Flood, "Fast
splittable pseudorandom number generators", OOPSLA 2014), applied to a Weyl
sequence: x_i = key(seed) + (i + 1) * 0x9E3779B97F4A7C15 (mod 2^64),
out_i = mix(x_i).  Uniforms take the top 53 bits; normals use the Box-Muller
transform (Box and Muller, 1958) on consecutive pairs, in float64.

This module holds no arithmetic of the attention method itself.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_TWO_M53 = 2.0 ** -53
_CHUNK = 1 << 22  # elements per worker chunk


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _key(seed: int) -> np.uint64:
    return _mix(np.array([seed & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64))[0]


def _raw(key: np.uint64, start: int, count: int) -> np.ndarray:
    i = np.arange(start + 1, start + 1 + count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix(key + i * _GOLDEN)


def _uniform53(key, start, count):
    return (_raw(key, start, count) >> np.uint64(11)).astype(np.float64) * _TWO_M53


def _normal_block(key, start, count):
    # element e uses pair e // 2: (u1, u2) = raw(2p), raw(2p+1)
    p0 = start // 2
    p1 = (start + count + 1) // 2
    r = _raw(key, 2 * p0, 2 * (p1 - p0))
    u1 = ((r[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * _TWO_M53  # (0, 1]
    u2 = (r[1::2] >> np.uint64(11)).astype(np.float64) * _TWO_M53          # [0, 1)
    rad = np.sqrt(-2.0 * np.log(u1))
    ang = 2.0 * np.pi * u2
    out = np.empty(2 * (p1 - p0), dtype=np.float64)
    out[0::2] = rad * np.cos(ang)
    out[1::2] = rad * np.sin(ang)
    off = start - 2 * p0
    return out[off:off + count]


def _parallel(fn, key, start, count, workers=None):
    if count <= _CHUNK:
        return fn(key, start, count)
    out = np.empty(count, dtype=np.float64)
    starts = list(range(0, count, _CHUNK))
    workers = workers or min(16, os.cpu_count() or 1)

    def job(s):
        n = min(_CHUNK, count - s)
        out[s:s + n] = fn(key, start + s, n)

    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(job, starts))
    return out


def uniform(seed: int, start: int, count: int, lo=0.0, hi=1.0) -> np.ndarray:
    """count float64 values U[lo, hi) for flat element indices [start, start+count)."""
    u = _parallel(_uniform53, _key(seed), start, count)
    return lo + (hi - lo) * u


def normal(seed: int, start: int, count: int, std=1.0) -> np.ndarray:
    """count float64 values N(0, std^2) for flat element indices [start, start+count)."""
    return std * _parallel(_normal_block, _key(seed), start, count)


def normal_rows(seed: int, shape, r0=0, r1=None, std=1.0) -> np.ndarray:
    """Rows [r0, r1) of a tensor of `shape` (row = first axis) drawn from N(0, std^2)."""
    shape = tuple(int(s) for s in shape)
    r1 = shape[0] if r1 is None else r1
    per_row = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    v = normal(seed, r0 * per_row, (r1 - r0) * per_row, std)
    return v.reshape((r1 - r0,) + shape[1:])


def uniform_rows(seed: int, shape, r0=0, r1=None, lo=0.0, hi=1.0) -> np.ndarray:
    shape = tuple(int(s) for s in shape)
    r1 = shape[0] if r1 is None else r1
    per_row = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    v = uniform(seed, r0 * per_row, (r1 - r0) * per_row, lo, hi)
    return v.reshape((r1 - r0,) + shape[1:])
