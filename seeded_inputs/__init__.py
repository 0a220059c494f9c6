"""Seeded synthetic inputs shared by the oracle's tests, the HIP path's tests
and the benchmark.

This module holds none of the layer's arithmetic: it only draws input bits.
Both sides receive the same bf16 bit patterns (numpy ``uint16``).

Generator (counter-based, so any block of a large logical tensor can be drawn
on its own and a rank's shard is exactly the matching block of the unsharded
draw):

* element ``c`` (row-major linear index in the full logical tensor) uses the
  SplitMix64 stream (Steele, Lea and Flood, "Fast splittable pseudorandom
  number generators", OOPSLA 2014) at positions ``2c`` and ``2c + 1``:
  ``x_n = mix64(s0 + n * 0x9E3779B97F4A7C15)`` with the published mixing
  constants ``0xBF58476D1CE4E5B9`` / ``0x94D049BB133111EB`` and shifts
  30 / 27 / 31, and stream origin ``s0 = mix64((seed + 1) * 0x9E3779B97F4A7C15)``;
* the two 53-bit uniforms ``u1 = ((x_2c >> 11) + 0.5) / 2^53`` (never 0) and
  ``u2 = (x_2c+1 >> 11) / 2^53`` give one standard normal by the Box-Muller
  transform ``sqrt(-2 ln u1) * cos(2 pi u2)`` in fp64;
* the value ``sigma * z`` is rounded to binary32 and then to bf16
  (round to nearest, ties to even).

Integer-valued inputs (exact in bf16) use ``lo + x_2c mod (hi - lo + 1)``.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _origin(seed: int) -> np.uint64:
    with np.errstate(over="ignore"):
        return _mix64(np.array([(seed + 1) % (1 << 64)], dtype=np.uint64) * _GAMMA)[0]


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """binary32 -> bf16 bits, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def _stream_pair(origin: np.uint64, counters: np.ndarray):
    with np.errstate(over="ignore"):
        n0 = counters * np.uint64(2)
        x1 = _mix64(origin + n0 * _GAMMA)
        x2 = _mix64(origin + (n0 + np.uint64(1)) * _GAMMA)
    return x1, x2


def _block_counters(full_cols: int, r0: int, r1: int, c0: int, c1: int) -> np.ndarray:
    rows = np.arange(r0, r1, dtype=np.uint64)[:, None] * np.uint64(full_cols)
    return rows + np.arange(c0, c1, dtype=np.uint64)[None, :]


def _fill_rows(fn, nrows: int, out: np.ndarray) -> np.ndarray:
    nth = _threads()
    if nrows * out.shape[1] < (1 << 16) or nth == 1:
        fn(0, nrows)
        return out
    step = max(1, (nrows + nth * 4 - 1) // (nth * 4))
    with ThreadPoolExecutor(nth) as ex:
        list(ex.map(lambda a: fn(a, min(nrows, a + step)), range(0, nrows, step)))
    return out


def normal_bf16(seed: int, shape, sigma: float, rows=None, cols=None) -> np.ndarray:
    """bf16 bits of sigma * N(0, 1) for the logical tensor ``shape`` (2-D),
    or of its block ``[rows) x [cols)`` (python ``range``/``slice`` pairs)."""
    R, C = int(shape[0]), int(shape[1])
    r0, r1 = (0, R) if rows is None else (rows.start, rows.stop)
    c0, c1 = (0, C) if cols is None else (cols.start, cols.stop)
    assert 0 <= r0 <= r1 <= R and 0 <= c0 <= c1 <= C
    out = np.empty((r1 - r0, c1 - c0), dtype=np.uint16)
    origin = _origin(seed)

    def fn(a, b):
        x1, x2 = _stream_pair(origin, _block_counters(C, r0 + a, r0 + b, c0, c1))
        u1 = ((x1 >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)
        u2 = (x2 >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
        z = np.sqrt(-2.0 * np.log(u1)) * np.cos((2.0 * np.pi) * u2)
        out[a:b] = f32_to_bf16_bits((z * sigma).astype(np.float32))

    return _fill_rows(fn, r1 - r0, out)


def normal_f32(seed: int, shape, sigma: float) -> np.ndarray:
    """binary32 values sigma * N(0, 1) from the same stream (no bf16 rounding)."""
    R, C = int(shape[0]), int(shape[1])
    out = np.empty((R, C), dtype=np.float32)
    origin = _origin(seed)

    def fn(a, b):
        x1, x2 = _stream_pair(origin, _block_counters(C, a, b, 0, C))
        u1 = ((x1 >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)
        u2 = (x2 >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
        out[a:b] = (np.sqrt(-2.0 * np.log(u1)) * np.cos((2.0 * np.pi) * u2) * sigma).astype(np.float32)

    return _fill_rows(fn, R, out)


def int_bf16(seed: int, shape, lo: int, hi: int) -> np.ndarray:
    """bf16 bits of uniform integers in [lo, hi] (exact in bf16 for |v| <= 256)."""
    R, C = int(shape[0]), int(shape[1])
    out = np.empty((R, C), dtype=np.uint16)
    origin = _origin(seed)
    span = np.uint64(hi - lo + 1)

    def fn(a, b):
        x1, _ = _stream_pair(origin, _block_counters(C, a, b, 0, C))
        v = (x1 % span).astype(np.int64) + lo
        out[a:b] = f32_to_bf16_bits(v.astype(np.float32))

    return _fill_rows(fn, R, out)


def identity_bf16(n: int) -> np.ndarray:
    out = np.zeros((n, n), dtype=np.uint16)
    out[np.arange(n), np.arange(n)] = 0x3F80  # 1.0
    return out


def permutation_bf16(seed: int, n: int) -> tuple[np.ndarray, np.ndarray]:
    """One-hot [n x n] weight W with W[perm[j], j] = 1, so (X W)[:, j] = X[:, perm[j]]."""
    origin = _origin(seed)
    x1, _ = _stream_pair(origin, np.arange(n, dtype=np.uint64))
    perm = np.argsort(x1, kind="stable").astype(np.int64)
    out = np.zeros((n, n), dtype=np.uint16)
    out[perm, np.arange(n)] = 0x3F80
    return out, perm


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to binary32 (no arithmetic)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
