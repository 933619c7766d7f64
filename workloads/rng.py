"""Counter-based seeded random numbers for synthetic inputs.

This module holds no quantization arithmetic: it only turns (seed, stream
name, counter) into numbers, so the oracle and the HIP path can be fed the
very same bytes.

Generator definition (stated here so any other implementation can match it):

* Stream key: ``key = mix64(seed * 0x9E3779B97F4A7C15 + fnv1a64(name))``.
* Raw word ``i`` of a stream: ``mix64(key + (i + 1) * 0x9E3779B97F4A7C15)``,
  where ``mix64`` is the SplitMix64 finaliser (Steele, Lea & Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014):
  ``z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
  z *= 0x94D049BB133111EB; z ^= z >> 31`` (all mod 2**64).
* Uniform in (0, 1]: ``((w >> 11) + 1) * 2**-53``.
* Standard normals by the Box-Muller transform on word pairs (2j, 2j+1):
  ``r = sqrt(-2 ln u1)``, ``z[2j] = r cos(2 pi u2)``, ``z[2j+1] = r sin(2 pi u2)``,
  evaluated in float64.
"""
from __future__ import annotations

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_MASK64 = (1 << 64) - 1


def fnv1a64(name: str) -> int:
    """64-bit FNV-1a hash of a UTF-8 string (stream names)."""
    h = 0xCBF29CE484222325
    for b in name.encode("utf-8"):
        h ^= b
        h = (h * 0x100000001B3) & _MASK64
    return h


def _mix64_int(z: int) -> int:
    z &= _MASK64
    z ^= z >> 30
    z = (z * 0xBF58476D1CE4E5B9) & _MASK64
    z ^= z >> 27
    z = (z * 0x94D049BB133111EB) & _MASK64
    z ^= z >> 31
    return z


def _mix64(z: np.ndarray) -> np.ndarray:
    z = z ^ (z >> np.uint64(30))
    z = z * _M1
    z = z ^ (z >> np.uint64(27))
    z = z * _M2
    z = z ^ (z >> np.uint64(31))
    return z


def stream_key(seed: int, name: str) -> int:
    return _mix64_int((seed * 0x9E3779B97F4A7C15 + fnv1a64(name)) & _MASK64)


class Stream:
    """One named substream of a seed. Draws are by absolute counter, so a
    slice of a large tensor can be regenerated without the rest."""

    CHUNK = 1 << 22

    def __init__(self, seed: int, name: str):
        self.seed = int(seed)
        self.name = name
        self.key = np.uint64(stream_key(self.seed, name))

    def words(self, start: int, n: int) -> np.ndarray:
        idx = np.arange(start + 1, start + n + 1, dtype=np.uint64)
        with np.errstate(over="ignore"):
            return _mix64(self.key + idx * _GOLDEN)

    def uniform(self, n: int, start: int = 0) -> np.ndarray:
        """float64 uniforms in (0, 1]."""
        w = self.words(start, n)
        return ((w >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)

    def normal(self, n: int) -> np.ndarray:
        """float64 standard normals, n of them (counter 0 .. 2*ceil(n/2))."""
        out = np.empty(n, dtype=np.float64)
        pairs = (n + 1) // 2
        done = 0
        while done < pairs:
            cnt = min(self.CHUNK, pairs - done)
            w = self.words(2 * done, 2 * cnt)
            u = ((w >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)
            u1 = u[0::2]
            u2 = u[1::2]
            r = np.sqrt(-2.0 * np.log(u1))
            th = (2.0 * np.pi) * u2
            blk = np.empty(2 * cnt, dtype=np.float64)
            blk[0::2] = r * np.cos(th)
            blk[1::2] = r * np.sin(th)
            lo = 2 * done
            hi = min(n, lo + 2 * cnt)
            out[lo:hi] = blk[: hi - lo]
            done += cnt
        return out

    def choice_without_replacement(self, population: int, k: int) -> np.ndarray:
        """k distinct indices of range(population): the k smallest random keys."""
        keys = self.words(0, population)
        order = np.argsort(keys, kind="stable")
        return np.sort(order[:k]).astype(np.int64)

    def integers(self, n: int, low: int, high: int) -> np.ndarray:
        """n integers uniform in [low, high) (high - low small)."""
        span = high - low
        w = self.words(0, n)
        return (low + (w % np.uint64(span)).astype(np.int64)).astype(np.int64)

    def permutation(self, n: int) -> np.ndarray:
        keys = self.words(0, n)
        return np.argsort(keys, kind="stable").astype(np.int64)
