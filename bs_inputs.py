"""Seeded synthetic inputs for the Benchmark Streaming (BS) operations.

This module draws random numbers and nothing else: it holds none of the
arithmetic of the operations themselves. The same arrays are handed to the
CPU oracle and to the HIP library, so the two sides never generate their
inputs separately.

Generator: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014), used in its counter form: the
i-th word of stream ``seed`` is ``mix(seed + (i + 1) * 0x9E3779B97F4A7C15)``
with the published finalizer (shifts 30/27/31, multipliers 0xBF58476D1CE4E5B9
and 0x94D049BB133111EB), all arithmetic modulo 2**64.

Values "uniform in [-1, 1]" are ``2 * ((w >> 11) * 2**-53) - 1``: a multiple of
2**-52 in [-1, 1), so every value, and every product of two values, is exactly
representable and no subnormal ever arises.

Random meshes ("shuffled locality", the 40^3 order-5 workload) take two random
permutations: a stable argsort of N_E words for the element order and of N_G
words for the global node numbering.
"""
from __future__ import annotations

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# Per-array seed offsets; the base seed of a workload is 1000 + its index.
SEED_X, SEED_P, SEED_R, SEED_Q, SEED_Y, SEED_ELEM, SEED_NODE = 1, 2, 3, 4, 5, 6, 7


def splitmix64(seed: int, n: int, start: int = 0) -> np.ndarray:
    """Words start .. start+n-1 of the SplitMix64 stream ``seed`` (uint64)."""
    with np.errstate(over="ignore"):
        i = np.arange(start + 1, start + n + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + i * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def uniform_pm1(seed: int, n: int, start: int = 0, chunk: int = 1 << 24) -> np.ndarray:
    """fp64 values in [-1, 1) from stream ``seed``; exact multiples of 2**-52."""
    out = np.empty(n, dtype=np.float64)
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        w = splitmix64(seed, b - a, start + a)
        out[a:b] = (w >> np.uint64(11)).astype(np.float64) * (2.0 ** -53) * 2.0 - 1.0
    return out


def small_ints(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    """fp64 integers in [lo, hi] (inclusive) from stream ``seed``."""
    w = splitmix64(seed, n)
    span = np.uint64(hi - lo + 1)
    return (w % span).astype(np.int64).astype(np.float64) + float(lo)


def permutation(seed: int, n: int) -> np.ndarray:
    """Random permutation of 0..n-1 (int32): stable argsort of n words."""
    w = splitmix64(seed, n)
    return np.argsort(w, kind="stable").astype(np.int32)


# The five workloads: (name, elements per side, order, shuffled).
MESHES = {
    "c1_box8_N3": (8, 3, False),
    "c2_box32_N7": (32, 7, False),
    "c4_shuffled40_N5": (40, 5, True),
    "c5_box24_N15": (24, 15, False),
}
CONFIG_INDEX = {"c1_box8_N3": 0, "c2_box32_N7": 1, "c3_sweep": 2,
                "c4_shuffled40_N5": 3, "c5_box24_N15": 4}


def base_seed(name: str) -> int:
    return 1000 + CONFIG_INDEX[name]


def mesh_perms(name: str, E: int, N: int):
    """(elem_perm, node_perm) for a shuffled workload, else (None, None)."""
    _, _, shuffled = MESHES[name]
    if not shuffled:
        return None, None
    G = E * N + 1
    b = base_seed(name)
    return permutation(b + SEED_ELEM, E ** 3), permutation(b + SEED_NODE, G ** 3)


def vectors(name: str, n: int, which: str = "xprqy") -> dict:
    """Uniform[-1, 1) vectors of length n for the named workload."""
    b = base_seed(name)
    off = {"x": SEED_X, "p": SEED_P, "r": SEED_R, "q": SEED_Q, "y": SEED_Y}
    return {k: uniform_pm1(b + off[k], n) for k in which}
