"""Seeded synthetic inputs for the Benchmark Streaming (BS) operations.

This module draws random numbers and lays out synthetic hexahedral meshes as
corner-vertex connectivity: it holds none of the arithmetic of the operations
themselves and none of the GLL node numbering that the mesh builders compute.
The same arrays are handed to the CPU oracle and to the HIP library, so the
two sides never generate their inputs separately.

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

# Per-array seed offsets from the base seed of a workload.
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


# The box meshes: (name, elements per side, order, shuffled).
MESHES = {
    "box8_N3": (8, 3, False),
    "box32_N7": (32, 7, False),
    "shuffled40_N5": (40, 5, True),
    "box24_N15": (24, 15, False),
}
BASE_SEED = {"box8_N3": 1000, "box32_N7": 1001, "sweep": 1002,
             "shuffled40_N5": 1003, "box24_N15": 1004,
             "tetsplit11_N7": 1005,  # unstructured: 11^3 cubes cut into 24 hexahedra each
             "slab32x32x4_N7": 1006}  # one of eight z-slabs of the 32^3 order-7 box


def base_seed(name: str) -> int:
    return BASE_SEED[name]


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


# ------------------------------------------------- hexahedral meshes ------
# A hex mesh is given by corner vertices: ev[e, c] is the vertex at corner
# c = a + 2b + 4d of the reference cube, (a, b, d) in {0,1}^3 along (x, y, z).

def hex_box(nx: int, ny: int, nz: int, periodic=(False, False, False), twist: bool = False):
    """Corner connectivity of the nx x ny x nz box of unit cubes, elements in
    lexicographic order (x fastest).

    An axis marked periodic wraps its last vertex layer onto the first (a
    torus); it needs at least 3 cells so that distinct edges keep distinct
    end points. ``twist`` (x periodic, y not) wraps x with a reflection of y,
    (nx, y, z) -> (0, ny - y, z): a non-orientable, still conforming mesh.
    Returns (ev int32[E, 8], n_vert)."""
    n = (nx, ny, nz)
    for a in range(3):
        if periodic[a] and n[a] < 3:
            raise ValueError("a periodic axis needs at least 3 cells")
    if twist and (not periodic[0] or periodic[1]):
        raise ValueError("twist wraps x (periodic) with a reflection of y (not periodic)")
    vx, vy, vz = (n[a] if periodic[a] else n[a] + 1 for a in range(3))

    def vid(X, Y, Z):
        if periodic[0] and X == nx:
            X = 0
            if twist:
                Y = ny - Y
        if periodic[1]:
            Y = Y % ny
        if periodic[2]:
            Z = Z % nz
        return X + vx * (Y + vy * Z)

    ev = np.empty((nx * ny * nz, 8), dtype=np.int32)
    e = 0
    for cz in range(nz):
        for cy in range(ny):
            for cx in range(nx):
                for c in range(8):
                    ev[e, c] = vid(cx + (c & 1), cy + ((c >> 1) & 1), cz + ((c >> 2) & 1))
                e += 1
    return ev, vx * vy * vz


def _axis_perms():
    return [(0, 1, 2), (0, 2, 1), (1, 0, 2), (1, 2, 0), (2, 0, 1), (2, 1, 0)]


def cube_symmetry(s: int):
    """The s-th of the 48 symmetries of the cube, 0 <= s < 48, as (perm,
    flip): new axis a is old axis perm[a], reflected when bit a of flip is
    set. Returns sigma, int[8]: new corner c takes old corner sigma[c]."""
    perm, flip = _axis_perms()[s // 8], s % 8
    sigma = []
    for c in range(8):
        old = 0
        for a in range(3):
            bit = ((c >> a) & 1) ^ ((flip >> a) & 1)
            old |= bit << perm[a]
        sigma.append(old)
    return perm, flip, sigma


def hex_orient(ev: np.ndarray, seed: int):
    """Present every element in a random one of the 48 corner orders of the
    cube (rotations and reflections). Returns (ev2, sym int[E]) with
    ev2[e, c] = ev[e, sigma_sym[e][c]]."""
    E = ev.shape[0]
    sym = (splitmix64(seed, E) % np.uint64(48)).astype(np.int64)
    return reorder_corners(ev, sym).astype(np.int32), sym


def reorder_corners(a: np.ndarray, sym: np.ndarray) -> np.ndarray:
    """a[e, c, ...] -> a[e, sigma_sym[e][c], ...] (corner data of elements, such
    as vertex ids or corner coordinates, in the orientation hex_orient chose)."""
    table = np.array([cube_symmetry(s)[2] for s in range(48)], dtype=np.int64)
    idx = table[np.asarray(sym)]
    return a[np.arange(a.shape[0])[:, None], idx]


def hex_box_coords(nx: int, ny: int, nz: int) -> np.ndarray:
    """Corner coordinates float64[E, 8, 3] of the unit cubes of hex_box (the
    lattice point of each corner, not wrapped, so periodic boxes get their
    true element shapes)."""
    xe = np.empty((nx * ny * nz, 8, 3))
    e = 0
    for cz in range(nz):
        for cy in range(ny):
            for cx in range(nx):
                for c in range(8):
                    xe[e, c] = (cx + (c & 1), cy + ((c >> 1) & 1), cz + ((c >> 2) & 1))
                e += 1
    return xe


def hex_relabel(ev: np.ndarray, n_vert: int, seed: int, spare: int = 0):
    """Rename the vertices by a random permutation of n_vert + spare ids (the
    spare ids are never used). Returns (ev2, n_vert + spare)."""
    perm = permutation(seed, n_vert + spare)
    return perm[ev].astype(np.int32), n_vert + spare


def hex_tet_split(nx: int, ny: int, nz: int):
    """An unstructured all-hex mesh: the box of unit cubes, each cut into the
    six Kuhn tetrahedra (one per ordering of the axes), each tetrahedron cut
    into four hexahedra, one per tetrahedron vertex V with corners V, the
    three edge midpoints at V, the three face centres at V and the centroid.
    Edges are shared by 1 to 6 hexahedra (a lattice has at most 4), so the
    mesh is not a lattice. Returns (ev int32[24 nx ny nz, 8], n_vert, coords f64[n_vert, 3])."""
    coords = []
    ids = {}

    def get(key, xyz):
        if key not in ids:
            ids[key] = len(coords)
            coords.append(xyz)
        return ids[key]

    def lattice(X, Y, Z):
        return get(("v", X, Y, Z), (float(X), float(Y), float(Z)))

    def mid(u, w):
        k = tuple(sorted((u, w)))
        return get(("e",) + k, tuple((coords[u][a] + coords[w][a]) / 2 for a in range(3)))

    def centre(u, w, t):
        k = tuple(sorted((u, w, t)))
        return get(("f",) + k, tuple((coords[u][a] + coords[w][a] + coords[t][a]) / 3 for a in range(3)))

    hexes = []
    for cz in range(nz):
        for cy in range(ny):
            for cx in range(nx):
                for perm in _axis_perms():
                    p = [cx, cy, cz]
                    tet = [lattice(*p)]
                    for a in perm:
                        p[a] += 1
                        tet.append(lattice(*p))
                    cen = get(("c",) + tuple(tet),
                              tuple(sum(coords[t][a] for t in tet) / 4 for a in range(3)))
                    for vi in range(4):
                        V = tet[vi]
                        P, Q, R = [tet[t] for t in range(4) if t != vi]
                        hexes.append([V, mid(V, P), mid(V, Q), centre(V, P, Q),
                                      mid(V, R), centre(V, P, R), centre(V, Q, R), cen])
    return np.array(hexes, dtype=np.int32), len(coords), np.array(coords, dtype=np.float64)
