"""CPU oracle for the Benchmark Streaming operations: test infrastructure.

Only the test suite, the smoke check and the CPU baseline leg of the
benchmark import this package. The product library never does, and this
package imports nothing from it.

The arithmetic lives in ``oracle.c`` (plain C, gcc, ``-ffp-contract=off``,
OpenMP on the obvious loops); this module compiles it and marshals numpy
arrays into it. Every function follows a passage of "Portable high-order
finite element kernels I: Streaming Operations" (arXiv 2009.10917) or of
"GPU accelerated spectral finite elements on all-hex meshes" (arXiv
1506.05996); the C source names them.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test may point the wrapper at a deliberately broken build of oracle.c to
# show that the pins catch the mistake.
_LIB = os.environ.get("BS_ORACLE_LIB", _LIB)

_c_int64 = ctypes.c_int64
_c_double = ctypes.c_double
_ptr = ctypes.c_void_p


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc; returns its path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-D_DEFAULT_SOURCE", "-fopenmp",
             "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
             "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        L.or_threads.argtypes = []
        L.or_threads.restype = ctypes.c_int
        L.or_set_threads.argtypes = [ctypes.c_int]
        L.or_set_threads.restype = None
        L.or_copy.argtypes = [_c_int64, _ptr, _ptr]
        L.or_copy.restype = None
        L.or_axpy.argtypes = [_c_int64, _c_double, _ptr, _c_double, _ptr]
        L.or_axpy.restype = None
        L.or_dot.argtypes = [_c_int64, _ptr, _ptr]
        L.or_dot.restype = _c_double
        L.or_norm.argtypes = [_c_int64, _ptr]
        L.or_norm.restype = _c_double
        L.or_cg_update.argtypes = [_c_int64, _c_double, _ptr, _ptr, _ptr, _ptr]
        L.or_cg_update.restype = _c_double
        L.or_scatter.argtypes = [_c_int64, _ptr, _ptr, _ptr]
        L.or_scatter.restype = None
        L.or_gather.argtypes = [_c_int64, _c_int64, _ptr, _ptr, _ptr]
        L.or_gather.restype = None
        L.or_gll_nodes.argtypes = [ctypes.c_int, _ptr]
        L.or_gll_nodes.restype = ctypes.c_int
        L.or_mesh_box.argtypes = [ctypes.c_int] * 4 + [_ptr, _ptr, _ptr]
        L.or_mesh_box.restype = _c_int64
        L.or_g2l.argtypes = [_c_int64, _c_int64, _ptr, _ptr, _ptr]
        L.or_g2l.restype = _c_int64
        L.or_gll_weights.argtypes = [ctypes.c_int, _ptr]
        L.or_gll_weights.restype = ctypes.c_int
        L.or_mesh_box_mass.argtypes = [ctypes.c_int] * 4 + [_ptr]
        L.or_mesh_box_mass.restype = ctypes.c_int
        L.or_scale.argtypes = [_c_int64, _ptr, _ptr, _ptr]
        L.or_mesh_hex.argtypes = [_c_int64, ctypes.c_int, _c_int64, _ptr, _ptr]
        L.or_mesh_hex.restype = _c_int64
        L.or_mesh_hex_mass.argtypes = [_c_int64, ctypes.c_int, _ptr, _ptr]
        L.or_mesh_hex_mass.restype = ctypes.c_int
        L.or_scale.restype = None
        _lib = L
    return _lib


def _f64(a):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data


def _i32(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data


def _nptr(a):
    return None if a is None else _i32(a)


def threads():
    """OpenMP threads the oracle's parallel loops use."""
    return lib().or_threads()


def set_threads(n):
    """Use n OpenMP threads from now on (results do not depend on it)."""
    lib().or_set_threads(int(n))


# --------------------------------------------------------------- BS1..BS7 --

def copy(x):
    """BS1: returns a bit copy of x."""
    x, px = _f64(x)
    y = np.empty_like(x)
    lib().or_copy(x.size, px, y.ctypes.data)
    return y


def axpy(alpha, x, beta, y):
    """BS2: returns (alpha*x) + (beta*y), products and sum rounded separately."""
    x, px = _f64(x)
    out = np.array(y, dtype=np.float64, copy=True)
    assert out.size == x.size
    lib().or_axpy(x.size, float(alpha), px, float(beta), out.ctypes.data)
    return out


def dot(x, y):
    """BS4: x . y, evaluated accurately (Dot2)."""
    x, px = _f64(x)
    y, py = _f64(y)
    assert x.size == y.size
    return lib().or_dot(x.size, px, py)


def norm(x):
    """BS3: the 2-norm, sqrt(x . x)."""
    x, px = _f64(x)
    return lib().or_norm(x.size, px)


def cg_update(alpha, p, q, x, r):
    """BS5: returns (x + alpha p, r - alpha q, |r_new|^2)."""
    p, pp = _f64(p)
    q, pq = _f64(q)
    xo = np.array(x, dtype=np.float64, copy=True)
    ro = np.array(r, dtype=np.float64, copy=True)
    assert p.size == q.size == xo.size == ro.size
    rr = lib().or_cg_update(p.size, float(alpha), pp, pq, xo.ctypes.data, ro.ctypes.data)
    return xo, ro, rr


def scatter(l2g, v_global):
    """BS7: v_L = Z v_G (negative ids give +0.0)."""
    l2g, pl = _i32(l2g)
    vg, pg = _f64(v_global)
    vl = np.empty(l2g.size, dtype=np.float64)
    lib().or_scatter(l2g.size, pl, pg, vl.ctypes.data)
    return vl


def gather(l2g, v_local, n_global):
    """BS6: v_G = Z^T v_L, each entry summed from +0.0 in ascending local index."""
    l2g, pl = _i32(l2g)
    vl, pv = _f64(v_local)
    assert vl.size == l2g.size
    if l2g.size:
        assert int(l2g.max()) < n_global
    vg = np.empty(int(n_global), dtype=np.float64)
    lib().or_gather(l2g.size, int(n_global), pl, pv, vg.ctypes.data)
    return vg


# ------------------------------------------------------------ mesh tables --

def gll_nodes(p):
    r = np.empty(p + 1, dtype=np.float64)
    if lib().or_gll_nodes(int(p), r.ctypes.data) != 0:
        raise ValueError("order must be >= 1")
    return r


def mesh_box(ex, ey, ez, p, elem_perm=None, node_perm=None):
    """I_l->g of a box mesh by deduplicating physical GLL node positions.

    Returns (l2g int32[K (p+1)^3], n_global)."""
    K = ex * ey * ez
    l2g = np.empty(K * (p + 1) ** 3, dtype=np.int32)
    ep = _nptr(elem_perm)
    npm = _nptr(node_perm)
    ng = lib().or_mesh_box(ex, ey, ez, p, None if ep is None else ep[1],
                           None if npm is None else npm[1], l2g.ctypes.data)
    if ng < 0:
        raise ValueError("bad mesh arguments")
    return l2g, int(ng)


def g2l(l2g, n_global):
    """CSR of I_g->l: (off int32[n_global+1], ids int32[entries]), ids ascending."""
    l2g, pl = _i32(l2g)
    off = np.empty(int(n_global) + 1, dtype=np.int32)
    ids = np.empty(max(1, l2g.size), dtype=np.int32)
    m = lib().or_g2l(l2g.size, int(n_global), pl, off.ctypes.data, ids.ctypes.data)
    if m < 0:
        raise ValueError("id out of range")
    return off, ids[:m].copy()


def gll_weights(p):
    """GLL quadrature weights of degree p on [-1, 1]."""
    w = np.empty(p + 1, dtype=np.float64)
    if lib().or_gll_weights(int(p), w.ctypes.data) != 0:
        raise ValueError("order must be >= 1")
    return w


def mesh_box_mass(ex, ey, ez, p):
    """Local lumped-mass weights of the unit-hexahedron box mesh."""
    w = np.empty(ex * ey * ez * (p + 1) ** 3, dtype=np.float64)
    if lib().or_mesh_box_mass(ex, ey, ez, p, w.ctypes.data) != 0:
        raise ValueError("bad mesh arguments")
    return w


def scale(x, d):
    """y = x / d elementwise, each quotient correctly rounded."""
    x, px = _f64(x)
    d, pd = _f64(d)
    assert x.size == d.size
    y = np.empty_like(x)
    lib().or_scale(x.size, px, pd, y.ctypes.data)
    return y


def cg_sequence(l2g, n_global, b, iters):
    """Unpreconditioned CG on A = Z^T Z (local operator the identity), x0 = 0.

    Each iteration: p_L = Z p; q = Z^T p_L; alpha = rr / (p . q); the fused
    update x += alpha p, r -= alpha q returning rr'; beta = rr' / rr;
    p = (1 r) + (beta p). Returns (x, r, list of rr per iteration)."""
    b = np.asarray(b, dtype=np.float64)
    x = np.zeros_like(b)
    r = b.copy()
    p = b.copy()
    rr = dot(r, r)
    hist = [rr]
    for _ in range(iters):
        pl = scatter(l2g, p)
        q = gather(l2g, pl, n_global)
        pq = dot(p, q)
        alpha = rr / pq
        x, r, rr_new = cg_update(alpha, p, q, x, r)
        beta = rr_new / rr
        p = axpy(1.0, r, beta, p)
        rr = rr_new
        hist.append(rr)
    return x, r, hist


def mesh_hex(ev, p, n_vert=None):
    """I_l->g of an unstructured hex mesh from its corner vertices.

    ev: int32[E, 8], corner c = a + 2b + 4d of the reference cube. Global
    nodes are the distinct points of the mesh (exact symbolic trilinear
    weights over the vertices), numbered by first appearance.
    Returns (l2g int32[E (p+1)^3], n_global)."""
    ev = np.ascontiguousarray(ev, dtype=np.int32).reshape(-1, 8)
    E = ev.shape[0]
    if n_vert is None:
        n_vert = int(ev.max()) + 1 if E else 0
    l2g = np.empty(E * (p + 1) ** 3, dtype=np.int32)
    ng = lib().or_mesh_hex(E, p, n_vert, ev.ctypes.data, l2g.ctypes.data)
    if ng < 0:
        raise ValueError("bad hex mesh")
    return l2g, int(ng)


def mesh_hex_mass(xe, p):
    """Local lumped-mass weights w_i w_j w_k |det J| of hexahedra given by
    their corner coordinates xe (float64[E, 8, 3], corner c = a + 2b + 4d)."""
    xe = np.ascontiguousarray(xe, dtype=np.float64).reshape(-1, 8, 3)
    E = xe.shape[0]
    w = np.empty(E * (p + 1) ** 3, dtype=np.float64)
    if lib().or_mesh_hex_mass(E, p, xe.ctypes.data, w.ctypes.data) != 0:
        raise ValueError("bad arguments")
    return w
