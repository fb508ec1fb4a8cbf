"""Python binding of libbs: the Benchmark Streaming operations on MI355X.

Argument marshalling only. Every operation runs in the HIP kernels of
``libbs.so`` (built in-tree for gfx950 by ``_build.py``); this module checks
shapes and dtypes, takes raw pointers from torch tensors, and turns a nonzero
status into ``BSError``. There is no fallback: if the library or a GPU is
missing, the calls raise.

Device operations take torch tensors on a HIP device (float64 vectors, int32
index tables) and enqueue on the current torch stream unless ``stream`` is
given. Reductions write their scalar into a one-element float64 device tensor
and return it, so no call synchronises the host. The table builders take and
return numpy arrays on the host.

Names and semantics are those of ``include/bs.h``: BS1 copy, BS2 AXPY, BS3
norm, BS4 dot, BS5 fused CG update, BS6 gather, BS7 scatter ("Portable
high-order finite element kernels I: Streaming Operations", arXiv
2009.10917).
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbs.so")

BS_OK, BS_EINVAL, BS_EALIGN, BS_ERANGE, BS_EHIP, BS_ENOMEM = 0, -1, -2, -3, -4, -5

_i64 = ctypes.c_int64
_dbl = ctypes.c_double
_ptr = ctypes.c_void_p
_int = ctypes.c_int


class BSError(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what}: {_lib().bs_strerror(status).decode()} ({status})")
        self.status = status


_L = None
_lock = threading.Lock()

# (name, argtypes) of every entry point in include/bs.h
SIGNATURES = {
    "bs_strerror": ([_int], ctypes.c_char_p),
    "bs_version": ([], _int),
    "bs_ctx_create": ([_int, ctypes.POINTER(_ptr)], _int),
    "bs_ctx_destroy": ([_ptr], None),
    "bs_ctx_info": ([_ptr, ctypes.POINTER(_int), ctypes.POINTER(_int), ctypes.POINTER(_int)], _int),
    "bs_ctx_time_next": ([_ptr, _ptr, _ptr], _int),
    "bs_copy": ([_ptr, _i64, _ptr, _ptr, _ptr], _int),
    "bs_axpy": ([_ptr, _i64, _dbl, _ptr, _dbl, _ptr, _ptr], _int),
    "bs_norm": ([_ptr, _i64, _ptr, _ptr, _ptr], _int),
    "bs_dot": ([_ptr, _i64, _ptr, _ptr, _ptr, _ptr], _int),
    "bs_cg_update": ([_ptr, _i64, _dbl, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr], _int),
    "bs_scatter": ([_ptr, _i64, _ptr, _ptr, _ptr, _ptr], _int),
    "bs_gather": ([_ptr, _i64, _ptr, _ptr, _ptr, _ptr, _ptr, _i64, _ptr], _int),
    "bs_gather_dot": ([_ptr, _i64, _ptr, _ptr, _ptr, _ptr, _ptr, _i64, _ptr, _ptr, _ptr], _int),
    "bs_scale": ([_ptr, _i64, _ptr, _ptr, _ptr, _ptr], _int),
    "bs_gll": ([_int, _ptr, _ptr], _int),
    "bs_mesh_box_mass": ([_int, _int, _int, _int, _ptr], _int),
    "bs_cg_solve": ([_ptr, _i64, _i64, _ptr, _ptr, _ptr, _ptr, _i64, _ptr, _ptr, _ptr, _ptr, _ptr, _int, _dbl,
                     _ptr, _ptr], _int),
    "bs_cg_solve_static": ([_i64, _i64, _ptr, _ptr, _ptr, _ptr, _i64, _ptr, _ptr, _ptr, _ptr, _ptr, _int, _dbl, _ptr,
                            _ptr], _int),
    "bs_mesh_box_count": ([_int, _int, _int, _int, ctypes.POINTER(_i64), ctypes.POINTER(_i64)], _int),
    "bs_mesh_box_l2g": ([_int, _int, _int, _int, _ptr, _ptr, _ptr], _int),
    "bs_mesh_hex_l2g": ([_i64, _int, _i64, _ptr, _ptr, ctypes.POINTER(_i64)], _int),
    "bs_mesh_hex_mass": ([_i64, _int, _ptr, _ptr], _int),
    "bs_mesh_hex_order": ([_i64, _ptr, _ptr], _int),
    "bs_validate_l2g": ([_i64, _i64, _ptr], _int),
    "bs_validate_g2l": ([_i64, _i64, _ptr, _ptr, _ptr], _int),
    "bs_validate_plan": ([_i64, _ptr, _ptr, _i64], _int),
    "bs_index_g2l": ([_i64, _i64, _ptr, _ptr, _ptr], _int),
    "bs_gather_plan": ([_i64, _ptr, _ptr, _int, _i64, _ptr, ctypes.POINTER(_i64)], _int),
    "bs_mesh_xcd_interleave": ([_i64, _i64, _ptr], _int),
    "bs_bench_loop": ([_ptr, _int, _i64, _dbl, _dbl, _i64, _int, _ptr, _ptr, _int, _ptr, ctypes.POINTER(_dbl)],
                      _int),
}


def _lib():
    global _L
    if _L is None:
        with _lock:
            if _L is None:
                if not os.path.exists(LIB_PATH):
                    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
                L = ctypes.CDLL(LIB_PATH)
                for name, (args, res) in SIGNATURES.items():
                    fn = getattr(L, name)
                    fn.argtypes = args
                    fn.restype = res
                _L = L
    return _L


def _check(status, what):
    if status != BS_OK:
        raise BSError(status, what)


# ---------------------------------------------------------------- context --

class Context:
    """A library context on one device (owns the reduction scratch)."""

    def __init__(self, device: int = 0):
        h = _ptr()
        _check(_lib().bs_ctx_create(int(device), ctypes.byref(h)), "bs_ctx_create")
        self._h = h
        self.device = int(device)

    @property
    def handle(self):
        return self._h

    def info(self):
        d, c, m = _int(), _int(), _int()
        _check(_lib().bs_ctx_info(self._h, ctypes.byref(d), ctypes.byref(c), ctypes.byref(m)), "bs_ctx_info")
        return {"device": d.value, "cu_count": c.value, "max_partials": m.value}

    def time_next(self, start=None, stop=None):
        """Arm kernel timing: the next kernel launched with this context
        records the torch.cuda.Events `start` and `stop` (timing enabled, each
        recorded once beforehand so that it exists) at its own start and end.
        No arguments disarm."""
        def handle(e):
            if e is None:
                return None
            h = e.cuda_event
            if not h:
                raise ValueError("record the event once before arming, so that it exists")
            return h
        _check(_lib().bs_ctx_time_next(self._h, handle(start), handle(stop)), "bs_ctx_time_next")

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            _lib().bs_ctx_destroy(self._h)
            self._h = _ptr()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


_contexts = {}
_ctx_lock = threading.Lock()  # not _lock: creating a Context may load the library under _lock


def _shared_context(dev: int, stream_handle: int) -> Context:
    """The shared context of one (device, stream) pair, created on first use.

    A context's reduction scratch (partials, arrival tickets, CG scalars) is
    ordered only by the stream its calls are enqueued on: two reductions on
    different streams sharing one context would race on it and could leave a
    ticket counter nonzero for every later call. Keying the shared contexts
    by stream as well as device gives each stream its own scratch."""
    key = (int(dev), int(stream_handle or 0))
    with _ctx_lock:
        ctx = _contexts.get(key)
        if ctx is None:
            ctx = _contexts[key] = Context(key[0])
    return ctx


def context(device=None, stream=None) -> Context:
    """The shared context of a device and stream (default: the current device
    and its current torch stream), created on first use."""
    import torch
    dev = torch.cuda.current_device() if device is None else int(device)
    return _shared_context(dev, _stream(stream, dev))


# ------------------------------------------------------------ marshalling --

def _dev_tensor(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a torch tensor on a HIP device")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream, device):
    import torch
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ctx_dev(t, ctx, stream=None):
    """The context a call on tensor t's device and `stream` uses: the one
    given, else the shared context of that device and stream."""
    if ctx is None:
        ctx = _shared_context(t.device.index, _stream(stream, t.device))
    return ctx


def _plan_dev(block_starts):
    """(pointer, n_blocks) of a device gather plan, or (None, 0) for none: the
    (n_blocks, 4) int32 tensor of (first row, end row, first entry, end
    entry) blocks in launch order that bs_gather_plan builds."""
    import torch
    if block_starts is None:
        return None, 0
    if block_starts.dim() != 2 or block_starts.shape[1] != 4 or block_starts.shape[0] < 1:
        raise ValueError("block_starts must be the (n_blocks, 4) plan of bs_gather_plan")
    return _dev_tensor(block_starts, torch.int32, "block_starts"), block_starts.shape[0]


def _scalar_out(out, like):
    import torch
    if out is None:
        out = torch.empty(1, dtype=torch.float64, device=like.device)
    _dev_tensor(out, torch.float64, "out")
    if out.numel() < 1:
        raise ValueError("out must hold one float64")
    return out


# ------------------------------------------------------------ operations --

def bs_copy(x, y, *, ctx=None, stream=None):
    """BS1: y[:] = x (bit copy)."""
    import torch
    if x.numel() != y.numel():
        raise ValueError("x and y differ in length")
    ctx = _ctx_dev(x, ctx, stream)
    _check(_lib().bs_copy(ctx.handle, x.numel(), _dev_tensor(x, torch.float64, "x"),
                          _dev_tensor(y, torch.float64, "y"), _stream(stream, x.device)), "bs_copy")
    return y


def bs_axpy(alpha, x, beta, y, *, ctx=None, stream=None):
    """BS2: y = (alpha*x) + (beta*y) in place."""
    import torch
    if x.numel() != y.numel():
        raise ValueError("x and y differ in length")
    ctx = _ctx_dev(x, ctx, stream)
    _check(_lib().bs_axpy(ctx.handle, x.numel(), float(alpha), _dev_tensor(x, torch.float64, "x"),
                          float(beta), _dev_tensor(y, torch.float64, "y"), _stream(stream, x.device)),
           "bs_axpy")
    return y


def bs_norm(x, out=None, *, ctx=None, stream=None):
    """BS3: out[0] = sqrt(sum x^2) on the device; returns out."""
    import torch
    ctx = _ctx_dev(x, ctx, stream)
    out = _scalar_out(out, x)
    _check(_lib().bs_norm(ctx.handle, x.numel(), _dev_tensor(x, torch.float64, "x"), out.data_ptr(),
                          _stream(stream, x.device)), "bs_norm")
    return out


def bs_dot(x, y, out=None, *, ctx=None, stream=None):
    """BS4: out[0] = sum x*y on the device; returns out."""
    import torch
    if x.numel() != y.numel():
        raise ValueError("x and y differ in length")
    ctx = _ctx_dev(x, ctx, stream)
    out = _scalar_out(out, x)
    _check(_lib().bs_dot(ctx.handle, x.numel(), _dev_tensor(x, torch.float64, "x"),
                         _dev_tensor(y, torch.float64, "y"), out.data_ptr(), _stream(stream, x.device)),
           "bs_dot")
    return out


def bs_cg_update(alpha, p, q, x, r, out=None, *, ctx=None, stream=None):
    """BS5: x += alpha p, r -= alpha q in place; out[0] = |r|^2; returns out."""
    import torch
    n = p.numel()
    if not (q.numel() == x.numel() == r.numel() == n):
        raise ValueError("p, q, x, r differ in length")
    ctx = _ctx_dev(p, ctx, stream)
    out = _scalar_out(out, p)
    _check(_lib().bs_cg_update(ctx.handle, n, float(alpha), _dev_tensor(p, torch.float64, "p"),
                               _dev_tensor(q, torch.float64, "q"), _dev_tensor(x, torch.float64, "x"),
                               _dev_tensor(r, torch.float64, "r"), out.data_ptr(),
                               _stream(stream, p.device)), "bs_cg_update")
    return out


def bs_scatter(l2g, v_global, v_local, *, ctx=None, stream=None):
    """BS7: v_local = Z v_global through l2g (negative ids give +0.0)."""
    import torch
    if l2g.numel() != v_local.numel():
        raise ValueError("l2g and v_local differ in length")
    ctx = _ctx_dev(v_local, ctx, stream)
    _check(_lib().bs_scatter(ctx.handle, l2g.numel(), _dev_tensor(l2g, torch.int32, "l2g"),
                             _dev_tensor(v_global, torch.float64, "v_global"),
                             _dev_tensor(v_local, torch.float64, "v_local"),
                             _stream(stream, v_local.device)), "bs_scatter")
    return v_local


def bs_gather(off, ids, v_local, v_global, block_starts=None, *, ctx=None, stream=None):
    """BS6: v_global = Z^T v_local through the CSR (off, ids), ascending order."""
    import torch
    ng = v_global.numel()
    if off.numel() != ng + 1:
        raise ValueError("off must hold n_global + 1 entries")
    ctx = _ctx_dev(v_global, ctx, stream)
    bp, nb = _plan_dev(block_starts)
    _check(_lib().bs_gather(ctx.handle, ng, _dev_tensor(off, torch.int32, "off"),
                            _dev_tensor(ids, torch.int32, "ids"),
                            _dev_tensor(v_local, torch.float64, "v_local"),
                            _dev_tensor(v_global, torch.float64, "v_global"), bp, nb,
                            _stream(stream, v_global.device)), "bs_gather")
    return v_global


def bs_scale(x, d, y, *, ctx=None, stream=None):
    """y = x / d elementwise (y may be x); returns y."""
    import torch
    if not (x.numel() == d.numel() == y.numel()):
        raise ValueError("x, d, y differ in length")
    ctx = _ctx_dev(x, ctx, stream)
    _check(_lib().bs_scale(ctx.handle, x.numel(), _dev_tensor(x, torch.float64, "x"),
                           _dev_tensor(d, torch.float64, "d"), _dev_tensor(y, torch.float64, "y"),
                           _stream(stream, x.device)), "bs_scale")
    return y


def bs_gll(order):
    """(nodes, weights) of the GLL rule of degree `order` (numpy, host)."""
    r = np.empty(int(order) + 1, dtype=np.float64)
    w = np.empty(int(order) + 1, dtype=np.float64)
    _check(_lib().bs_gll(int(order), r.ctypes.data, w.ctypes.data), "bs_gll")
    return r, w


def bs_mesh_box_mass(ex, ey, ez, order):
    """Local lumped-mass weights of the unit-hexahedron box mesh (numpy)."""
    nl, _ = bs_mesh_box_count(ex, ey, ez, order)
    w = np.empty(nl, dtype=np.float64)
    _check(_lib().bs_mesh_box_mass(ex, ey, ez, order, w.ctypes.data), "bs_mesh_box_mass")
    return w


def bs_gather_dot(off, ids, v_local, v_global, w, block_starts=None, out=None, *, ctx=None, stream=None):
    """BS6 with w . v_global in the same pass: returns the one-element out."""
    import torch
    ng = v_global.numel()
    if off.numel() != ng + 1 or w.numel() != ng:
        raise ValueError("off must hold n_global + 1 entries and w n_global")
    ctx = _ctx_dev(v_global, ctx, stream)
    out = _scalar_out(out, v_global)
    bp, nb = _plan_dev(block_starts)
    _check(_lib().bs_gather_dot(ctx.handle, ng, _dev_tensor(off, torch.int32, "off"),
                                _dev_tensor(ids, torch.int32, "ids"),
                                _dev_tensor(v_local, torch.float64, "v_local"),
                                _dev_tensor(v_global, torch.float64, "v_global"), bp, nb,
                                _dev_tensor(w, torch.float64, "w"), out.data_ptr(),
                                _stream(stream, v_global.device)), "bs_gather_dot")
    return out


def bs_cg_solve(l2g, off, ids, x, r, p, q, p_local, iters, tol=0.0, block_starts=None, rr_hist=None, *,
                ctx=None, stream=None):
    """Device-resident CG on Z^T Z: runs up to `iters` iterations on the
    device (x, r, p updated in place); returns rr_hist (device, iters+1).
    A caller-supplied rr_hist must hold at least iters + 1 entries (the
    device writes that many; ValueError before anything is enqueued)."""
    import torch
    ng, nl = x.numel(), l2g.numel()
    if not (r.numel() == p.numel() == q.numel() == ng) or p_local.numel() != nl or off.numel() != ng + 1:
        raise ValueError("inconsistent sizes")
    if int(iters) < 0:
        raise ValueError("iters must be >= 0")
    if rr_hist is not None and rr_hist.numel() < int(iters) + 1:
        # the device writes rr_hist[0 .. iters]; the C ABI cannot see its length
        raise ValueError(f"rr_hist holds {rr_hist.numel()} entries; {int(iters) + 1} are written")
    ctx = _ctx_dev(x, ctx, stream)
    if rr_hist is None:
        rr_hist = torch.empty(int(iters) + 1, dtype=torch.float64, device=x.device)
    bp, nb = _plan_dev(block_starts)
    _check(_lib().bs_cg_solve(ctx.handle, ng, nl, _dev_tensor(l2g, torch.int32, "l2g"),
                              _dev_tensor(off, torch.int32, "off"), _dev_tensor(ids, torch.int32, "ids"), bp, nb,
                              _dev_tensor(x, torch.float64, "x"), _dev_tensor(r, torch.float64, "r"),
                              _dev_tensor(p, torch.float64, "p"), _dev_tensor(q, torch.float64, "q"),
                              _dev_tensor(p_local, torch.float64, "p_local"), int(iters), float(tol),
                              _dev_tensor(rr_hist, torch.float64, "rr_hist"), _stream(stream, x.device)),
           "bs_cg_solve")
    return rr_hist


def bs_cg_solve_static(l2g, off, ids, x, r, p, q, p_local, iters, rr_hist, tol=0.0, block_starts=None, *,
                       stream=None):
    """bs_cg_solve without a context or any allocation (the library's static
    device scratch; on the current device): for callers that cannot allocate,
    e.g. under graph capture. The caller passes rr_hist (iters + 1 entries).
    Overlapping calls on one GPU race on the shared scratch."""
    import torch
    ng, nl = x.numel(), l2g.numel()
    if not (r.numel() == p.numel() == q.numel() == ng) or p_local.numel() != nl or off.numel() != ng + 1:
        raise ValueError("inconsistent sizes")
    if int(iters) < 0:
        raise ValueError("iters must be >= 0")
    if rr_hist.numel() < int(iters) + 1:
        raise ValueError(f"rr_hist holds {rr_hist.numel()} entries; {int(iters) + 1} are written")
    bp, nb = _plan_dev(block_starts)
    _check(_lib().bs_cg_solve_static(ng, nl, _dev_tensor(l2g, torch.int32, "l2g"),
                                     _dev_tensor(off, torch.int32, "off"), _dev_tensor(ids, torch.int32, "ids"), bp,
                                     nb, _dev_tensor(x, torch.float64, "x"), _dev_tensor(r, torch.float64, "r"),
                                     _dev_tensor(p, torch.float64, "p"), _dev_tensor(q, torch.float64, "q"),
                                     _dev_tensor(p_local, torch.float64, "p_local"), int(iters), float(tol),
                                     _dev_tensor(rr_hist, torch.float64, "rr_hist"), _stream(stream, x.device)),
           "bs_cg_solve_static")
    return rr_hist


# ------------------------------------------------------------ host tables --

def _host_i32(a, name):
    a = np.ascontiguousarray(a)
    if a.dtype != np.int32:
        raise TypeError(f"{name} must be int32")
    return a


def bs_mesh_box_count(ex, ey, ez, order):
    nl, ng = _i64(), _i64()
    _check(_lib().bs_mesh_box_count(ex, ey, ez, order, ctypes.byref(nl), ctypes.byref(ng)), "bs_mesh_box_count")
    return nl.value, ng.value


def bs_mesh_box_l2g(ex, ey, ez, order, elem_perm=None, node_perm=None):
    """I_l->g of a box mesh (int32 numpy array of length n_local)."""
    nl, _ = bs_mesh_box_count(ex, ey, ez, order)
    l2g = np.empty(nl, dtype=np.int32)
    ep = None if elem_perm is None else _host_i32(elem_perm, "elem_perm")
    npm = None if node_perm is None else _host_i32(node_perm, "node_perm")
    _check(_lib().bs_mesh_box_l2g(ex, ey, ez, order, None if ep is None else ep.ctypes.data,
                                  None if npm is None else npm.ctypes.data, l2g.ctypes.data), "bs_mesh_box_l2g")
    return l2g


def bs_mesh_hex_l2g(ev, order, n_vertices=None):
    """I_l->g of an unstructured hex mesh from corner vertices ev (int32
    [n_elements, 8]). Returns (l2g int32[n_elements (order+1)^3], n_global)."""
    ev = _host_i32(ev, "ev")
    if ev.size % 8:
        raise ValueError("ev must hold 8 vertices per element")
    E = ev.size // 8
    if n_vertices is None:
        n_vertices = int(ev.max()) + 1 if E else 0
    nl = E * (int(order) + 1) ** 3
    # a table too large for int32 ids is refused (BS_ERANGE) before anything
    # is written, so a token buffer stands in for it
    l2g = np.empty(nl if 0 <= nl <= 2 ** 31 - 1 else 1, dtype=np.int32)
    ng = _i64()
    _check(_lib().bs_mesh_hex_l2g(E, int(order), int(n_vertices), ev.ctypes.data, l2g.ctypes.data,
                                  ctypes.byref(ng)), "bs_mesh_hex_l2g")
    return l2g, ng.value


def bs_mesh_hex_mass(xe, order):
    """Local lumped-mass weights (float64[n_elements (order+1)^3]) of hexahedra
    given by their corner coordinates xe (float64[n_elements, 8, 3])."""
    xe = np.ascontiguousarray(xe)
    if xe.dtype != np.float64 or xe.size % 24:
        raise TypeError("xe must be float64 with 8 x 3 coordinates per element")
    E = xe.size // 24
    nl = E * (int(order) + 1) ** 3
    w = np.empty(nl if 0 <= nl <= 2 ** 31 - 1 else 1, dtype=np.float64)
    _check(_lib().bs_mesh_hex_mass(E, int(order), xe.ctypes.data, w.ctypes.data), "bs_mesh_hex_mass")
    return w


def bs_mesh_hex_order(xe):
    """Element storage order along a Hilbert curve through the centroids of
    hexahedra given by corner coordinates xe (float64[n_elements, 8, 3]):
    int32 perm, perm[s] = the element for slot s."""
    xe = np.ascontiguousarray(xe)
    if xe.dtype != np.float64 or xe.size % 24:
        raise TypeError("xe must be float64 with 8 x 3 coordinates per element")
    E = xe.size // 24
    perm = np.empty(max(E, 1), dtype=np.int32)
    _check(_lib().bs_mesh_hex_order(E, xe.ctypes.data, perm.ctypes.data), "bs_mesh_hex_order")
    return perm[:E]


def bs_validate_l2g(l2g, n_global):
    l2g = _host_i32(l2g, "l2g")
    _check(_lib().bs_validate_l2g(l2g.size, int(n_global), l2g.ctypes.data), "bs_validate_l2g")


def bs_validate_g2l(off, ids, n_local, l2g=None):
    """Raise BSError unless (off, ids) is a well-formed CSR of I_g->l for
    n_local local entries (and, given l2g, exactly its transpose)."""
    off = _host_i32(off, "off")
    ids = _host_i32(ids, "ids")
    ng = off.size - 1
    if ng < 0:
        raise ValueError("off must hold n_global + 1 entries")
    if ids.size < max(int(off[-1]), 0):
        raise ValueError("ids must hold off[-1] entries")
    lp = None
    if l2g is not None:
        l2g = _host_i32(l2g, "l2g")
        if l2g.size != int(n_local):
            raise ValueError("l2g must hold n_local entries")
        lp = l2g.ctypes.data
    _check(_lib().bs_validate_g2l(ng, int(n_local), off.ctypes.data, ids.ctypes.data if ids.size else None, lp),
           "bs_validate_g2l")


def bs_validate_plan(plan, off):
    """Raise BSError unless plan is a well-formed gather plan for the CSR
    offsets off (n_global + 1 entries): (n_blocks, 4) int32 blocks of (first
    row, end row, first entry, end entry)."""
    p = np.asarray(plan)
    if p.ndim != 2 or p.shape[1] != 4:
        raise ValueError("plan must be (n_blocks, 4)")
    p = _host_i32(p, "plan")
    off = _host_i32(off, "off")
    if off.size < 1:
        raise ValueError("off needs n_global + 1 >= 1 entries")
    _check(_lib().bs_validate_plan(off.size - 1, off.ctypes.data, p.ctypes.data if p.size else None, p.shape[0]),
           "bs_validate_plan")


def bs_index_g2l(l2g, n_global):
    """CSR of I_g->l: (off int32[n_global+1], ids int32[entries])."""
    l2g = _host_i32(l2g, "l2g")
    off = np.empty(int(n_global) + 1, dtype=np.int32)
    ids = np.empty(max(1, l2g.size), dtype=np.int32)
    _check(_lib().bs_index_g2l(l2g.size, int(n_global), l2g.ctypes.data, off.ctypes.data, ids.ctypes.data),
           "bs_index_g2l")
    return off, ids[:int(off[-1])]


def bs_gather_plan(off, nodes_per_block=1024, ids=None, region_entries=0):
    """The LDS-staged gather's plan: an int32 numpy array of shape
    (n_blocks, 4), each block's (first row, end row, first entry, end entry)
    in launch order. region_entries > 0 places the blocks by mesh region
    (the local layout of bs_mesh_xcd_interleave) and needs the CSR ids."""
    off = _host_i32(off, "off")
    ng = off.size - 1
    if int(region_entries) > 0:
        if ids is None:
            raise ValueError("region placement needs the CSR ids")
        ids = _host_i32(ids, "ids")
        if ids.size < int(off[-1]):
            raise ValueError("ids holds fewer entries than off names")
    plan = np.empty((max(ng, 1), 4), dtype=np.int32)
    nb = _i64()
    _check(_lib().bs_gather_plan(ng, off.ctypes.data, None if ids is None else ids.ctypes.data,
                                 int(nodes_per_block), int(region_entries), plan.ctypes.data, ctypes.byref(nb)),
           "bs_gather_plan")
    return plan[:nb.value].copy()


def bs_mesh_xcd_interleave(n_elements, chunk):
    """Storage order interleaving eight consecutive regions of the given
    element order in runs of chunk elements: int32 perm, perm[s] = the
    element stored at slot s."""
    perm = np.empty(max(int(n_elements), 1), dtype=np.int32)
    _check(_lib().bs_mesh_xcd_interleave(int(n_elements), int(chunk), perm.ctypes.data), "bs_mesh_xcd_interleave")
    return perm[:int(n_elements)].copy()


BS_OP = {"copy": 0, "axpy": 1, "norm": 2, "dot": 3, "cg_update": 4, "scale": 5, "scatter": 6, "gather": 7}
BS_BENCH_SET = 6
# per op: (dtype letter per pointer slot, length each slot must reach: "n" or an int)
_BENCH_SLOTS = {"copy": "dd", "axpy": "dd", "norm": "d", "dot": "dd", "cg_update": "dddd", "scale": "ddd",
                "scatter": "idd", "gather": "iiddi"}


def bs_bench_loop(op, n, sets, reps, result=None, alpha=0.37, beta=1.0, *, n_blocks=0, ctx=None, stream=None):
    """Host seconds for `reps` back-to-back launches of `op` issued from C++,
    cycling through `sets` (a list of tuples of device tensors in the order
    the header lists for the op). Vector operations take n = their length,
    scatter n = n_local, gather n = n_global; a gather set's fifth tensor is
    the gather plan ((n_blocks, 4) blocks) or None."""
    import torch
    if op not in BS_OP:
        raise ValueError(f"unknown op {op!r}")
    slots = _BENCH_SLOTS[op]
    if not sets:
        raise ValueError("at least one pointer set is needed")
    ptrs = (ctypes.c_void_p * (BS_BENCH_SET * len(sets)))()
    for k, group in enumerate(sets):
        group = tuple(group)
        if op == "gather" and len(group) == 4:
            group = group + (None,)
        if len(group) != len(slots):
            raise ValueError(f"{op} takes {len(slots)} tensors per set")
        if op == "scatter":
            if group[0].numel() < n or group[2].numel() < n:
                raise ValueError("scatter: l2g and v_local need n_local entries")
        elif op == "gather":
            if group[0].numel() < n + 1 or group[3].numel() < n:
                raise ValueError("gather: off needs n_global + 1 entries and v_global n_global")
            if group[4] is not None and (group[4].dim() != 2 or group[4].shape[1] != 4 or
                                         group[4].shape[0] < n_blocks):
                raise ValueError("gather: block_starts must be a (>= n_blocks, 4) plan")
        for j, (t, kind) in enumerate(zip(group, slots)):
            if t is None:
                if not (op == "gather" and j == 4):
                    raise ValueError(f"sets[{k}][{j}] is required")
                continue
            ptrs[BS_BENCH_SET * k + j] = _dev_tensor(t, torch.float64 if kind == "d" else torch.int32,
                                                     f"sets[{k}][{j}]")
            if op not in ("scatter", "gather") and t.numel() < n:
                raise ValueError(f"sets[{k}][{j}] holds fewer than n elements")
    first = sets[0][0]
    if op in ("norm", "dot", "cg_update"):
        result = _scalar_out(result, first)
    ctx = _ctx_dev(first, ctx, stream)
    sec = _dbl()
    _check(_lib().bs_bench_loop(ctx.handle, BS_OP[op], int(n), float(alpha), float(beta), int(n_blocks), len(sets),
                                ptrs, None if result is None else result.data_ptr(), int(reps),
                                _stream(stream, first.device), ctypes.byref(sec)), "bs_bench_loop")
    return sec.value


__all__ = [
    "BSError", "Context", "context", "LIB_PATH", "SIGNATURES",
    "bs_copy", "bs_axpy", "bs_norm", "bs_dot", "bs_cg_update", "bs_scatter", "bs_gather",
    "bs_gather_dot", "bs_cg_solve", "bs_cg_solve_static", "bs_scale", "bs_gll", "bs_mesh_box_mass",
    "bs_bench_loop", "BS_OP", "BS_BENCH_SET",
    "bs_mesh_box_count", "bs_mesh_box_l2g", "bs_mesh_hex_l2g", "bs_mesh_hex_mass", "bs_mesh_hex_order", "bs_validate_l2g", "bs_validate_g2l", "bs_validate_plan", "bs_index_g2l", "bs_gather_plan", "bs_mesh_xcd_interleave",
]
