"""Benchmark of the seven Benchmark Streaming (BS) operations on one MI355X.

One step is one pass of the whole path over the 32^3-element, order-7 box
mesh (N_G = 11,390,625 global nodes, N_L = 16,777,216 local entries), fp64:
BS1 copy, BS2 AXPY (alpha 0.37, beta 1), BS3 norm, BS4 dot and BS5 fused CG
update on global-length vectors, BS7 scatter through I_l->g and BS6 gather
through the CSR form of I_g->l. Each operation works on arrays of its own,
and consecutive steps run on 12 different sets of all these arrays, so
between two touches of the same array about 21 GB stream through the 256 MB
last-level cache: every operation reads cold data from HBM. (With a single
set, arrays read with the ordinary cache policy, such as the gather's v_L,
were found to survive in that cache from one step to the next, past the
non-temporal traffic of the other operations.)

The figure of merit is effective bandwidth, algorithmic bytes over time
("Portable high-order finite element kernels I", arXiv 2009.10917, where
time is taken on the host around the launches). Algorithmic bytes per
operation count every array once, index tables included:
  copy 16n, AXPY 24n, norm 8n, dot 16n, fused update 48n,
  scatter 12 N_L + 8 N_G, gather 12 N_L + 12 N_G + 4.

Printed: one JSON line (value = bytes of a step / host-timed seconds of a
step, whole job), with per-operation times (HIP events around loops of
back-to-back launches that cycle through distinct array sets, so every launch
reads cold data), the roofline of the dominant operation (HIP events around
it in every fourth timed step), and the CPU oracle timed on a bounded sample of the
same step. After the timed region (skipped with --no-extras): the size
sweep n = 2^10 .. 2^28 fitted to the latency-plus-bandwidth model
T(B) = T0 + B/W_max (eq. 8) with B_0.8 = 4 T0 W_max (eq. 10), and the other
workloads: the shuffled 40^3 order-5, tet-split and 24^3 order-15 meshes, one
GPU's slab share of the 32^3 order-7 mesh, and the CG streaming sequence
(host-driven and device-resident) on the slab, the 24^3 order-15 mesh and the
whole 32^3 order-7 mesh. Their compact figures join the line; --out writes
everything (JSON).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bs_inputs  # noqa: E402

PEAK_GBPS = 8000.0  # MI355X HBM3E, published
METRIC = "effective GB/s and % of HBM peak per BS op (fp64, N=7 hex mesh, 1 GPU)"
OPS = ["copy", "axpy", "norm", "dot", "cg_update", "scatter", "gather"]
KERNEL_NAME = {  # op -> its kernels as rocprofv3 names them (namespace and arguments stripped)
    "copy": ["k_copy<1, 768>"], "axpy": ["k_axpy<1>"], "norm": ["k_dot<4, true, 256>"],
    "dot": ["k_dot<2, false, 512>"], "cg_update": ["k_cg_update<1, 2, 512>"],
    "scatter": ["k_scatter"], "gather": ["k_gather_plan<false>"],
}
GATHER_NPB = 1024
PER_OP_FIELDS = ["bytes", "us", "us_best", "GBps", "pct_peak", "pct_copy_ceiling", "hot_us"]
EVENT_STRIDE = 4  # default: timed steps per step whose dominant kernel records events
MIN_TIMED_LAUNCHES = 10  # a short run times the dominant kernel more often, down to every step


def op_bytes(op, n=0, nl=0, ng=0):
    return {
        "copy": 16 * n, "axpy": 24 * n, "norm": 8 * n, "dot": 16 * n, "cg_update": 48 * n,
        "scatter": 12 * nl + 8 * ng, "gather": 12 * nl + 12 * ng + 4,
    }[op]


class TimingEvents:
    """Pairs of HIP events for timing kernels only, created through the HIP
    runtime the process has loaded (the one torch and libbs share) with
    hipEventDisableSystemFence: recording such an event performs no
    system-scope fence, so the timed kernel pays no cache write-back or
    invalidation for being measured. (torch.cuda.Event has no such flag;
    fence="system" uses its events instead, for comparison.)"""

    DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence

    def __init__(self, torch, count, fence="none"):
        import ctypes
        self.torch, self.fence = torch, fence
        if fence == "system":
            self.pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                          for _ in range(count)]
            cur = torch.cuda.current_stream()
            for a, b in self.pairs:  # create them
                a.record(cur)
                b.record(cur)
            return
        path = next((line.split()[-1] for line in open("/proc/self/maps") if "libamdhip64" in line), None)
        if path is None:
            raise RuntimeError("no HIP runtime (libamdhip64) is loaded; use --event-fence system")
        self.hip = ctypes.CDLL(path)
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        self.pairs = []
        for _ in range(count):
            pair = []
            for _ in range(2):
                h = ctypes.c_void_p()
                if self.hip.hipEventCreateWithFlags(ctypes.byref(h), self.DISABLE_SYSTEM_FENCE) != 0:
                    raise RuntimeError("hipEventCreateWithFlags failed")
                # recorded once here, so that the runtime's first-use work on
                # an event happens before the timed region, not inside it
                if self.hip.hipEventRecord(h, stream) != 0:
                    raise RuntimeError("hipEventRecord failed")
                pair.append(h)
            self.pairs.append(tuple(pair))

    def arm(self, ctx, i):
        """The next kernel ctx launches records pair i at its start and end."""
        a, b = self.pairs[i]
        if self.fence == "system":
            ctx.time_next(a, b)
        else:
            import cg_streaming_vector_amd as bs
            bs._check(bs._lib().bs_ctx_time_next(ctx.handle, a, b), "bs_ctx_time_next")

    def mean_seconds(self):
        """Average kernel time over the pairs (call after the stream has synchronised)."""
        import ctypes
        if self.fence == "system":
            return float(np.mean([a.elapsed_time(b) for a, b in self.pairs])) * 1e-3
        ms = []
        for a, b in self.pairs:
            f = ctypes.c_float()
            if self.hip.hipEventElapsedTime(ctypes.byref(f), a, b) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            ms.append(f.value)
        return float(np.mean(ms)) * 1e-3

    def close(self):
        if self.fence != "system":
            for pair in self.pairs:
                for h in pair:
                    self.hip.hipEventDestroy(h)
        self.pairs = []


def kernel_source_sha():
    path = os.path.join(ROOT, "cg_streaming_vector_amd", "csrc", "bs_kernels.hip")
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


class Mesh:
    """Device tables and vectors of one mesh workload, one set per operation.

    With layout "arena" every array of the set comes from one allocation, in
    the order below (each operation's arrays adjacent), on 2 MB boundaries;
    with "torch" each array is a separate torch allocation."""

    # (attribute, source) in arena order; source: host array name or ("empty", length kind)
    ORDER = ["copy_x", "copy_y", "axpy_x", "axpy_y", "norm_x", "dot_x", "dot_y", "cg_p", "cg_q", "cg_x",
             "cg_r", "l2g", "sc_vg", "sc_vl", "off", "ids", "plan", "ga_vl", "ga_vg", "out"]

    def __init__(self, bs, torch, dev, name, E, N, gather_lds, layout="arena", tables=None, plan_region=0):
        """A box of E^3 elements of order N, or, with tables = (l2g, n_global),
        any mesh whose I_l->g is given. plan_region > 0: the gather plan
        places its blocks by mesh region (a local layout made by
        bs_mesh_xcd_interleave with runs of plan_region entries)."""
        self.name, self.E, self.N = name, E, N
        self.torch, self.dev, self.layout = torch, dev, layout
        if tables is None:
            ep, npm = bs_inputs.mesh_perms(name, E, N)
            self.nl, self.ng = bs.bs_mesh_box_count(E, E, E, N)
            l2g = bs.bs_mesh_box_l2g(E, E, E, N, ep, npm)
        else:
            l2g, self.ng = tables
            self.nl = l2g.size
        off, ids = bs.bs_index_g2l(l2g, self.ng)
        plan = bs.bs_gather_plan(off, GATHER_NPB, ids, plan_region)
        v = bs_inputs.vectors(name, self.ng)
        b = bs_inputs.base_seed(name)
        self.gather_lds = gather_lds
        n, nl = self.ng, self.nl
        # per-operation arrays (distinct, so no operation finds another's data in cache)
        host = {"copy_x": v["x"], "copy_y": ("f64", n), "axpy_x": v["p"], "axpy_y": v["y"], "norm_x": v["q"],
                "dot_x": v["r"], "dot_y": v["x"], "cg_p": v["p"], "cg_q": v["q"], "cg_x": v["x"], "cg_r": v["r"],
                "l2g": l2g, "sc_vg": v["y"], "sc_vl": ("f64", nl), "off": off, "ids": ids, "plan": plan,
                "ga_vl": bs_inputs.uniform_pm1(b + 9, nl), "ga_vg": ("f64", n), "out": np.zeros(4)}
        self._materialize({k: (torch.from_numpy(np.ascontiguousarray(h)) if not isinstance(h, tuple) else h)
                           for k, h in host.items()})
        del v, host

    def _materialize(self, src):
        """Place every array of ORDER on the device from src (tensors or ("f64", n))."""
        torch = self.torch
        def nbytes(x):
            return x[1] * 8 if isinstance(x, tuple) else x.numel() * x.element_size()
        if self.layout == "arena":
            from cg_streaming_vector_amd.arena import Arena
            arena = Arena(sum(Arena.slot(nbytes(src[k])) for k in self.ORDER), self.dev)
            for k in self.ORDER:
                x = src[k]
                setattr(self, k, arena.empty(x[1], torch.float64) if isinstance(x, tuple) else arena.put(x))
            self._arena = arena
        else:
            for k in self.ORDER:
                x = src[k]
                setattr(self, k, torch.empty(x[1], dtype=torch.float64, device=self.dev) if isinstance(x, tuple)
                        else x.to(self.dev).clone())

    def clone(self):
        """Another set of the same device arrays (fresh memory, same values)."""
        m = object.__new__(Mesh)
        m.__dict__.update({k: v for k, v in self.__dict__.items() if k not in self.ORDER and k != "_arena"})
        m._materialize({k: getattr(self, k) for k in self.ORDER})
        return m

    def launchers(self, bs, stream):
        """op -> zero-argument callable issuing that op through the C ABI."""
        L, h = bs._lib(), bs.context().handle
        n, nl, ng = self.ng, self.nl, self.ng
        P = lambda t: t.data_ptr()  # noqa: E731
        o = P(self.out)
        plan = P(self.plan) if self.gather_lds else None
        nb = self.plan.shape[0] if self.gather_lds else 0
        a = dict(
            copy=(L.bs_copy, (h, n, P(self.copy_x), P(self.copy_y), stream)),
            axpy=(L.bs_axpy, (h, n, 0.37, P(self.axpy_x), 1.0, P(self.axpy_y), stream)),
            norm=(L.bs_norm, (h, n, P(self.norm_x), o, stream)),
            dot=(L.bs_dot, (h, n, P(self.dot_x), P(self.dot_y), o + 8, stream)),
            cg_update=(L.bs_cg_update, (h, n, 0.37, P(self.cg_p), P(self.cg_q), P(self.cg_x), P(self.cg_r),
                                        o + 16, stream)),
            scatter=(L.bs_scatter, (h, nl, P(self.l2g), P(self.sc_vg), P(self.sc_vl), stream)),
            gather=(L.bs_gather, (h, ng, P(self.off), P(self.ids), P(self.ga_vl), P(self.ga_vg), plan, nb,
                                  stream)),
        )

        def mk(fn, args, op):
            def call():
                s = fn(*args)
                if s != 0:
                    raise RuntimeError(f"bs_{op} returned {s}")
            return call
        return {op: mk(fn, args, op) for op, (fn, args) in a.items()}

    def bench_set(self, op):
        """(n, tensors, n_blocks) of this set for bs_bench_loop."""
        plan = self.plan if self.gather_lds else None
        return {
            "copy": (self.ng, (self.copy_x, self.copy_y), 0),
            "axpy": (self.ng, (self.axpy_x, self.axpy_y), 0),
            "norm": (self.ng, (self.norm_x,), 0),
            "dot": (self.ng, (self.dot_x, self.dot_y), 0),
            "cg_update": (self.ng, (self.cg_p, self.cg_q, self.cg_x, self.cg_r), 0),
            "scatter": (self.nl, (self.l2g, self.sc_vg, self.sc_vl), 0),
            "gather": (self.ng, (self.off, self.ids, self.ga_vl, self.ga_vg, plan),
                       self.plan.shape[0] if self.gather_lds else 0),
        }[op]

    def bytes(self, op):
        return op_bytes(op, self.ng, self.nl, self.ng)


def time_ops_native(bs, sets, ops, reps, trials=1):
    """Average host-timed seconds per launch of each op: `reps` launches
    issued back to back by the library's C++ loop, cycling through the
    distinct array sets `sets` (Mesh objects) so that no launch finds its
    operands in cache. With trials > 1, returns op -> list of the trials'
    averages."""
    out = {}
    for op in ops:
        n, _, nb = sets[0].bench_set(op)
        groups = [m.bench_set(op)[1] for m in sets]
        res_t = sets[0].out[:1]
        bs.bs_bench_loop(op, n, groups, len(groups), res_t, n_blocks=nb)  # one pass to warm up
        res = [bs.bs_bench_loop(op, n, groups, reps, res_t, n_blocks=nb) / reps for _ in range(trials)]
        out[op] = res if trials > 1 else res[0]
    return out


def copy_ceiling(bs, torch, dev, k=28):
    """GB/s of the library's own copy at 2^k doubles (two array pairs used in
    turn, 4.3 GB per pair at k = 28): the best sustained mixed read+write rate
    this memory system gave any kernel here."""
    n = 1 << k
    pairs = [(torch.empty(n, dtype=torch.float64, device=dev), torch.empty(n, dtype=torch.float64, device=dev))
             for _ in range(2)]
    for a, _ in pairs:
        a.uniform_(-1, 1)
    bs.bs_bench_loop("copy", n, pairs, 4)
    t = min(bs.bs_bench_loop("copy", n, pairs, 20) / 20 for _ in range(3))
    del pairs
    torch.cuda.empty_cache()
    return 16 * n / t / 1e9


def traffic_for(kernels):
    """HBM bytes per launch of an operation (the sum over its kernels) from the
    committed rocprofv3 --pmc summary, if the kernel source has not changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic_box32_N7.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except ValueError:
        return None
    if d.get("kernel_source_sha256") != kernel_source_sha():
        return None
    total = 0.0
    for kernel in kernels:
        k = d.get("kernels", {}).get(kernel)
        if not k or "hbm_bytes_per_launch" not in k:
            return None
        total += float(k["hbm_bytes_per_launch"])
    return total


def _oracle_steps(h, budget_s):
    """Full oracle steps on the host arrays until about budget_s seconds;
    returns (steps, seconds)."""
    import oracle
    n = h["ng"]
    reps, t = 0, 0.0
    while t < budget_s and reps < 1000:
        t0 = time.perf_counter()
        oracle.copy(h["x"])
        oracle.axpy(0.37, h["p"], 1.0, h["y"])
        oracle.norm(h["q"])
        oracle.dot(h["r"], h["x"])
        oracle.cg_update(0.37, h["p"], h["q"], h["x"], h["r"])
        oracle.scatter(h["l2g"], h["y"])
        oracle.gather(h["l2g"], h["vl"], n)
        t += time.perf_counter() - t0
        reps += 1
    return reps, t


def cpu_baseline(mesh_host, budget_s=12.0, budget_1_thread_s=4.0):
    """The oracle, as it stands, on the same step (host arrays), repeated
    until about budget_s seconds on all of the host's OpenMP threads, then
    for about budget_1_thread_s on one; GB/s over the algorithmic bytes."""
    import oracle
    h = mesh_host
    n = h["ng"]
    nb = sum(op_bytes(op, n, h["nl"], n) for op in OPS)
    threads = oracle.threads()
    reps, t = _oracle_steps(h, budget_s)
    oracle.set_threads(1)
    try:
        reps1, t1 = _oracle_steps(h, budget_1_thread_s)
    finally:
        oracle.set_threads(threads)
    model = "unknown CPU"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"value": round(nb * reps / t / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{reps} steps (7 ops, 32^3 N=7), {t:.1f} s, {threads} OpenMP threads, {model[:16]}",
            "affinity_cpus": affinity, "value_1_thread": round(nb * reps1 / t1 / 1e9, 3)}


SWEEP_OPS = ["copy", "axpy", "norm", "dot", "cg_update"]
SWEEP_ARITY = {"copy": 2, "axpy": 2, "norm": 1, "dot": 2, "cg_update": 4}


def sweep_sets(torch, dev, n, R, layout):
    """R sets of four vectors of n doubles, uniform [-1, 1). "arena": each
    set is one allocation whose arrays sit on 2 MB boundaries, each followed
    by one unused 2 MB granule, so that no two operands of power-of-two
    length are a power of two apart (the step's own arrays sit on 2 MB
    boundaries at distances of 92 MB). "torch": each vector a separate torch
    allocation."""
    from cg_streaming_vector_amd.arena import Arena
    sets = []
    for _ in range(R):
        if layout == "arena":
            a = Arena(4 * (Arena.slot(8 * n) + Arena.slot(1)), dev)
            vs = [a.empty(n, torch.float64, pad=1) for _ in range(4)]
        else:
            vs = [torch.empty(n, dtype=torch.float64, device=dev) for _ in range(4)]
        for v in vs:
            v.uniform_(-1, 1)
        sets.append(vs)
    return sets


def sweep(bs, torch, dev, reps_min=100, min_seconds=0.05, ks=range(10, 29), layout="arena"):
    """The size sweep: each vector op over n = 2^k, fitted to T(B) = T0 + B/W_max
    (eq. 8). The launches of each point are issued by the library's C++ loop
    (bs_bench_loop), timed on the host around the whole run as the pages time
    it; at least reps_min launches and min_seconds per point, cycling through
    enough sets (>= 1 GiB of footprint) that every launch reads cold data.
    Returns per op: the points, the fit (T0, W_max, B_0.8, R^2 of the
    bandwidth), each point's relative bandwidth residual (measured - model) /
    measured, and the measured plateau (median GB/s of the points of at least
    0.5 GB)."""
    stream = torch.cuda.current_stream().cuda_stream
    res = {op: [] for op in SWEEP_OPS}
    out = torch.zeros(1, dtype=torch.float64, device=dev)
    for k in ks:
        n = 1 << k
        R = min(64, max(2, int(np.ceil(2 ** 30 / (32 * n)))))
        sets = sweep_sets(torch, dev, n, R, layout)
        for op in res:
            groups = [tuple(s[:SWEEP_ARITY[op]]) for s in sets]
            w = max(R, 8)
            bs.bs_bench_loop(op, n, groups, w, out, stream=stream)  # warm-up
            t_one = bs.bs_bench_loop(op, n, groups, w, out, stream=stream) / w
            reps = max(reps_min, R, int(np.ceil(min_seconds / max(t_one, 1e-7))))
            T = bs.bs_bench_loop(op, n, groups, reps, out, stream=stream) / reps
            res[op].append((op_bytes(op, n), T))
        del sets
        torch.cuda.empty_cache()
    return {op: sweep_fit(pts) for op, pts in res.items()}


def sweep_fit(pts):
    """Eq. 8 fitted to one operation's (bytes, seconds) points, with each
    point's relative bandwidth residual (measured - model) / measured and the
    measured plateau: the median GB/s of the points of at least 0.5 GB."""
    from cg_streaming_vector_amd.model import fit_streaming_model, w_eff
    B = np.array([p[0] for p in pts], dtype=np.float64)
    T = np.array([p[1] for p in pts], dtype=np.float64)
    f = fit_streaming_model(B, T)
    W = B / T
    resid = (W - w_eff(B, f["T0_s"], f["W_max"])) / W
    big = W[B >= 0.5e9]
    return {"points": [[int(b), float(t)] for b, t in pts], **f,
            "rel_residuals": [round(float(x), 4) for x in resid],
            "plateau_GBps": round(float(np.median(big)) / 1e9, 1) if big.size else None}


SWEEP_FIELDS = ["T0_us", "W_max_GBps", "B_08_MB", "r2", "max_abs_rel_residual", "plateau_GBps"]


def sweep_summary(fits):
    """The compact per-op figures of a sweep for the benchmark's JSON line
    (values in the order of SWEEP_FIELDS)."""
    return {op: [round(f["T0_s"] * 1e6, 2), round(f["W_max_GBps"], 1), round(f["B_08_bytes"] / 1e6, 1),
                 round(f["r2_bandwidth"], 4), round(max(abs(x) for x in f["rel_residuals"]), 3),
                 f["plateau_GBps"]] for op, f in fits.items()}


XCD_CHUNK = 64  # elements per run of the XCD-interleaved storage order


def tet_split_tables(bs, cubes, N, seed, order="gen"):
    """I_l->g of the unstructured tet-split mesh (cubes^3 unit cubes, 24
    hexahedra each, every element in a random orientation), with its elements
    stored in the generator's order (cube by cube, x fastest: "gen"), in a
    random order, as a mesh file might present them ("shuffled"), in that
    random order put back along the library's Hilbert curve through the
    element centroids (bs_mesh_hex_order: "curve"), or in the generator's
    order cut into eight regions interleaved in runs of XCD_CHUNK elements
    (bs_mesh_xcd_interleave: "xcd"; its gather plan places blocks by region).
    Global ids are numbered by first appearance in storage order, so they
    follow the element order."""
    ev, nv, coords = bs_inputs.hex_tet_split(cubes, cubes, cubes)
    ev, _ = bs_inputs.hex_orient(ev, seed)
    if order in ("shuffled", "curve"):
        ev = np.ascontiguousarray(ev[bs_inputs.permutation(seed + 1, len(ev))])
    if order == "curve":
        ev = np.ascontiguousarray(ev[bs.bs_mesh_hex_order(coords[ev])])
    if order == "xcd":
        ev = np.ascontiguousarray(ev[bs.bs_mesh_xcd_interleave(len(ev), XCD_CHUNK)])
    return bs.bs_mesh_hex_l2g(ev, N, nv)


WORKLOADS = ["shuffled40_N5", "tetsplit11_N7", "tetsplit11_N7_xcd", "tetsplit11_N7_shuffled", "tetsplit11_N7_curve",
             "slab32x32x4_N7", "box24_N15", "cg_box32_N7"]


def workloads(bs, torch, dev, gather_lds, steps=30, only=None):
    """The shuffled 40^3 order-5 mesh (scatter, gather), the unstructured
    tet-split mesh of 11^3 cubes (31944 hexahedra) at order 7 (scatter,
    gather) with its elements in the generator's order, interleaved by region
    for the XCDs, in a random order, and in that random order put back along
    the Hilbert curve, one GPU's share of the 32^3 order-7 mesh cut into eight z-slabs
    (32 x 32 x 4 elements, all 7 ops, and the CG streaming sequence, whose
    device-resident iteration there fits in the last-level cache), the 24^3
    order-15 mesh (all 7 ops, and the CG streaming sequence) and the CG
    streaming sequence alone on the 32^3 order-7 mesh (whose r and p, but not
    the whole iteration, fit in the last-level cache; the step already times
    its seven operations)."""
    out = {}
    for name, E, N, ops in [("shuffled40_N5", 40, 5, ["scatter", "gather"]),
                            ("tetsplit11_N7", 11, 7, ["scatter", "gather"]),
                            ("tetsplit11_N7_xcd", 11, 7, ["scatter", "gather"]),
                            ("tetsplit11_N7_shuffled", 11, 7, ["scatter", "gather"]),
                            ("tetsplit11_N7_curve", 11, 7, ["scatter", "gather"]),
                            ("slab32x32x4_N7", 32, 7, OPS),
                            ("box24_N15", 24, 15, OPS),
                            ("cg_box32_N7", 32, 7, [])]:
        if only and name not in only:
            continue
        tables = None
        if name.startswith("tetsplit"):
            tables = tet_split_tables(bs, E, N, bs_inputs.base_seed("tetsplit11_N7") + bs_inputs.SEED_ELEM,
                                      order={"tetsplit11_N7_shuffled": "shuffled", "tetsplit11_N7_curve": "curve",
                                             "tetsplit11_N7_xcd": "xcd"}.get(name, "gen"))
        elif name.startswith("slab"):
            tables = (bs.bs_mesh_box_l2g(E, E, 4, N), bs.bs_mesh_box_count(E, E, 4, N)[1])
        # the CG-only workload runs on the step's own mesh and inputs
        src = "box32_N7" if name == "cg_box32_N7" else "tetsplit11_N7" if name.startswith("tetsplit") else name
        region = XCD_CHUNK * (N + 1) ** 3 if name.endswith("_xcd") else 0
        m = Mesh(bs, torch, dev, src, E, N, gather_lds, tables=tables, plan_region=region)
        if tables is not None:
            out[name + "_mesh"] = {"elements": 24 * E ** 3 if name.startswith("tetsplit") else E * E * 4, "order": N,
                                   "n_local": m.nl, "n_global": m.ng}
        if ops:
            # rotated sets: >= 1 GB through the cache between two touches
            R = 3 if name.startswith("box24") else 48 if name.startswith("slab") else 5
            sets = [m] + [m.clone() for _ in range(R - 1)]
            per_op = time_ops_native(bs, sets, ops, max(3 * R, 96))
            del sets
            res = {op: {"bytes": m.bytes(op), "us": round(per_op[op] * 1e6, 2),
                        "GBps": round(m.bytes(op) / per_op[op] / 1e9, 1),
                        "pct_peak": round(100 * m.bytes(op) / per_op[op] / 1e9 / PEAK_GBPS, 1)} for op in ops}
            out[name] = res
        if name in ("box24_N15", "slab32x32x4_N7", "cg_box32_N7"):
            out["cg_sequence_" + name] = cg_sequence(bs, torch, dev, m)
        del m
        torch.cuda.empty_cache()
    return out


def cg_sequence(bs, torch, dev, m, iters=100):
    """CG-iteration streaming sequence on Z^T Z: scatter, gather, dot, fused
    update, AXPY. (i) fixed scalars, no readback, `iters` iterations; (ii) true
    CG, 4 iterations, reading alpha and beta back to the host."""
    L, h = bs._lib(), bs.context().handle
    st = torch.cuda.current_stream().cuda_stream
    ng, nl = m.ng, m.nl
    P = lambda t: t.data_ptr()  # noqa: E731
    b = m.cg_r
    x, r, p = torch.zeros_like(b), b.clone(), b.clone()
    q, pl = torch.empty_like(b), m.sc_vl
    o = torch.zeros(2, dtype=torch.float64, device=dev)
    plan = P(m.plan) if m.gather_lds else None
    nb = m.plan.shape[0] if m.gather_lds else 0

    def it(alpha, beta):
        assert L.bs_scatter(h, nl, P(m.l2g), P(p), P(pl), st) == 0
        assert L.bs_gather(h, ng, P(m.off), P(m.ids), P(pl), P(q), plan, nb, st) == 0
        assert L.bs_dot(h, ng, P(p), P(q), P(o), st) == 0
        assert L.bs_cg_update(h, ng, alpha, P(p), P(q), P(x), P(r), P(o) + 8, st) == 0
        assert L.bs_axpy(h, ng, 1.0, P(r), beta, P(p), st) == 0

    per_iter = 24 * nl + 108 * ng
    for _ in range(3):
        it(1e-3, 0.5)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(iters):
        it(1e-3, 0.5)
    torch.cuda.synchronize()
    T = (time.perf_counter() - t0) / iters
    # true CG with readbacks
    x.zero_()
    r.copy_(b)
    p.copy_(b)
    assert L.bs_dot(h, ng, P(r), P(r), P(o) + 8, st) == 0
    rr0 = rr = o[1].item()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(4):
        assert L.bs_scatter(h, nl, P(m.l2g), P(p), P(pl), st) == 0
        assert L.bs_gather(h, ng, P(m.off), P(m.ids), P(pl), P(q), plan, nb, st) == 0
        assert L.bs_dot(h, ng, P(p), P(q), P(o), st) == 0
        alpha = rr / o[0].item()
        assert L.bs_cg_update(h, ng, alpha, P(p), P(q), P(x), P(r), P(o) + 8, st) == 0
        rr_new = o[1].item()
        assert L.bs_axpy(h, ng, 1.0, P(r), rr_new / rr, P(p), st) == 0
        rr = rr_new
    torch.cuda.synchronize()
    Tcg = (time.perf_counter() - t0) / 4
    # device-resident CG (alpha, beta on the device, p.q fused into the
    # gather): K iterations, no host synchronisation; tolerance 0 so every
    # iteration runs (after the 4th the values are rounding noise, the
    # traffic is the same). Bytes actually moved per iteration:
    # scatter 12 N_L + 8 N_G, gather + p.q 12 N_L + 20 N_G, update 48 N_G,
    # p update 24 N_G.
    K = 40
    fused_iter = 24 * nl + 100 * ng
    hist = torch.empty(K + 1, dtype=torch.float64, device=dev)
    plan_t = m.plan if m.gather_lds else None
    for _ in range(2):
        x.zero_()
        r.copy_(b)
        p.copy_(b)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        bs.bs_cg_solve(m.l2g, m.off, m.ids, x, r, p, q, pl, K, 0.0, plan_t, hist)
        torch.cuda.synchronize()
        Tdev = (time.perf_counter() - t0) / K
    h4 = hist[:5].cpu().numpy()
    return {"bytes_per_iter": per_iter, "fixed_scalars_us_per_iter": round(T * 1e6, 1),
            "fixed_scalars_GBps": round(per_iter / T / 1e9, 1),
            "true_cg_us_per_iter": round(Tcg * 1e6, 1), "true_cg_GBps": round(per_iter / Tcg / 1e9, 1),
            "true_cg_rel_residual_after_4": float(np.sqrt(rr / rr0)),
            "device_cg_us_per_iter": round(Tdev * 1e6, 1), "device_cg_bytes_per_iter": fused_iter,
            "device_cg_GBps_moved": round(fused_iter / Tdev / 1e9, 1),
            "device_cg_GBps_unfused_bytes": round(per_iter / Tdev / 1e9, 1),
            "device_cg_rel_residual_after_4": float(np.sqrt(h4[4] / h4[0]))}


def workload_summary(wl):
    """Compact figures of the other workloads for the JSON line: per mesh and
    operation [us, % of 8 TB/s]; per CG sequence [device-resident, host-driven
    with fixed scalars, true CG with readbacks] in us per iteration, and the
    device-resident iteration's GB/s of bytes actually moved."""
    out = {}
    for name, r in wl.items():
        # the slab share and the tet-split mesh in other element orders stay in --out
        if name.endswith("_mesh") or "slab" in name or name.endswith(("_shuffled", "_curve")):
            continue
        if name.startswith("cg_sequence_"):
            out["cg_" + name[len("cg_sequence_"):].replace("cg_", "")] = [
                r["device_cg_us_per_iter"], r["fixed_scalars_us_per_iter"], r["true_cg_us_per_iter"],
                r["device_cg_GBps_moved"]]
        else:
            out[name] = {op: [v["us"], v["pct_peak"]] for op, v in r.items()}
    out["fields"] = "op: [us, %peak]; cg_*: [device, fixed-scalar, true-CG us/iter, device GB/s]"
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--gather", choices=["span", "lds"], default="lds",
                    help="lds: the gather with a blockStarts plan; span: without a plan (fixed spans of 512 rows)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy-ceiling", action="store_true", help="skip the 2^28-double copy (profiling runs)")
    ap.add_argument("--rotate", type=int, default=12, help="array sets cycled in the per-op loops")
    ap.add_argument("--layout", choices=["arena", "torch"], default="arena",
                    help="arena: each set's arrays packed in one allocation on 2 MB boundaries")
    ap.add_argument("--per-op-reps", type=int, default=96)
    ap.add_argument("--trials", type=int, default=5, help="per-op loops repeated; the median is reported")
    ap.add_argument("--event-fence", choices=["none", "system"], default="none",
                    help="timing events of the dominant kernel: none = created with hipEventDisableSystemFence, "
                         "system = torch's events (a system-scope fence each)")
    ap.add_argument("--event-stride", type=int, default=None,
                    help="the dominant kernel records its timing events in every this many timed steps "
                         f"(default {EVENT_STRIDE}, less when that would time fewer than {MIN_TIMED_LAUNCHES} launches)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the size sweep and the other workloads (profiling runs of the step)")
    ap.add_argument("--sweep-layout", choices=["arena", "torch"], default="arena",
                    help="arena: each sweep set in one allocation, arrays 2 MB-aligned and staggered")
    ap.add_argument("--out", default=None)
    ap.add_argument("--workload", action="append", choices=WORKLOADS, default=[],
                    help="time only this workload (repeatable; skips the step; for profiling one mesh at a time)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the BS operations here run on a single MI355X. Across GPUs "
              "each global vector would split into per-GPU slices and the mesh into z-slabs, with one "
              "partial per reduction and the slab-plane interface nodes exchanged; that exchange is not "
              "built. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import cg_streaming_vector_amd as bs
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a HIP device")
    dev = torch.device("cuda:0")
    bs._lib()
    ctx = bs.context(0)
    if args.workload:
        res = workloads(bs, torch, dev, args.gather == "lds", only=args.workload)
        if args.out:
            with open(args.out, "w") as f:
                json.dump({"workloads": res}, f, indent=1)
        print(json.dumps({"workloads": res}), flush=True)
        return

    name, E, N = "box32_N7", 32, 7
    mesh = Mesh(bs, torch, dev, name, E, N, gather_lds=(args.gather == "lds"), layout=args.layout)
    stream = torch.cuda.current_stream().cuda_stream
    step_bytes = sum(mesh.bytes(op) for op in OPS)

    # per operation: back-to-back launches over ROT sets of distinct arrays
    # (ROT x the smallest operation's bytes > 1 GB, beyond the 256 MB cache)
    sets = [mesh] + [mesh.clone() for _ in range(args.rotate - 1)]
    trials = time_ops_native(bs, sets, OPS, args.per_op_reps, trials=args.trials)
    per_op = {op: float(np.median(t)) for op, t in trials.items()}
    dom = max(OPS, key=lambda op: per_op[op])
    # the same loops on one set (only ordinary-policy reads can hit the 256 MB cache)
    hot = time_ops_native(bs, [mesh], OPS, args.per_op_reps)

    # timed region: host clock around K steps; step k runs on array set
    # k mod ROT, so that every operation of a step reads data no step has
    # touched for ROT - 1 steps (about 21 GB of traffic): cold in the cache,
    # as in the per-operation loops. In every EVENT_STRIDE-th step the
    # dominant kernel records a pair of HIP events at its own start and end
    # (the library launches it with them, as armed by time_next), on its
    # stream. The events are fence-free (TimingEvents); even so a timed
    # launch costs its step about 1 us (events in every step: 319.9 against
    # 319.2 us per step), so by default every fourth step carries them; a
    # run of fewer than 40 steps times more of its steps (20 steps: every
    # second one), since an average of five launches moves by a few percent
    # from run to run.
    step_launch = [m.launchers(bs, stream) for m in sets]
    for w in range(args.warmup):
        for op in OPS:
            step_launch[w % len(sets)][op]()
    cur = torch.cuda.current_stream()
    stride = args.event_stride or max(1, min(EVENT_STRIDE, args.steps // MIN_TIMED_LAUNCHES))
    ev = TimingEvents(torch, (args.steps + stride - 1) // stride, args.event_fence)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        run = step_launch[k % len(sets)]
        for op in OPS:
            if op == dom and k % stride == 0:
                ev.arm(ctx, k // stride)
            run[op]()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    del step_launch, sets
    torch.cuda.empty_cache()
    dom_live = ev.mean_seconds()
    n_timed = len(ev.pairs)
    ev.close()
    ms_step = dt / args.steps * 1e3
    value = step_bytes / (dt / args.steps) / 1e9

    # (profiling runs leave it out, so that the trace holds only this mesh's launches)
    ceiling = None if args.no_copy_ceiling else copy_ceiling(bs, torch, dev)
    ops_out = {}
    for op in OPS:
        t = per_op[op]
        gbps = mesh.bytes(op) / t / 1e9
        ops_out[op] = [mesh.bytes(op), round(t * 1e6, 2), round(min(trials[op]) * 1e6, 2), round(gbps, 1),
                       round(100 * gbps / PEAK_GBPS, 1), round(100 * gbps / ceiling, 1) if ceiling else None,
                       round(hot[op] * 1e6, 2)]
    achieved = mesh.bytes(dom) / dom_live / 1e9
    traffic = traffic_for(KERNEL_NAME[dom])
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_GBPS, 4), "traffic": traffic,
                "op": dom, "kernel": " + ".join(KERNEL_NAME[dom]), "bytes_per_launch": mesh.bytes(dom),
                "us_per_launch": round(dom_live * 1e6, 2), "launches_timed": n_timed,
                "event_fence": args.event_fence}

    # the runtime's own device-to-device copy at this size, on rotated buffers
    R = args.rotate
    src = [mesh.copy_x.clone() for _ in range(R)]
    dst = [torch.empty_like(mesh.copy_x) for _ in range(R)]
    for i in range(R):
        dst[i].copy_(src[i])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(cur)
    for i in range(args.per_op_reps):
        dst[i % R].copy_(src[i % R])
    e1.record(cur)
    e1.synchronize()
    rt_copy = 16 * mesh.ng / (e0.elapsed_time(e1) * 1e-3 / args.per_op_reps) / 1e9
    del src, dst

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64",
        "data": "synthetic (seeded SplitMix64 uniform[-1,1) vectors, structured box mesh)",
        "config": {"workload": "box mesh 32^3 elements, order N=7, lexicographic numbering; "
                               "all 7 BS ops per step", "elements": E ** 3, "order": N,
                   "n_global": mesh.ng, "n_local": mesh.nl, "step_bytes": step_bytes,
                   "gather_kernel": args.gather, "layout": args.layout, "step_sets": args.rotate,
                   "cu_count": ctx.info()["cu_count"]},
        "pct_peak": round(100 * value / PEAK_GBPS, 1),
        "per_op": ops_out,
        "per_op_fields": PER_OP_FIELDS,
        "runtime_copy_GBps": round(rt_copy, 1),
        "copy_ceiling_GBps": round(ceiling, 1) if ceiling else None,
        "per_op_note": f"median of {args.trials}x{args.per_op_reps} launches, {args.rotate} cold sets; hot: 1 set",
        "roofline": roofline,
    }

    # Outside the timed region: the size sweep with its eq. 8 fit, and the
    # other meshes and the CG sequence. Their compact figures join the line;
    # --out keeps everything.
    extra = {}
    if not args.no_extras:
        t_x = time.perf_counter()
        fits = sweep(bs, torch, dev, layout=args.sweep_layout)
        extra["sweep"] = fits
        line["sweep_fit"] = sweep_summary(fits)
        line["sweep_fit_fields"] = SWEEP_FIELDS
        line["sweep_fit_note"] = f"n=2^10..2^28 ({args.sweep_layout}); eq. 8; plateau: median of >= 0.5 GB"
        wl = workloads(bs, torch, dev, args.gather == "lds")
        extra["workloads"] = wl
        line["workloads"] = workload_summary(wl)
        line["extras_s"] = round(time.perf_counter() - t_x, 1)

    if not args.no_cpu_baseline:
        import oracle
        host = {"ng": mesh.ng, "nl": mesh.nl}
        v = bs_inputs.vectors(name, mesh.ng)
        host.update(v)
        ol2g, _ = oracle.mesh_box(E, E, E, N)
        host["l2g"] = ol2g
        host["vl"] = bs_inputs.uniform_pm1(bs_inputs.base_seed(name) + 9, mesh.nl)
        line["cpu_baseline"] = cpu_baseline(host)
    else:
        line["cpu_baseline"] = None

    if args.out:
        with open(args.out, "w") as f:
            json.dump({"bench": line, **extra}, f, indent=1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
