"""Summaries of rocprofv3 output for the BS kernels.

Reads the CSV files that ``rocprofv3 --kernel-trace --stats`` and
``rocprofv3 --pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` write, and turns them
into the short text summaries kept with the sources: average duration per
kernel, and HBM bytes per launch.

FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are calibrated against a plain
copy kernel of known size: on a copy of n doubles the true traffic is 8n bytes
read and 8n bytes written, and the ratio of that to what each counter reports
is the scale applied to every other kernel's reading. On MI355X the read
counter reports half the bytes of the copy and the write counter all of them.

Any other counters (``--pmc`` files of several runs) are summarised as plain
per-kernel averages per dispatch.

Usage:
  python -m cg_streaming_vector_amd.profiling --stats S.csv --fetch F.csv \\
      --write W.csv --copy-kernel 'k_copy<1, 768>' --copy-doubles 11390625 \\
      --source cg_streaming_vector_amd/csrc/bs_kernels.hip --json out.json --md out.md
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import statistics


def short_name(kernel: str) -> str:
    """'void (anonymous namespace)::k_dot<2, true>(Split, ...)' -> 'k_dot<2, true>'."""
    k = kernel.strip()
    if k.startswith("void "):
        k = k[5:]
    k = k.replace("(anonymous namespace)::", "")
    depth = 0
    for i, ch in enumerate(k):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return k[:i].strip()
    return k


def load_stats(path):
    """kernel -> (calls, average ns) from a *_kernel_stats.csv file."""
    out = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            out[short_name(row["Name"])] = (int(row["Calls"]), float(row["AverageNs"]))
    return out


def load_counter(path, counter):
    """kernel -> list of per-dispatch values of one counter."""
    out = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            out.setdefault(short_name(row["Kernel_Name"]), []).append(float(row["Counter_Value"]))
    return out


def load_counters(paths, kernels=None):
    """kernel -> counter -> list of per-dispatch values, over several
    *_counter_collection.csv files (one counter set per rocprofv3 run);
    kernels, if given, keeps only those short names."""
    out = {}
    for path in paths:
        with open(path) as f:
            for row in csv.DictReader(f):
                k = short_name(row["Kernel_Name"])
                if kernels and k not in kernels:
                    continue
                out.setdefault(k, {}).setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
    return out


def counters_markdown(table, title, commands):
    """Average per dispatch of every counter, one table per kernel."""
    lines = [f"# {title}", "", "Commands:", ""]
    lines += [f"    {c}" for c in commands]
    for k in sorted(table):
        lines += ["", f"`{k}`:", "", "| counter | dispatches | average per dispatch |", "|---|---|---|"]
        for c in sorted(table[k]):
            v = table[k][c]
            lines.append(f"| {c} | {len(v)} | {statistics.fmean(v):.6g} |")
    return "\n".join(lines) + "\n"


def load_resources(path):
    """kernel -> LDS, scratch and launch shape from a *_kernel_trace.csv file
    (the first dispatch of each kernel; the largest grid seen). Register
    counts are taken from the compiler's report instead (load_remarks): the
    trace's VGPR field counts allocation granules of 4 registers, while gfx950
    allocates in granules of 8."""
    out = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            k = short_name(row["Kernel_Name"])
            wg = int(row["Workgroup_Size_X"]) * int(row["Workgroup_Size_Y"]) * int(row["Workgroup_Size_Z"])
            grid = int(row["Grid_Size_X"]) * int(row["Grid_Size_Y"]) * int(row["Grid_Size_Z"])
            if k not in out:
                out[k] = {"lds_bytes": int(row["LDS_Block_Size"]), "scratch_bytes": int(row["Scratch_Size"]),
                          "workgroup": wg, "max_workgroups": 0}
            out[k]["max_workgroups"] = max(out[k]["max_workgroups"], grid // max(wg, 1))
    return out


def load_in_step(path, before, kernel, after):
    """Durations (ns) of the launches of `kernel` that a trace shows between a
    launch of `before` and one of `after` on the same queue, in start order:
    the launches inside the timed steps of a benchmark whose step runs the
    kernels in a fixed sequence, without the per-operation loops around them."""
    rows = []
    with open(path) as f:
        for row in csv.DictReader(f):
            rows.append((row.get("Queue_Id", ""), int(row["Start_Timestamp"]), int(row["End_Timestamp"]),
                         short_name(row["Kernel_Name"])))
    rows.sort()
    out = []
    for i in range(1, len(rows) - 1):
        q, t0, t1, k = rows[i]
        if k == kernel and rows[i - 1][0] == q == rows[i + 1][0] and rows[i - 1][3] == before \
                and rows[i + 1][3] == after:
            out.append(t1 - t0)
    return out


REMARK_KEYS = {"TotalSGPRs": "sgpr", "VGPRs": "vgpr", "AGPRs": "agpr", "ScratchSize [bytes/lane]": "scratch_per_lane",
               "Occupancy [waves/SIMD]": "occupancy", "SGPRs Spill": "sgpr_spill", "VGPRs Spill": "vgpr_spill",
               "LDS Size [bytes/block]": "lds_static"}


def load_remarks(path, demangle=None):
    """kernel -> register use, spills and occupancy from the compiler's
    -Rpass-analysis=kernel-resource-usage remarks (hipcc's stderr)."""
    import re
    if demangle is None:
        demangle = _cxxfilt
    out, cur = {}, None
    with open(path) as f:
        for line in f:
            m = re.search(r"Function Name: (\S+)", line)
            if m:
                cur = short_name(demangle(m.group(1)))
                out[cur] = {}
                continue
            m = re.search(r"remark: \s*([^:]+?): (\S+) \[-Rpass-analysis", line)
            if cur and m and m.group(1).strip() in REMARK_KEYS:
                v = m.group(2)
                out[cur][REMARK_KEYS[m.group(1).strip()]] = int(v) if v.isdigit() else v
    return out


def _cxxfilt(name):
    import subprocess
    try:
        return subprocess.run(["c++filt", name], capture_output=True, text=True, check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return name


def summarize(stats_csv, fetch_csv, write_csv, copy_kernel, copy_doubles, source=None, ops=None, trace_csv=None,
              remarks=None, calibration=None, in_step=None):
    """calibration: (fetch_scale, write_scale) to use when the run has no copy
    kernel of its own (taken from an earlier summary's calibration block).
    in_step: {name: (before, kernel, after)}, averaged over the trace's
    launches of kernel between those two neighbours (needs trace_csv)."""
    stats = load_stats(stats_csv) if stats_csv else {}
    res = load_resources(trace_csv) if trace_csv else {}
    rem = load_remarks(remarks) if remarks else {}
    fetch = load_counter(fetch_csv, "FETCH_SIZE") if fetch_csv else {}
    write = load_counter(write_csv, "WRITE_SIZE") if write_csv else {}
    known = 8.0 * copy_doubles
    f_scale = w_scale = None
    if copy_kernel in fetch and copy_kernel in write:
        f_scale = known / (statistics.median(fetch[copy_kernel]) * 1024.0)
        w_scale = known / (statistics.median(write[copy_kernel]) * 1024.0)
        # a copy writes its bytes once: WRITE_SIZE of a copy of the stated
        # size reads back within a few percent, so a scale far from 1 means
        # copy_doubles is not the size the run copied
        if not 0.8 <= w_scale <= 1.25:
            raise ValueError(f"{copy_kernel}: WRITE_SIZE scale {w_scale:.3g} for {copy_doubles} doubles; "
                             "pass the run's copy size (--copy-doubles)")
    reused = False
    if f_scale is None and calibration:
        f_scale, w_scale = calibration
        reused = True
    kernels = {}
    names = set(stats) | set(fetch) | set(write) | set(res)
    for k in sorted(names or set(rem)):
        if k.startswith("__amd") or "at::native" in k:
            continue
        d = {}
        if k in stats:
            d["calls"], d["avg_ns"] = stats[k]
        if k in fetch:
            d["fetch_kib_median"] = statistics.median(fetch[k])
        if k in write:
            d["write_kib_median"] = statistics.median(write[k])
        if k in res:
            d["resources"] = res[k]
        if k in rem:
            d["compiler"] = rem[k]
        if f_scale and k in fetch and k in write:
            d["hbm_bytes_per_launch"] = (d["fetch_kib_median"] * 1024.0 * f_scale
                                         + d["write_kib_median"] * 1024.0 * w_scale)
        kernels[k] = d
    out = {"calibration": {"copy_kernel": copy_kernel, "copy_doubles": copy_doubles,
                           "fetch_scale": f_scale, "write_scale": w_scale, "reused": reused},
           "kernels": kernels}
    if ops:
        # an operation may be several kernels launched back to back (a
        # reduction's first stage and its finish): sum their averages
        out["ops"] = {}
        for name, ks in ops.items():
            if all(k in kernels and "avg_ns" in kernels[k] for k in ks):
                out["ops"][name] = {"kernels": ks, "avg_ns": sum(kernels[k]["avg_ns"] for k in ks)}
    if in_step and trace_csv:
        out["in_step"] = {}
        for name, (before, kernel, after) in in_step.items():
            d = load_in_step(trace_csv, before, kernel, after)
            out["in_step"][name] = {"before": before, "kernel": kernel, "after": after, "launches": len(d),
                                    "avg_ns": statistics.mean(d) if d else None}
    if source:
        out["kernel_source_sha256"] = hashlib.sha256(open(source, "rb").read()).hexdigest()
    return out


def to_markdown(summary, title, commands):
    lines = [f"# {title}", "", "Commands:", ""]
    lines += [f"    {c}" for c in commands]
    cal = summary["calibration"]
    if cal["fetch_scale"] and cal.get("reused"):
        note = (f"Counter calibration reused from the step profile's `{cal['copy_kernel']}` run: "
                f"fetch x{cal['fetch_scale']}, write x{cal['write_scale']}")
    elif cal["fetch_scale"]:
        note = (f"Counter calibration on `{cal['copy_kernel']}` ({cal['copy_doubles']} doubles copied): "
                f"fetch x{cal['fetch_scale']}, write x{cal['write_scale']}")
    else:
        note = ""
    lines += ["", note, ""]
    lines += ["| kernel | calls | avg us | FETCH KiB | WRITE KiB | HBM MB/launch |",
              "|---|---|---|---|---|---|"]
    for k, d in summary["kernels"].items():
        lines.append("| `{}` | {} | {} | {} | {} | {} |".format(
            k, d.get("calls", ""), f"{d['avg_ns'] / 1e3:.2f}" if "avg_ns" in d else "",
            f"{d['fetch_kib_median']:.0f}" if "fetch_kib_median" in d else "",
            f"{d['write_kib_median']:.0f}" if "write_kib_median" in d else "",
            f"{d['hbm_bytes_per_launch'] / 1e6:.2f}" if "hbm_bytes_per_launch" in d else ""))
    if any("resources" in d or "compiler" in d for d in summary["kernels"].values()):
        lines += ["", "| kernel | VGPR | AGPR | SGPR | spills (V/S) | occupancy (waves/SIMD) | LDS B | scratch B "
                  "| workgroup | max workgroups |", "|---|---|---|---|---|---|---|---|---|---|"]
        for k, d in summary["kernels"].items():
            c, r = d.get("compiler", {}), d.get("resources", {})
            if not c and not r:
                continue
            lines.append(f"| `{k}` | {c.get('vgpr', '')} | {c.get('agpr', '')} | {c.get('sgpr', '')} | "
                         f"{c.get('vgpr_spill', '')}/{c.get('sgpr_spill', '')} | {c.get('occupancy', '')} | "
                         f"{r.get('lds_bytes', c.get('lds_static', ''))} | {r.get('scratch_bytes', '')} | "
                         f"{r.get('workgroup', '')} | {r.get('max_workgroups', '')} |")
    if summary.get("ops"):
        lines += ["", "| operation | kernels | avg us (sum) |", "|---|---|---|"]
        for name, d in summary["ops"].items():
            lines.append(f"| {name} | {' + '.join('`%s`' % k for k in d['kernels'])} | {d['avg_ns'] / 1e3:.2f} |")
    if summary.get("in_step"):
        lines += ["", "Launches inside the timed steps (the trace's launches of the kernel between the two "
                  "neighbours the step runs it between):", "",
                  "| operation | kernel | between | launches | avg us |", "|---|---|---|---|---|"]
        for name, d in summary["in_step"].items():
            avg = f"{d['avg_ns'] / 1e3:.2f}" if d["avg_ns"] is not None else ""
            lines.append(f"| {name} | `{d['kernel']}` | `{d['before']}` and `{d['after']}` | {d['launches']} | {avg} |")
    if "kernel_source_sha256" in summary:
        lines += ["", f"Kernel source sha256: `{summary['kernel_source_sha256']}`"]
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description="Summarize rocprofv3 CSV output of the BS kernels")
    ap.add_argument("--stats")
    ap.add_argument("--trace", help="*_kernel_trace.csv: LDS, scratch and grid per kernel")
    ap.add_argument("--remarks", help="hipcc -Rpass-analysis=kernel-resource-usage output: registers, occupancy")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-kernel", default="k_copy<1, 768>")
    ap.add_argument("--copy-doubles", type=int, default=11390625)
    ap.add_argument("--source")
    ap.add_argument("--title", default="BS kernels")
    ap.add_argument("--command", action="append", default=[])
    ap.add_argument("--op", action="append", default=[], help="NAME=kernel1+kernel2 (summed averages)")
    ap.add_argument("--calibration", help="summary JSON whose counter calibration to reuse")
    ap.add_argument("--in-step", action="append", default=[],
                    help="NAME=before|kernel|after: average of kernel's launches between those neighbours")
    ap.add_argument("--pmc", action="append", default=[],
                    help="*_counter_collection.csv of any counters: with --md, write their per-kernel averages")
    ap.add_argument("--kernel", action="append", default=[], help="with --pmc: the kernels to keep (short names)")
    ap.add_argument("--json")
    ap.add_argument("--md")
    a = ap.parse_args(argv)
    if a.pmc:
        table = load_counters(a.pmc, set(a.kernel) or None)
        if a.json:
            with open(a.json, "w") as f:
                json.dump({k: {c: statistics.fmean(v) for c, v in d.items()} for k, d in table.items()}, f, indent=1)
        if a.md:
            with open(a.md, "w") as f:
                f.write(counters_markdown(table, a.title, a.command))
        return
    ops = {o.split("=", 1)[0]: o.split("=", 1)[1].split("+") for o in a.op}
    cal = None
    if a.calibration:
        c = json.load(open(a.calibration))["calibration"]
        cal = (c["fetch_scale"], c["write_scale"])
    in_step = {}
    for o in a.in_step:
        name, spec = o.split("=", 1)
        parts = spec.split("|")
        if len(parts) != 3:
            ap.error(f"--in-step {o!r}: expected NAME=before|kernel|after")
        in_step[name] = tuple(p.strip() for p in parts)
    s = summarize(a.stats, a.fetch, a.write, a.copy_kernel, a.copy_doubles, a.source, ops, a.trace, a.remarks,
                  cal, in_step)
    if a.json:
        with open(a.json, "w") as f:
            json.dump(s, f, indent=1)
    if a.md:
        with open(a.md, "w") as f:
            f.write(to_markdown(s, a.title, a.command))
    if not a.json and not a.md:
        print(json.dumps(s, indent=1))


if __name__ == "__main__":
    main()
