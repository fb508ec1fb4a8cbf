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

Usage:
  python -m cg_streaming_vector_amd.profiling --stats S.csv --fetch F.csv \\
      --write W.csv --copy-kernel 'k_copy<1>' --copy-doubles 11390625 \\
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


def summarize(stats_csv, fetch_csv, write_csv, copy_kernel, copy_doubles, source=None, ops=None):
    stats = load_stats(stats_csv) if stats_csv else {}
    fetch = load_counter(fetch_csv, "FETCH_SIZE") if fetch_csv else {}
    write = load_counter(write_csv, "WRITE_SIZE") if write_csv else {}
    known = 8.0 * copy_doubles
    f_scale = w_scale = None
    if copy_kernel in fetch and copy_kernel in write:
        f_scale = known / (statistics.median(fetch[copy_kernel]) * 1024.0)
        w_scale = known / (statistics.median(write[copy_kernel]) * 1024.0)
    kernels = {}
    for k in sorted(set(stats) | set(fetch) | set(write)):
        if k.startswith("__amd") or "at::native" in k:
            continue
        d = {}
        if k in stats:
            d["calls"], d["avg_ns"] = stats[k]
        if k in fetch:
            d["fetch_kib_median"] = statistics.median(fetch[k])
        if k in write:
            d["write_kib_median"] = statistics.median(write[k])
        if f_scale and k in fetch and k in write:
            d["hbm_bytes_per_launch"] = (d["fetch_kib_median"] * 1024.0 * f_scale
                                         + d["write_kib_median"] * 1024.0 * w_scale)
        kernels[k] = d
    out = {"calibration": {"copy_kernel": copy_kernel, "copy_doubles": copy_doubles,
                           "fetch_scale": f_scale, "write_scale": w_scale},
           "kernels": kernels}
    if ops:
        # an operation may be several kernels launched back to back (a
        # reduction's first stage and its finish): sum their averages
        out["ops"] = {}
        for name, ks in ops.items():
            if all(k in kernels and "avg_ns" in kernels[k] for k in ks):
                out["ops"][name] = {"kernels": ks, "avg_ns": sum(kernels[k]["avg_ns"] for k in ks)}
    if source:
        out["kernel_source_sha256"] = hashlib.sha256(open(source, "rb").read()).hexdigest()
    return out


def to_markdown(summary, title, commands):
    lines = [f"# {title}", "", "Commands:", ""]
    lines += [f"    {c}" for c in commands]
    cal = summary["calibration"]
    lines += ["", f"Counter calibration on `{cal['copy_kernel']}` ({cal['copy_doubles']} doubles copied): "
              f"fetch x{cal['fetch_scale']}, write x{cal['write_scale']}" if cal["fetch_scale"] else "", ""]
    lines += ["| kernel | calls | avg us | FETCH KiB | WRITE KiB | HBM MB/launch |",
              "|---|---|---|---|---|---|"]
    for k, d in summary["kernels"].items():
        lines.append("| `{}` | {} | {} | {} | {} | {} |".format(
            k, d.get("calls", ""), f"{d['avg_ns'] / 1e3:.2f}" if "avg_ns" in d else "",
            f"{d['fetch_kib_median']:.0f}" if "fetch_kib_median" in d else "",
            f"{d['write_kib_median']:.0f}" if "write_kib_median" in d else "",
            f"{d['hbm_bytes_per_launch'] / 1e6:.2f}" if "hbm_bytes_per_launch" in d else ""))
    if summary.get("ops"):
        lines += ["", "| operation | kernels | avg us (sum) |", "|---|---|---|"]
        for name, d in summary["ops"].items():
            lines.append(f"| {name} | {' + '.join('`%s`' % k for k in d['kernels'])} | {d['avg_ns'] / 1e3:.2f} |")
    if "kernel_source_sha256" in summary:
        lines += ["", f"Kernel source sha256: `{summary['kernel_source_sha256']}`"]
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description="Summarize rocprofv3 CSV output of the BS kernels")
    ap.add_argument("--stats")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-kernel", default="k_copy<1>")
    ap.add_argument("--copy-doubles", type=int, default=11390625)
    ap.add_argument("--source")
    ap.add_argument("--title", default="BS kernels")
    ap.add_argument("--command", action="append", default=[])
    ap.add_argument("--op", action="append", default=[], help="NAME=kernel1+kernel2 (summed averages)")
    ap.add_argument("--json")
    ap.add_argument("--md")
    a = ap.parse_args(argv)
    ops = {o.split("=", 1)[0]: o.split("=", 1)[1].split("+") for o in a.op}
    s = summarize(a.stats, a.fetch, a.write, a.copy_kernel, a.copy_doubles, a.source, ops)
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
