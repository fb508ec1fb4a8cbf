"""The host-side table builders of libbs (bs_host.cpp) and the CPU oracle
(oracle.c) under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/sanitize_tables.cpp links both, instrumented with g++/gcc
-fsanitize=address,undefined (no GPU code is involved), and runs every
builder on boxes and on the unstructured meshes written here (tet-split and
periodic lattices in random orientations, relabelled and shuffled), compares
the library's tables with the oracle's, runs the validators, and walks the
error paths. Any out-of-bounds access, leak, overflow or other undefined
behaviour ends the run with a sanitizer report and a nonzero status.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import bs_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def write_meshes(d):
    lines = []
    cases = []
    ev, nv, coords = bs_inputs.hex_tet_split(3, 2, 2)
    cases.append(("tetsplit", ev, nv, coords[ev], [1, 2, 4]))
    ev, nv = bs_inputs.hex_box(4, 3, 3, periodic=(True, False, True))
    cases.append(("torus", ev, nv, bs_inputs.hex_box_coords(4, 3, 3), [3]))
    for name, ev, nv, xe, orders in cases:
        ev2, sym = bs_inputs.hex_orient(ev, 901)
        xe2 = bs_inputs.reorder_corners(np.asarray(xe, dtype=np.float64), sym)
        ev3, nv3 = bs_inputs.hex_relabel(ev2, nv, 902, spare=3)
        order = bs_inputs.permutation(903, len(ev3))
        ev4 = np.ascontiguousarray(ev3[order], dtype=np.int32)
        xe4 = np.ascontiguousarray(xe2[order], dtype=np.float64)
        ev4.tofile(os.path.join(d, name + ".ev"))
        xe4.tofile(os.path.join(d, name + ".xe"))
        for p in orders:
            lines.append(f"{name} {len(ev4)} {nv3} {p}")
    with open(os.path.join(d, "meshes.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None, reason="needs gcc/g++")
def test_host_tables_under_address_and_ub_sanitizers(tmp_path):
    d = str(tmp_path)
    write_meshes(d)
    obj = os.path.join(d, "oracle.o")
    exe = os.path.join(d, "sanitize_tables")
    subprocess.run(["gcc", "-std=c11", "-D_DEFAULT_SOURCE", "-fopenmp", "-ffp-contract=off", *SAN, "-c",
                    os.path.join(ROOT, "oracle", "oracle.c"), "-o", obj], check=True)
    subprocess.run(["g++", "-std=c++17", "-fopenmp", *SAN, "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "sanitize_tables.cpp"),
                    os.path.join(ROOT, "cg_streaming_vector_amd", "csrc", "bs_host.cpp"), obj, "-o", exe, "-lm"],
                   check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")
    r = subprocess.run([exe, d], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "OK" in r.stdout, r.stdout
