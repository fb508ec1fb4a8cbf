"""Plants plausible mistakes in a copy of the oracle and checks that the pin
suite catches every one (CPU only).

Each mutant is oracle.c with one textual change (a flipped sign, a transposed
operand, a dropped term, an off-by-one, a contraction the pages' rounding
forbids, a reversed order), built with the same flags, and the pins of
tests/test_oracle_pins.py run against it in a subprocess. A mutant that
passes every pin would be a mistake the pins cannot see.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text in oracle.c, replacement, pin tests to run)
MUTANTS = [
    ("axpy_sign", "y[i] = t1 + t2;", "y[i] = t1 - t2;", "axpy"),
    ("axpy_operand", "double t2 = beta * y[i];", "double t2 = beta * x[i];", "axpy"),
    ("axpy_fma", "y[i] = t1 + t2;", "y[i] = fma(alpha, x[i], t2);", "axpy"),
    ("dot_drop_error_term", "s = s + (q + r);", "s = s + q;", "dot or norm"),
    ("dot_chunk_off_by_one", "int64_t len = (n - a < OR_CHUNK) ? (n - a) : OR_CHUNK;",
     "int64_t len = (n - a < OR_CHUNK) ? (n - a) : OR_CHUNK - 1;", "dot"),
    ("dot_drop_lo_parts", "for (int64_t k = 1; k < 2 * nc; ++k) {", "for (int64_t k = 2; k < 2 * nc; k += 2) {",
     "dot or norm"),
    ("norm_no_root", "return sqrt(or_dot(n, x, x));", "return or_dot(n, x, x);", "norm"),
    ("cg_r_sign", "r[i] = r[i] - aq;", "r[i] = r[i] + aq;", "cg"),
    ("cg_returns_x", "return or_dot(n, r, r);", "return or_dot(n, x, x);", "cg"),
    ("cg_swaps_pq", "double ap = alpha * p[i];", "double ap = alpha * q[i];", "cg"),
    ("scatter_mask_value", "v_local[i] = (l2g[i] >= 0) ? v_global[l2g[i]] : 0.0;",
     "v_local[i] = (l2g[i] >= 0) ? v_global[l2g[i]] : -0.0;", "scatter"),
    ("scatter_off_by_one", "v_local[i] = (l2g[i] >= 0) ? v_global[l2g[i]] : 0.0;",
     "v_local[i] = (l2g[i] > 0) ? v_global[l2g[i]] : 0.0;", "scatter"),
    ("gather_descending", "for (int64_t i = 0; i < n_local; ++i)\n        if (l2g[i] >= 0) v_global",
     "for (int64_t i = n_local - 1; i >= 0; --i)\n        if (l2g[i] >= 0) v_global", "gather"),
    ("gather_start_negative_zero", "for (int64_t g = 0; g < n_global; ++g) v_global[g] = 0.0;",
     "for (int64_t g = 0; g < n_global; ++g) v_global[g] = -0.0;", "gather"),
    ("gll_wrong_derivative", "double d1 = p * (t * P - Pm) / (t * t - 1.0);",
     "double d1 = p * (t * P + Pm) / (t * t - 1.0);", "gll"),
    ("mesh_y_fastest", "key[L] = (iz * ny + iy) * nx + ix;", "key[L] = (iz * nx + ix) * ny + iy;", "box"),
    ("mesh_ignores_elem_perm", "int64_t e = elem_perm ? elem_perm[s] : s;", "int64_t e = s;", "box or shuffled"),
    ("mesh_end_node_not_shared", "return (double)c + (1.0 + ri) / 2.0;", "return (double)c * 1.000001 + (1.0 + ri) / 2.0;",
     "box or scatter or gather"),
    ("g2l_descending", "if (a->g != b->g) return a->g < b->g ? -1 : 1;\n    return (a->i < b->i) ? -1 : (a->i > b->i);",
     "if (a->g != b->g) return a->g < b->g ? -1 : 1;\n    return (a->i > b->i) ? -1 : (a->i < b->i);", "g2l"),
    ("hex_factors_in_axis_order", "if (m[y] < m[x])", "if (0 && m[y] < m[x])", "hex"),
    ("hex_keeps_zero_weights", "if (zero) continue;", "(void)zero;", "hex"),
    ("hex_factor_from_own_end", "m[a] = ((c >> a) & 1) ? idx[a] : p - idx[a];",
     "m[a] = ((c >> a) & 1) ? p - idx[a] : idx[a];", "hex"),
    ("hex_vertices_in_corner_order", "y > 0 && s[2 * y] < s[2 * (y - 1)]", "y > 0 && 0", "hex"),
    ("hex_numbered_by_signature", "if (first[cls[L]] < 0) first[cls[L]] = NG++;",
     "if (first[cls[L]] < 0) first[cls[L]] = NG++;\n        first[cls[L]] = cls[L];", "hex"),
    ("hexmass_factors_mirrored", "else d *= bit ? (1.0 + t[b]) / 2.0 : (1.0 - t[b]) / 2.0;",
     "else d *= bit ? (1.0 - t[b]) / 2.0 : (1.0 + t[b]) / 2.0;", "hexmass"),
    ("hexmass_signed_det", "w[i] * w[j] * w[k] * fabs(det);", "w[i] * w[j] * w[k] * det;", "hexmass"),
    ("hexmass_derivative_scale", "if (b == a) d *= bit ? 0.5 : -0.5;", "if (b == a) d *= bit ? 1.0 : -1.0;",
     "hexmass"),
    ("hexmass_cofactor_sign", "- J[0][1] * (J[1][0] * J[2][2] - J[1][2] * J[2][0])",
     "+ J[0][1] * (J[1][0] * J[2][2] - J[1][2] * J[2][0])", "hexmass"),
]


@pytest.mark.parametrize("name,old,new,sel", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new, sel):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mutant = tmp_path / "oracle_mutant.c"
    mutant.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-D_DEFAULT_SOURCE", "-fopenmp", "-ffp-contract=off",
                           "-fno-fast-math", "-fPIC", "-shared", "-o", str(lib), str(mutant), "-lm"])
    env = dict(os.environ, BS_ORACLE_LIB=str(lib), OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-k", sel],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
