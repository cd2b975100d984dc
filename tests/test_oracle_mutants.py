"""Plant plausible mistakes in copies of the oracle source; the pins must catch each one.

Every mutant is a one-token edit of keops_oracle.c (a dropped term, a flipped
sign, a wrong index, a broken tie-break).  The copy is compiled to a temporary
library and the full pin set runs against it; the test passes only if at
least one pin fails.  The committed oracle is never modified.
"""
import os

import pytest

import oracle
import oracle_pins

MUTANTS = {
    "sqdist_no_square": ("s += t * t;", "s += t;"),
    "sqdist_abs": ("s += t * t;", "s += t * (t < 0 ? -t : t);"),
    "kernel_sign": ("const double k = exp(-sq_dist(x + i * D, y + j * D, D) * inv_s2);\n"
                    "            for (int e = 0; e < E; ++e) {",
                    "const double k = exp(sq_dist(x + i * D, y + j * D, D) * inv_s2 - 1.0);\n"
                    "            for (int e = 0; e < E; ++e) {"),
    "sigma_not_squared": ("const double inv_s2 = 1.0 / (sigma * sigma);\n#pragma omp parallel for schedule(dynamic, 1)\n"
                          "    for (int64_t r = 0; r < nrows; ++r) {\n        const int64_t i = rows ? rows[r] : r;\n"
                          "        /* the row's accumulators",
                          "const double inv_s2 = 1.0 / (2.0 * sigma * sigma);\n#pragma omp parallel for schedule(dynamic, 1)\n"
                          "    for (int64_t r = 0; r < nrows; ++r) {\n        const int64_t i = rows ? rows[r] : r;\n"
                          "        /* the row's accumulators"),
    "sum_b_column": ("const double t = k * (double)b[j * E + e];", "const double t = k * (double)b[j * E];"),
    "sum_row_index": ("const int64_t i = rows ? rows[r] : r;\n        /* the row's accumulators",
                      "const int64_t i = r;\n        /* the row's accumulators"),
    "lse_drop_max": ("out[r * E + e] = m + log(s);", "out[r * E + e] = log(s);"),
    "lse_b_sign": ("* inv_s2 + (double)b[j * E + e];\n                    s += exp(v - m);",
                   "* inv_s2 - (double)b[j * E + e];\n                    s += exp(v - m);"),
    "grad_factor": ("const double t = -2.0 * inv_s2 * k * gb", "const double t = -1.0 * inv_s2 * k * gb"),
    "grad_sign": ("((double)x[i * D + d] - (double)y[j * D + d]);\n                o[d] += t;",
                  "((double)y[j * D + d] - (double)x[i * D + d]);\n                o[d] += t;"),
    "grad_g_index": ("gb += (double)g[i * E + e] * (double)b[j * E + e];",
                     "gb += (double)g[e] * (double)b[j * E + e];"),
    "grad_transposed_gb": ("gb += (double)g[i * E + e] * (double)b[j * E + e];",
                           "gb += (double)g[i * E + (E - 1 - e)] * (double)b[j * E + e];"),
    "grad_y_sign": ("const double t = 2.0 * inv_s2 * k * gb", "const double t = -2.0 * inv_s2 * k * gb"),
    "grad_y_factor": ("const double t = 2.0 * inv_s2 * k * gb", "const double t = 1.0 * inv_s2 * k * gb"),
    "grad_y_b_column": ("gb += (double)g[i * E + e] * (double)b[j * E + e];\n            for (int d = 0; d < D; ++d) {\n"
                        "                const double t = 2.0",
                        "gb += (double)g[i * E + e] * (double)b[j * E];\n            for (int d = 0; d < D; ++d) {\n"
                        "                const double t = 2.0"),
    "grad_y_ignores_cols": ("const int64_t j = cols ? cols[c] : c;\n        double o[D],",
                            "const int64_t j = c;\n        double o[D],"),
    "grad_b_g_column": ("const double t = k * (double)g[i * E + e];", "const double t = k * (double)g[i * E];"),
    "grad_b_kernel_sign": ("const double k = exp(-sq_dist(x + i * D, y + j * D, D) * inv_s2);\n            for (int e = 0; e < E; ++e) {\n"
                           "                const double t = k * (double)g",
                           "const double k = exp(sq_dist(x + i * D, y + j * D, D) * inv_s2 - 1.0);\n            for (int e = 0; e < E; ++e) {\n"
                           "                const double t = k * (double)g"),
    "matrix_sigma_not_squared": ("const double inv_s2 = 1.0 / (sigma * sigma);\n#pragma omp parallel for schedule(dynamic, 1)\n"
                                 "    for (int64_t i = 0; i < M; ++i)",
                                 "const double inv_s2 = 1.0 / (2.0 * sigma * sigma);\n#pragma omp parallel for schedule(dynamic, 1)\n"
                                 "    for (int64_t i = 0; i < M; ++i)"),
    "matrix_row_stride": ("out[i * N + j] = exp(", "out[j * M + i] = exp("),
    "ranges_slice_start": ("const int64_t k0 = c == 0 ? 0 : slices_i[c - 1], k1 = slices_i[c];\n#pragma omp parallel for schedule(dynamic, 1)\n"
                           "        for (int64_t i = ranges_i[2 * c]; i < ranges_i[2 * c + 1]; ++i) {\n            double o[E]",
                           "const int64_t k0 = c == 0 ? 0 : slices_i[c - 1] + 1, k1 = slices_i[c];\n#pragma omp parallel for schedule(dynamic, 1)\n"
                           "        for (int64_t i = ranges_i[2 * c]; i < ranges_i[2 * c + 1]; ++i) {\n            double o[E]"),
    "ranges_j_end": ("for (int64_t j = redranges_j[2 * k]; j < redranges_j[2 * k + 1]; ++j) {\n                    const double kv",
                     "for (int64_t j = redranges_j[2 * k]; j + 1 < redranges_j[2 * k + 1]; ++j) {\n                    const double kv"),
    "ranges_lse_drop_max": ("out[i * E + e] = m + log(s);", "out[i * E + e] = log(s);"),
    "max_ties_last": ("if (v > out[r * E + e]) { out[r * E + e] = v;", "if (v >= out[r * E + e]) { out[r * E + e] = v;"),
    "max_no_sign": ("const double v = (double)sgn * k * (double)b[j * E + e];", "const double v = k * (double)b[j * E + e];"),
    "laplace_no_sqrt": ("const double k = exp(-sqrt(sq_dist(x + i * D, y + j * D, D)) / sigma);",
                        "const double k = exp(-sq_dist(x + i * D, y + j * D, D) / sigma);"),
    "laplace_sigma_squared": ("const double k = exp(-sqrt(sq_dist(x + i * D, y + j * D, D)) / sigma);",
                              "const double k = exp(-sqrt(sq_dist(x + i * D, y + j * D, D)) / (sigma * sigma));"),
    "kmin_tie_break": ("(dj == bd[pos - 1] && j < bj[pos - 1])", "(dj == bd[pos - 1] && j > bj[pos - 1])"),
    "kmin_keep_last": ("if (count == K && !(dj < bd[K - 1]", "if (count == K && !(dj <= bd[K - 1]"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new, 1)
    path = os.path.join(str(tmp_path), "mutant.c")
    with open(path, "w") as f:
        f.write(mutated)
    lib = oracle.open_library(oracle.compile_source(path, os.path.join(str(tmp_path), "libm.so")))
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib=lib)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} survived every pin"


# Planted mistakes in a copy of the Python checker of the conjugate-gradient solver
# (oracle.gauss_system_residual); pin_system_residual must catch each one.
RESIDUAL_MUTANTS = {
    "residual_lam_sign": ("- float(lam) * a[sel]", "+ float(lam) * a[sel]"),
    "residual_lam_dropped": ("- float(lam) * a[sel]", "- 0.0 * a[sel]"),
    "residual_rows_ignored_in_product": ("gauss_sum(x[rows] if rows is not None else x, x, a",
                                         "gauss_sum(x, x, a"),
    "residual_rows_ignored_in_b": ("return b[sel] - Ka", "return b[:Ka.shape[0]] - Ka"),
    "residual_product_sign": ("return b[sel] - Ka", "return b[sel] + Ka"),
}


@pytest.mark.parametrize("name", sorted(RESIDUAL_MUTANTS))
def test_residual_mutant_is_caught(name):
    import inspect
    import textwrap
    old, new = RESIDUAL_MUTANTS[name]
    src = textwrap.dedent(inspect.getsource(oracle.gauss_system_residual))
    assert src.count(old) == 1, f"mutation site for {name} not found"
    ns = dict(vars(oracle))
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), ns)
    try:
        oracle_pins.pin_system_residual(residual=ns["gauss_system_residual"])
    except (AssertionError, ValueError, IndexError):
        return
    pytest.fail(f"mutant {name} survived pin_system_residual")
