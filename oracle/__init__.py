"""The oracle: plain double-precision CPU reference of the four Gaussian map-reductions.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
(``geometric_map_reduce_amd``) never imports it and shares no code with it.

The arithmetic lives in ``keops_oracle.c`` (plain C, double precision, OpenMP
over independent rows); this module only builds it with gcc and marshals numpy
arrays.  Each function cites the passage of the KeOps pages it follows:

* ``gauss_sum``   -- "Kernel Operations on the GPU, with Autodiff, without
  Memory Overflows", §1 "Target operation" (a_i = sum_j k(x_i, y_j) b_j with a
  Gaussian k of deviation sigma); KeOps README PyTorch example (K_ij.sum).
* ``gauss_lse``   -- same paper, §2 reductions list (log-sum-exp); README
  ``.logsumexp()``.
* ``gauss_grad_x``-- same paper, §2 "Performance and differentiation"
  (autodiff); README ``torch.autograd.grad((a_i ** 2).sum(), [x])``.
* ``kmin``        -- same paper, §2 (argmin, argKmin); README feature list
  (ArgMin, K-min reductions).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "keops_oracle.c")
_LIB = os.path.join(_HERE, "_build", "liboracle.so")
_lock = threading.Lock()
_lib = None


def compile_source(src: str, out: str) -> str:
    """gcc -O2 -fopenmp, no fast-math and no FMA contraction; returns ``out``."""
    os.makedirs(os.path.dirname(out) or ".", exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fno-fast-math", "-ffp-contract=off", "-std=c11",
           "-fPIC", "-shared", "-Wall", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile keops_oracle.c into oracle/_build/liboracle.so."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(SOURCE):
        return _LIB
    return compile_source(SOURCE, _LIB)


def open_library(path: str):
    """ctypes handle on an oracle library built from keops_oracle.c (or a copy of it)."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i64, i32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.oracle_gauss_sum.argtypes = [P, P, P, i64, i64, i32, i32, f64, P, i64, P, P]
    lib.oracle_gauss_lse.argtypes = [P, P, P, i64, i64, i32, i32, f64, P, i64, P]
    lib.oracle_gauss_grad_x.argtypes = [P, P, P, P, i64, i64, i32, i32, f64, P, i64, P, P]
    lib.oracle_gauss_grad_y.argtypes = [P, P, P, P, i64, i64, i32, i32, f64, P, i64, P, P]
    lib.oracle_gauss_grad_b.argtypes = [P, P, P, i64, i64, i32, i32, f64, P, i64, P, P]
    lib.oracle_kmin.argtypes = [P, P, i64, i64, i32, i32, P, i64, P, P]
    lib.oracle_sq_dist_pairs.argtypes = [P, P, i32, P, P, i64, P]
    lib.oracle_gauss_matrix.argtypes = [P, P, i64, i64, i32, f64, P]
    lib.oracle_laplace_sum.argtypes = [P, P, P, i64, i64, i32, i32, f64, P, i64, P, P]
    lib.oracle_gauss_max.argtypes = [P, P, P, i64, i64, i32, i32, f64, i32, P, i64, P, P]
    lib.oracle_gauss_sum_ranges.argtypes = [P, P, P, i64, i64, i32, i32, f64, P, i64, P, P, i64, P, P]
    lib.oracle_gauss_lse_ranges.argtypes = [P, P, P, i64, i64, i32, i32, f64, P, i64, P, P, i64, P]
    for f in ("oracle_gauss_sum", "oracle_gauss_lse", "oracle_gauss_grad_x", "oracle_gauss_grad_y",
              "oracle_gauss_grad_b", "oracle_kmin", "oracle_sq_dist_pairs", "oracle_num_threads"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


def _load():
    """The library built from the committed source (``lib=`` arguments below accept another
    handle from ``open_library``, e.g. one built from a deliberately broken copy in a test)."""
    global _lib
    with _lock:
        if _lib is None:
            _lib = open_library(build(force=False))
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle uses (OMP_NUM_THREADS, else all host cores)."""
    return int(_load().oracle_num_threads())


def _f32(a, ndim):
    a = np.ascontiguousarray(a, dtype=np.float32)
    if a.ndim == 1 and ndim == 2:
        a = a.reshape(-1, 1)
    assert a.ndim == ndim
    return a


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _rows(rows, M):
    if rows is None:
        return None, M
    r = np.ascontiguousarray(rows, dtype=np.int64)
    return r, r.shape[0]


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"oracle {name}: invalid argument")


def gauss_sum(x, y, b, sigma, rows=None, lib=None):
    """a[r, e] = sum_j exp(-|x_i - y_j|^2 / sigma^2) b[j, e]  for i = rows[r].

    Returns (a, norm) in float64, norm[r, e] = sum_j |K_ij b_je|.
    """
    x, y, b = _f32(x, 2), _f32(y, 2), _f32(b, 2)
    M, D = x.shape
    N, E = b.shape
    assert y.shape == (N, D)
    r, n = _rows(rows, M)
    out = np.empty((n, E), np.float64)
    nrm = np.empty((n, E), np.float64)
    _check((lib or _load()).oracle_gauss_sum(_ptr(x), _ptr(y), _ptr(b), M, N, D, E, float(sigma),
                                    _ptr(r), n, _ptr(out), _ptr(nrm)), "gauss_sum")
    return out, nrm


def gauss_lse(x, y, b, sigma, rows=None, lib=None):
    """l[r, e] = log sum_j exp(-|x_i - y_j|^2 / sigma^2 + b[j, e]) in float64 (two-pass)."""
    x, y, b = _f32(x, 2), _f32(y, 2), _f32(b, 2)
    M, D = x.shape
    N, E = b.shape
    assert y.shape == (N, D)
    r, n = _rows(rows, M)
    out = np.empty((n, E), np.float64)
    _check((lib or _load()).oracle_gauss_lse(_ptr(x), _ptr(y), _ptr(b), M, N, D, E, float(sigma),
                                    _ptr(r), n, _ptr(out)), "gauss_lse")
    return out


def gauss_grad_x(x, y, b, g, sigma, rows=None, lib=None):
    """G[r, d] = sum_j (-2/sigma^2) K_ij <g_i, b_j> (x_id - y_jd)  for i = rows[r].

    ``g`` is the full [M, E] cotangent dL/da.  Returns (G, nu) in float64 with
    nu[r, d] = sum_j |(2/sigma^2) K_ij <g_i, b_j> (x_id - y_jd)|.
    """
    x, y, b, g = _f32(x, 2), _f32(y, 2), _f32(b, 2), _f32(g, 2)
    M, D = x.shape
    N, E = b.shape
    assert y.shape == (N, D) and g.shape == (M, E)
    r, n = _rows(rows, M)
    out = np.empty((n, D), np.float64)
    nu = np.empty((n, D), np.float64)
    _check((lib or _load()).oracle_gauss_grad_x(_ptr(x), _ptr(y), _ptr(b), _ptr(g), M, N, D, E,
                                       float(sigma), _ptr(r), n, _ptr(out), _ptr(nu)),
           "gauss_grad_x")
    return out, nu


def gauss_grad_y(x, y, b, g, sigma, cols=None, lib=None):
    """Gy[c, d] = sum_i (2/sigma^2) K_ij <g_i, b_j> (x_id - y_jd)  for j = cols[c]:
    dL/dy of L = sum g * a.  Returns (Gy, nu) in float64, nu the sum of the terms' moduli."""
    x, y, b, g = _f32(x, 2), _f32(y, 2), _f32(b, 2), _f32(g, 2)
    M, D = x.shape
    N, E = b.shape
    assert y.shape == (N, D) and g.shape == (M, E)
    c, n = _rows(cols, N)
    out = np.empty((n, D), np.float64)
    nu = np.empty((n, D), np.float64)
    _check((lib or _load()).oracle_gauss_grad_y(_ptr(x), _ptr(y), _ptr(b), _ptr(g), M, N, D, E,
                                       float(sigma), _ptr(c), n, _ptr(out), _ptr(nu)),
           "gauss_grad_y")
    return out, nu


def gauss_grad_b(x, y, g, sigma, cols=None, lib=None):
    """Gb[c, e] = sum_i K_ij g_ie  for j = cols[c]: dL/db of L = sum g * a.
    Returns (Gb, nu) in float64, nu[c, e] = sum_i |K_ij g_ie|."""
    x, y, g = _f32(x, 2), _f32(y, 2), _f32(g, 2)
    M, D = x.shape
    N = y.shape[0]
    E = g.shape[1]
    assert y.shape == (N, D) and g.shape == (M, E)
    c, n = _rows(cols, N)
    out = np.empty((n, E), np.float64)
    nu = np.empty((n, E), np.float64)
    _check((lib or _load()).oracle_gauss_grad_b(_ptr(x), _ptr(y), _ptr(g), M, N, D, E,
                                       float(sigma), _ptr(c), n, _ptr(out), _ptr(nu)),
           "gauss_grad_b")
    return out, nu


def kmin(x, y, K, rows=None, lib=None):
    """K smallest |x_i - y_j|^2 (float64) and their int64 indices, ascending by (d^2, j)."""
    x, y = _f32(x, 2), _f32(y, 2)
    M, D = x.shape
    N = y.shape[0]
    assert y.shape == (N, D)
    r, n = _rows(rows, M)
    out_d = np.empty((n, K), np.float64)
    out_i = np.empty((n, K), np.int64)
    _check((lib or _load()).oracle_kmin(_ptr(x), _ptr(y), M, N, D, int(K), _ptr(r), n,
                               _ptr(out_d), _ptr(out_i)), "kmin")
    return out_d, out_i


def sq_dist_pairs(x, y, ii, jj, lib=None):
    """|x_ii[p] - y_jj[p]|^2 in float64 for each pair p."""
    x, y = _f32(x, 2), _f32(y, 2)
    ii = np.ascontiguousarray(ii, dtype=np.int64).ravel()
    jj = np.ascontiguousarray(jj, dtype=np.int64).ravel()
    assert ii.shape == jj.shape
    assert ii.size == 0 or (ii.min() >= 0 and ii.max() < x.shape[0])
    assert jj.size == 0 or (jj.min() >= 0 and jj.max() < y.shape[0])
    out = np.empty(ii.shape[0], np.float64)
    _check((lib or _load()).oracle_sq_dist_pairs(_ptr(x), _ptr(y), x.shape[1], _ptr(ii), _ptr(jj),
                                        ii.shape[0], _ptr(out)), "sq_dist_pairs")
    return out


def gauss_matrix(x, y, sigma, lib=None):
    """K[i, j] = exp(-|x_i - y_j|^2 / sigma^2) materialised in float64 (small inputs only)."""
    x, y = _f32(x, 2), _f32(y, 2)
    M, D = x.shape
    N = y.shape[0]
    assert y.shape == (N, D)
    out = np.empty((M, N), np.float64)
    _check((lib or _load()).oracle_gauss_matrix(_ptr(x), _ptr(y), M, N, D, float(sigma), _ptr(out)),
           "gauss_matrix")
    return out


def gauss_solve(x, b, sigma, lam, lib=None):
    """The exact solution a* of (K + lam I) a = b, K = exp(-|x_i - x_j|^2/sigma^2), by a dense
    float64 solve (what the conjugate gradient solver approximates; [README] feature list:
    conjugate gradient solver for spline interpolation or kriging).  Small N only."""
    b = np.asarray(b, np.float64)
    if b.ndim == 1:
        b = b.reshape(-1, 1)
    K = gauss_matrix(x, x, sigma, lib=lib)
    A = K + float(lam) * np.eye(K.shape[0])
    return np.linalg.solve(A, b)


def gauss_system_residual(x, b, a, sigma, lam, rows=None, lib=None):
    """r = b - (K + lam I) a in float64 for the selected rows (all by default), with the
    products K a taken by the sum oracle over all points: for checking an approximate
    solution a (float32, e.g. from the GPU solver) at any size."""
    x, b, a = _f32(x, 2), np.asarray(b, np.float64), _f32(a, 2)
    if b.ndim == 1:
        b = b.reshape(-1, 1)
    Ka, _ = gauss_sum(x[rows] if rows is not None else x, x, a, sigma, lib=lib)
    sel = rows if rows is not None else slice(None)
    return b[sel] - Ka - float(lam) * a[sel].astype(np.float64)


def _ranges(ranges_i, slices_i, redranges_j):
    ri = np.ascontiguousarray(ranges_i, dtype=np.int64).reshape(-1, 2)
    si = np.ascontiguousarray(slices_i, dtype=np.int64).ravel()
    rj = np.ascontiguousarray(redranges_j, dtype=np.int64).reshape(-1, 2)
    assert si.shape[0] == ri.shape[0]
    return ri, si, rj


def gauss_sum_ranges(x, y, b, sigma, ranges_i, slices_i, redranges_j, lib=None):
    """Block-sparse Gaussian sum over the kept pairs given by (ranges_i, slices_i, redranges_j)
    (row range c meets the j ranges slices_i[c-1] .. slices_i[c]-1).  Returns (a, norm) for all
    M rows, float64; rows in no row range get 0."""
    x, y, b = _f32(x, 2), _f32(y, 2), _f32(b, 2)
    M, D = x.shape
    N, E = b.shape
    assert y.shape == (N, D)
    ri, si, rj = _ranges(ranges_i, slices_i, redranges_j)
    out = np.empty((M, E), np.float64)
    norm = np.empty((M, E), np.float64)
    _check((lib or _load()).oracle_gauss_sum_ranges(_ptr(x), _ptr(y), _ptr(b), M, N, D, E, float(sigma),
                                           _ptr(ri), ri.shape[0], _ptr(si), _ptr(rj), rj.shape[0],
                                           _ptr(out), _ptr(norm)), "gauss_sum_ranges")
    return out, norm


def gauss_lse_ranges(x, y, b, sigma, ranges_i, slices_i, redranges_j, lib=None):
    """Block-sparse LogSumExp over the kept pairs (rows with none get -inf), float64 [M, E]."""
    x, y, b = _f32(x, 2), _f32(y, 2), _f32(b, 2)
    M, D = x.shape
    N, E = b.shape
    assert y.shape == (N, D)
    ri, si, rj = _ranges(ranges_i, slices_i, redranges_j)
    out = np.empty((M, E), np.float64)
    _check((lib or _load()).oracle_gauss_lse_ranges(_ptr(x), _ptr(y), _ptr(b), M, N, D, E, float(sigma),
                                           _ptr(ri), ri.shape[0], _ptr(si), _ptr(rj), rj.shape[0],
                                           _ptr(out)), "gauss_lse_ranges")
    return out


def gauss_max(x, y, b, sigma, sign=1, rows=None, lib=None):
    """max_j sign * K_ij b_je and the smallest j reaching it, per row and column: sign = +1 is
    Max / ArgMax of K b, sign = -1 is -(Min) / ArgMin.  Returns (values float64, indices int64);
    N = 0 gives -inf and -1."""
    x, y, b = _f32(x, 2), _f32(y, 2), _f32(b, 2)
    M, D = x.shape
    N, E = b.shape
    assert y.shape == (N, D)
    r, n = _rows(rows, M)
    out = np.empty((n, E), np.float64)
    idx = np.empty((n, E), np.int64)
    _check((lib or _load()).oracle_gauss_max(_ptr(x), _ptr(y), _ptr(b), M, N, D, E, float(sigma), int(sign),
                                    _ptr(r), n, _ptr(out), _ptr(idx)), "gauss_max")
    return out, idx


def laplace_sum(x, y, b, sigma, rows=None, lib=None):
    """a[r, e] = sum_j exp(-|x_i - y_j| / sigma) b[j, e] for i = rows[r]; returns (a, norm) in float64."""
    x, y, b = _f32(x, 2), _f32(y, 2), _f32(b, 2)
    M, D = x.shape
    N, E = b.shape
    assert y.shape == (N, D)
    r, n = _rows(rows, M)
    out = np.empty((n, E), np.float64)
    norm = np.empty((n, E), np.float64)
    _check((lib or _load()).oracle_laplace_sum(_ptr(x), _ptr(y), _ptr(b), M, N, D, E, float(sigma), _ptr(r), n,
                                      _ptr(out), _ptr(norm)), "laplace_sum")
    return out, norm

