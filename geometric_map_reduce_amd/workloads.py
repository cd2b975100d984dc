"""Seeded synthetic inputs for the Gaussian map-reduce workloads.

This module only draws random numbers; it holds none of the method's
arithmetic, so both the GPU path and the oracle can use it.

Every array is drawn in float64 from ``numpy.random.default_rng(seed)`` (PCG64)
and rounded to float32, in the fixed order x, y, b.  Large arrays are drawn in
chunks of ``CHUNK_ROWS`` rows, which is part of the recipe.

Workloads (shapes from the KeOps pages: the paper's benchmark uses M = N points
in dimension D = 3 and scales N from 10k to 1M; the README example uses
3-column randn point clouds; the Falkon issue "Transparent interface for
billion-scale matrices" quotes N = 1G, M = 100k, D = 50, here scaled to one
GPU's share N = 10M):

=========================  ========  ========  ===  ======  =====  =========================
name                       M         N         D    E / K   sigma  distribution
=========================  ========  ========  ===  ======  =====  =========================
sum_1k                     1,000     1,000     3    E=1     1.0    x, y, b ~ N(0, 1)
sum_grad_10k               10,000    10,000    3    E=1     0.5    x, y, b ~ N(0, 1)
sum_lse_1M                 1e6       1e6       3    E=1     0.1    x, y ~ U[0,1)^3, b ~ N(0,1)
solver_matvec_100k_x_10M   1e5       1e7       50   E=1     1.0    x, y ~ N(0, I/50), b ~ N(0,1)
kmin10_1M_d3               1e6       1e6       3    K=10    --     16-component mixture
kmin10_1M_d64              1e6       1e6       64   K=10    --     16-component mixture
stream_16_x_100M           16        1e8       3    E=1     0.1    x, y ~ U[0,1)^3, b ~ N(0,1)
kmin10_16_x_100M           16        1e8       3    K=10    --     x, y ~ U[0,1)^3
krige_100k                 1e5       1e5       3    E=1     0.1    x ~ U[0,1)^3, b ~ N(0,1); lambda = 1
=========================  ========  ========  ===  ======  =====  =========================

stream_16_x_100M is the few-rows, many-j case (the Falkon issue's M << N taken
to its end): 16 rows against 1e8 points, where streaming y and b from HBM
once, not arithmetic, bounds the time; kmin10_16_x_100M is the K-min over
the same shape.  krige_100k is the conjugate-gradient
solve of (K + lambda I) a = b on the points x (the README's kriging / spline
use of the solver); its y draw is made, to keep the recipe's order, and unused.

Mixture recipe: centres ~ U[-5, 5)^D (16 of them, drawn first), then for x:
labels ~ U{0..15}, x = centres[label] + 0.5 * N(0, I); then the same for y.
N(0, I/50) means covariance I/50, i.e. standard deviation 1/sqrt(50).
"""
from __future__ import annotations

import dataclasses

import numpy as np

CHUNK_ROWS = 1 << 20


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    D: int
    E: int = 1
    K: int = 0
    sigma: float = 1.0
    dist: str = "normal"      # normal | uniform | normal_scaled | mixture16
    ops: tuple = ("sum",)
    lam: float = 0.0          # ridge of the linear solve (cg only)

    def describe(self) -> dict:
        d = {"workload": self.name, "M": self.M, "N": self.N, "D": self.D}
        if self.K:
            d["K"] = self.K
        else:
            d["E"] = self.E
            d["sigma"] = self.sigma
        if self.lam:
            d["lambda"] = self.lam
        d["inputs"] = self.dist
        return d


WORKLOADS = {
    w.name: w for w in [
        Workload("sum_1k", 1000, 1000, 3, E=1, sigma=1.0, dist="normal", ops=("sum",)),
        Workload("sum_grad_10k", 10_000, 10_000, 3, E=1, sigma=0.5, dist="normal",
                 ops=("sum", "grad_x")),
        Workload("sum_lse_1M", 1_000_000, 1_000_000, 3, E=1, sigma=0.1, dist="uniform",
                 ops=("sum", "lse")),
        Workload("solver_matvec_100k_x_10M", 100_000, 10_000_000, 50, E=1, sigma=1.0,
                 dist="normal_scaled", ops=("sum",)),
        Workload("kmin10_1M_d3", 1_000_000, 1_000_000, 3, K=10, dist="mixture16",
                 ops=("kmin",)),
        Workload("kmin10_1M_d64", 1_000_000, 1_000_000, 64, K=10, dist="mixture16",
                 ops=("kmin",)),
        Workload("stream_16_x_100M", 16, 100_000_000, 3, E=1, sigma=0.1, dist="uniform",
                 ops=("sum", "lse", "grad_x")),
        Workload("kmin10_16_x_100M", 16, 100_000_000, 3, K=10, dist="uniform", ops=("kmin",)),
        Workload("krige_100k", 100_000, 100_000, 3, E=1, sigma=0.1, dist="uniform", ops=("cg",), lam=1.0),
    ]
}


def _chunked(rng, fn, rows, cols):
    out = np.empty((rows, cols), np.float32)
    for s in range(0, rows, CHUNK_ROWS):
        e = min(rows, s + CHUNK_ROWS)
        out[s:e] = fn(rng, (e - s, cols))
    return out


def _normal(rng, shape):
    return rng.standard_normal(shape)


def _uniform(rng, shape):
    return rng.random(shape)


def make_points(dist: str, M: int, N: int, D: int, E: int, seed: int = 0):
    """Draw (x[M,D], y[N,D], b[N,E]) as float32 with the recipe named by ``dist``.

    For ``mixture16`` no b is drawn (K-min takes none) and b is None.
    """
    rng = np.random.default_rng(seed)
    if dist == "normal":
        x = _chunked(rng, _normal, M, D)
        y = _chunked(rng, _normal, N, D)
        b = _chunked(rng, _normal, N, E)
    elif dist == "uniform":
        x = _chunked(rng, _uniform, M, D)
        y = _chunked(rng, _uniform, N, D)
        b = _chunked(rng, _normal, N, E)
    elif dist == "normal_scaled":
        std = 1.0 / np.sqrt(50.0)
        x = _chunked(rng, lambda r, s: r.standard_normal(s) * std, M, D)
        y = _chunked(rng, lambda r, s: r.standard_normal(s) * std, N, D)
        b = _chunked(rng, _normal, N, E)
    elif dist == "mixture16":
        centres = rng.uniform(-5.0, 5.0, (16, D))
        pts = []
        for n in (M, N):
            lab = rng.integers(0, 16, n)
            p = np.empty((n, D), np.float32)
            for s in range(0, n, CHUNK_ROWS):
                e = min(n, s + CHUNK_ROWS)
                p[s:e] = centres[lab[s:e]] + 0.5 * rng.standard_normal((e - s, D))
            pts.append(p)
        x, y = pts
        b = None
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return x, y, b


def make_inputs(w: Workload | str, seed: int = 0, M: int | None = None, N: int | None = None):
    """Inputs of a named workload; ``M``/``N`` override the sizes (same recipe)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    return make_points(w.dist, w.M if M is None else M, w.N if N is None else N, w.D, w.E, seed)


def sample_rows(M: int, n: int, seed: int = 1) -> np.ndarray:
    """Sorted seeded sample of ``n`` distinct row indices in [0, M) (all rows if n >= M)."""
    if n >= M:
        return np.arange(M, dtype=np.int64)
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(M, n, replace=False)).astype(np.int64)


def random_points(rng: np.random.Generator, M: int, N: int, D: int, E: int,
                  scale: float = 1.0, offset: float = 0.0):
    """Small ad-hoc normal inputs for tests (x, y, b float32)."""
    x = (rng.standard_normal((M, D)) * scale + offset).astype(np.float32)
    y = (rng.standard_normal((N, D)) * scale + offset).astype(np.float32)
    b = rng.standard_normal((N, E)).astype(np.float32)
    return x, y, b
