"""Pins of the oracle against facts that do not come from the oracle itself.

Each ``pin_*`` function takes an optional ``lib`` (a handle from
``oracle.open_library``) and raises AssertionError when the oracle disagrees
with brute force (an explicitly materialised matrix evaluated with numpy,
scipy or torch float64 autograd), a closed form, a limit or an invariant.
``tests/test_oracle.py`` runs them on the committed oracle;
``tests/test_oracle_mutants.py`` runs them on deliberately broken copies of
the oracle source and checks that every planted mistake is caught.

Passages (KeOps pages): "Kernel Operations on the GPU, with Autodiff, without
Memory Overflows" §1 "Target operation" (Gaussian kernel sum), §2 reductions
list and autodiff; KeOps README PyTorch example (D_ij, K_ij = exp(-D_ij),
.sum, .logsumexp, .argmin, grad of (a**2).sum()).
"""
from __future__ import annotations

import math

import numpy as np
import scipy.special
import torch

import oracle


# --------------------------------------------------------------------------- helpers
def dyadic(rng, shape, lo=-4.0, hi=4.0, step=1 / 64):
    """float32 values on a grid of spacing ``step`` (sums/products stay exact in fp32)."""
    n = int(round((hi - lo) / step))
    return (lo + step * rng.integers(0, n + 1, size=shape)).astype(np.float32)


def brute_sqdist(x, y):
    """Materialised |x_i - y_j|^2 in float64, summed over d in index order."""
    x = x.astype(np.float64)
    y = y.astype(np.float64)
    out = np.zeros((x.shape[0], y.shape[0]))
    for d in range(x.shape[1]):
        out += (x[:, None, d] - y[None, :, d]) ** 2
    return out


def brute_K(x, y, sigma):
    return np.exp(-brute_sqdist(x, y) / float(sigma) ** 2)


def rel_close(a, b, rtol, atol=0.0):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    err = np.abs(a - b)
    bad = err > rtol * np.abs(b) + atol
    assert not bad.any(), f"max err {err.max():.3e} at {np.argwhere(bad)[:3].tolist()}"


SHAPES = [(1, 1, 1, 1), (5, 7, 2, 1), (17, 33, 3, 1), (16, 9, 3, 3), (8, 64, 5, 2),
          (12, 20, 32, 1), (6, 11, 50, 1), (9, 13, 64, 3)]


# --------------------------------------------------------------------------- sum
def pin_sum_brute(lib=None):
    """Sum and its normaliser equal the materialised K @ b (numpy float64)."""
    rng = np.random.default_rng(11)
    for (M, N, D, E) in SHAPES:
        for sigma in (0.7, 1.0, 2.5 * math.sqrt(D)):
            x = rng.standard_normal((M, D)).astype(np.float32)
            y = rng.standard_normal((N, D)).astype(np.float32)
            b = rng.standard_normal((N, E)).astype(np.float32)
            a, n = oracle.gauss_sum(x, y, b, np.float32(sigma), lib=lib)
            K = brute_K(x, y, np.float32(sigma))
            rel_close(a, K @ b.astype(np.float64), 1e-12, 1e-300)
            rel_close(n, np.abs(K[:, :, None] * b.astype(np.float64)[None]).sum(1), 1e-12, 1e-300)
            rows = np.array(sorted(rng.choice(M, min(M, 3), replace=False)), np.int64)
            a2, _ = oracle.gauss_sum(x, y, b, np.float32(sigma), rows=rows, lib=lib)
            assert np.array_equal(a2, a[rows])


def pin_sum_single_point(lib=None):
    """M = N = 1 and x = y: K = exp(0) = 1, so a = b exactly."""
    rng = np.random.default_rng(3)
    for D in (1, 3, 64):
        for E in (1, 4):
            x = rng.standard_normal((1, D)).astype(np.float32)
            b = rng.standard_normal((1, E)).astype(np.float32)
            a, n = oracle.gauss_sum(x, x.copy(), b, 0.3, lib=lib)
            assert np.array_equal(a, b.astype(np.float64))
            assert np.array_equal(n, np.abs(b.astype(np.float64)))


def pin_sum_sigma_infinite(lib=None):
    """sigma -> infinity: every K_ij -> 1, so a_i -> sum_j b_j."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((6, 3)).astype(np.float32)
    y = rng.standard_normal((40, 3)).astype(np.float32)
    b = rng.standard_normal((40, 2)).astype(np.float32)
    a, _ = oracle.gauss_sum(x, y, b, 1e8, lib=lib)
    expect = np.broadcast_to(b.astype(np.float64).sum(0), a.shape)
    rel_close(a, expect, 1e-12, 1e-12)


def pin_sum_sigma_zero(lib=None):
    """sigma -> 0: a_i -> sum of b_j over the y_j equal to x_i (others vanish)."""
    rng = np.random.default_rng(5)
    x = dyadic(rng, (10, 3), step=1 / 8)
    y = np.concatenate([x[[1, 4, 4, 7]], dyadic(rng, (30, 3), step=1 / 8) + np.float32(0.0625)])
    b = rng.standard_normal((y.shape[0], 1)).astype(np.float32)
    a, _ = oracle.gauss_sum(x, y, b, 1e-3, lib=lib)
    expect = np.zeros((10, 1))
    for j in range(y.shape[0]):
        for i in range(10):
            if np.array_equal(x[i], y[j]):
                expect[i, 0] += float(b[j, 0])
    rel_close(a, expect, 1e-12, 1e-300)


def pin_sum_separable_grid(lib=None):
    """y on a Cartesian grid G1 x G2 x G3 with b = 1: a_i is a product of 1-D sums."""
    rng = np.random.default_rng(6)
    grids = [np.float32([-1.0, 0.0, 0.5, 2.0]), np.float32([-0.75, 0.25, 1.0, 1.5, 3.0]),
             np.float32([0.0, 1.0, -2.0])]
    y = np.array([[g0, g1, g2] for g0 in grids[0] for g1 in grids[1] for g2 in grids[2]],
                 np.float32)
    b = np.ones((y.shape[0], 1), np.float32)
    x = rng.standard_normal((7, 3)).astype(np.float32)
    sigma = 0.8
    a, _ = oracle.gauss_sum(x, y, b, sigma, lib=lib)
    for i in range(7):
        prod = 1.0
        for d in range(3):
            prod *= sum(math.exp(-((float(x[i, d]) - float(g)) ** 2) / sigma ** 2)
                        for g in grids[d])
        assert abs(a[i, 0] - prod) <= 1e-12 * prod, (i, a[i, 0], prod)


def pin_sum_translation(lib=None):
    """Shifting x and y by the same vector leaves a unchanged (inputs exact on a dyadic grid)."""
    rng = np.random.default_rng(7)
    x = dyadic(rng, (9, 3))
    y = dyadic(rng, (25, 3))
    b = rng.standard_normal((25, 1)).astype(np.float32)
    shift = np.float32([8.0, -4.0, 2.0])
    a1, _ = oracle.gauss_sum(x, y, b, 1.3, lib=lib)
    a2, _ = oracle.gauss_sum(x + shift, y + shift, b, 1.3, lib=lib)
    n1, _ = oracle.gauss_sum(x, y, np.abs(b), 1.3, lib=lib)
    assert np.all(np.abs(a1 - a2) <= 1e-13 * n1)


def pin_sum_columns_independent(lib=None):
    """Column e of a depends only on column e of b (E=3 equals three E=1 calls)."""
    rng = np.random.default_rng(8)
    x = rng.standard_normal((5, 4)).astype(np.float32)
    y = rng.standard_normal((12, 4)).astype(np.float32)
    b = rng.standard_normal((12, 3)).astype(np.float32)
    a, _ = oracle.gauss_sum(x, y, b, 1.1, lib=lib)
    for e in range(3):
        ae, _ = oracle.gauss_sum(x, y, b[:, e:e + 1], 1.1, lib=lib)
        assert np.array_equal(ae[:, 0], a[:, e])


def pin_sum_empty(lib=None):
    """N = 0: empty sums are 0; M = 0 gives an empty output."""
    x = np.ones((3, 2), np.float32)
    a, n = oracle.gauss_sum(x, np.zeros((0, 2), np.float32), np.zeros((0, 1), np.float32), 1.0,
                            lib=lib)
    assert a.shape == (3, 1) and not a.any() and not n.any()
    a, n = oracle.gauss_sum(np.zeros((0, 2), np.float32), x, np.ones((3, 1), np.float32), 1.0,
                            lib=lib)
    assert a.shape == (0, 1)


# --------------------------------------------------------------------------- lse
def pin_lse_brute(lib=None):
    """LSE equals scipy.special.logsumexp of the materialised -D_ij/sigma^2 + b_j."""
    rng = np.random.default_rng(21)
    for (M, N, D, E) in SHAPES:
        for sigma in (0.2, 1.0, 3.0):
            x = rng.standard_normal((M, D)).astype(np.float32)
            y = rng.standard_normal((N, D)).astype(np.float32)
            b = (3 * rng.standard_normal((N, E))).astype(np.float32)
            l = oracle.gauss_lse(x, y, b, np.float32(sigma), lib=lib)
            s2 = float(np.float32(sigma)) ** 2
            V = -brute_sqdist(x, y)[:, :, None] / s2 + b.astype(np.float64)[None]
            ref = scipy.special.logsumexp(V, axis=1)
            rel_close(l, ref, 1e-12, 1e-12)


def pin_lse_naive(lib=None):
    """On moderate values LSE equals log(sum(exp(v))) written out naively."""
    rng = np.random.default_rng(22)
    x = rng.standard_normal((6, 3)).astype(np.float32)
    y = rng.standard_normal((15, 3)).astype(np.float32)
    b = rng.standard_normal((15, 1)).astype(np.float32)
    l = oracle.gauss_lse(x, y, b, 1.5, lib=lib)
    for i in range(6):
        s = 0.0
        for j in range(15):
            d2 = sum((float(x[i, d]) - float(y[j, d])) ** 2 for d in range(3))
            s += math.exp(-d2 / 2.25 + float(b[j, 0]))
        assert abs(l[i, 0] - math.log(s)) <= 1e-12 * (1 + abs(math.log(s)))


def pin_lse_shift_and_sum(lib=None):
    """b -> b + c shifts LSE by c; with b = log w, LSE = log(sum with weights w)."""
    rng = np.random.default_rng(23)
    x = rng.standard_normal((8, 3)).astype(np.float32)
    y = rng.standard_normal((30, 3)).astype(np.float32)
    b = dyadic(rng, (30, 2), lo=-2, hi=2, step=1 / 32)
    l0 = oracle.gauss_lse(x, y, b, 0.9, lib=lib)
    l1 = oracle.gauss_lse(x, y, b + np.float32(40.0), 0.9, lib=lib)
    rel_close(l1 - 40.0, l0, 0, 1e-12)
    w = np.exp(b.astype(np.float64)).astype(np.float32)   # fp32 weights: rounding <= 6e-8 rel
    a, _ = oracle.gauss_sum(x, y, w, 0.9, lib=lib)
    rel_close(l0, np.log(a), 0, 2e-7)


def pin_lse_large_offsets(lib=None):
    """Huge |b| and tiny sigma do not overflow: the max is factored out."""
    rng = np.random.default_rng(24)
    x = rng.standard_normal((4, 2)).astype(np.float32)
    y = rng.standard_normal((20, 2)).astype(np.float32)
    b = (rng.standard_normal((20, 1)) * 3 + 800.0).astype(np.float32)
    l = oracle.gauss_lse(x, y, b, np.float32(0.01), lib=lib)
    V = -brute_sqdist(x, y) / float(np.float32(0.01)) ** 2 + b.astype(np.float64)[:, 0][None]
    rel_close(l[:, 0], scipy.special.logsumexp(V, axis=1), 1e-13, 0)
    assert np.isfinite(l).all()


def pin_lse_empty(lib=None):
    """N = 0: the log of an empty sum is -inf."""
    l = oracle.gauss_lse(np.ones((2, 3), np.float32), np.zeros((0, 3), np.float32),
                         np.zeros((0, 1), np.float32), 1.0, lib=lib)
    assert np.all(np.isneginf(l))


# --------------------------------------------------------------------------- grad_x
def pin_grad_autograd(lib=None):
    """grad_x equals torch float64 autograd of sum(g * a) on the materialised matrix."""
    rng = np.random.default_rng(31)
    for (M, N, D, E) in SHAPES:
        sigma = np.float32(0.9 * math.sqrt(D))
        x = rng.standard_normal((M, D)).astype(np.float32)
        y = rng.standard_normal((N, D)).astype(np.float32)
        b = rng.standard_normal((N, E)).astype(np.float32)
        g = rng.standard_normal((M, E)).astype(np.float32)
        G, nu = oracle.gauss_grad_x(x, y, b, g, sigma, lib=lib)
        xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
        yt = torch.tensor(y, dtype=torch.float64)
        d2 = ((xt[:, None, :] - yt[None, :, :]) ** 2).sum(-1)
        a = torch.exp(-d2 / float(sigma) ** 2) @ torch.tensor(b, dtype=torch.float64)
        (ref,) = torch.autograd.grad((a * torch.tensor(g, dtype=torch.float64)).sum(), [xt])
        rel_close(G, ref.numpy(), 0, 1e-12 * (1 + nu.max()))
        assert np.all(np.abs(G) <= nu * (1 + 1e-12))


def pin_grad_finite_differences(lib=None):
    """Central differences of L(x) = sum_ie g_ie a_ie(x), all in double, match grad_x."""
    rng = np.random.default_rng(32)
    M, N, D, E = 4, 25, 3, 2
    x = dyadic(rng, (M, D), lo=-1, hi=1, step=1 / 16)
    y = rng.standard_normal((N, D)).astype(np.float32)
    b = rng.standard_normal((N, E)).astype(np.float32)
    g = rng.standard_normal((M, E)).astype(np.float32)
    sigma = 1.25
    G, nu = oracle.gauss_grad_x(x, y, b, g, sigma, lib=lib)
    h = np.float32(2.0 ** -10)            # x +- h stays exact in fp32
    for i in range(M):
        for d in range(D):
            xp, xm = x.copy(), x.copy()
            xp[i, d] += h
            xm[i, d] -= h
            ap, _ = oracle.gauss_sum(xp, y, b, sigma, lib=lib)
            am, _ = oracle.gauss_sum(xm, y, b, sigma, lib=lib)
            fd = ((ap - am) * g.astype(np.float64)).sum() / (2 * float(h))
            assert abs(fd - G[i, d]) <= 1e-5 * nu[i, d] + 1e-12, (i, d, fd, G[i, d], nu[i, d])


def pin_grad_identity(lib=None):
    """E = 1: G_i = (-2/sigma^2) g_i (x_i a_i - sum_j K_ij b_j y_j), from sum-oracle calls."""
    rng = np.random.default_rng(33)
    M, N, D = 6, 40, 3
    x = dyadic(rng, (M, D), step=1 / 16)
    y = dyadic(rng, (N, D), step=1 / 16)
    b = dyadic(rng, (N, 1), step=1 / 16)
    g = dyadic(rng, (M, 1), step=1 / 16)
    sigma = 1.5
    G, nu = oracle.gauss_grad_x(x, y, b, g, sigma, lib=lib)
    a, _ = oracle.gauss_sum(x, y, b, sigma, lib=lib)
    by = (b * y).astype(np.float32)       # exact: few mantissa bits on each side
    assert np.array_equal(by.astype(np.float64), b.astype(np.float64) * y.astype(np.float64))
    s, _ = oracle.gauss_sum(x, y, by, sigma, lib=lib)
    expect = (-2 / sigma ** 2) * g.astype(np.float64) * (x.astype(np.float64) * a - s)
    rel_close(G, expect, 0, 1e-12 * (1 + nu.max()))


# --------------------------------------------------------------------------- grad_y, grad_b
def pin_grad_yb_autograd(lib=None):
    """grad_y and grad_b equal torch float64 autograd of sum(g * a) in y and in b; a
    scrambled subset of the points gives the same values for those points."""
    rng = np.random.default_rng(51)
    for (M, N, D, E) in SHAPES:
        sigma = np.float32(0.9 * math.sqrt(D))
        x = rng.standard_normal((M, D)).astype(np.float32)
        y = rng.standard_normal((N, D)).astype(np.float32)
        b = rng.standard_normal((N, E)).astype(np.float32)
        g = rng.standard_normal((M, E)).astype(np.float32)
        Gy, nuy = oracle.gauss_grad_y(x, y, b, g, sigma, lib=lib)
        Gb, nub = oracle.gauss_grad_b(x, y, g, sigma, lib=lib)
        xt = torch.tensor(x, dtype=torch.float64)
        yt = torch.tensor(y, dtype=torch.float64, requires_grad=True)
        bt = torch.tensor(b, dtype=torch.float64, requires_grad=True)
        d2 = ((xt[:, None, :] - yt[None, :, :]) ** 2).sum(-1)
        a = torch.exp(-d2 / float(sigma) ** 2) @ bt
        ref_y, ref_b = torch.autograd.grad((a * torch.tensor(g, dtype=torch.float64)).sum(), [yt, bt])
        rel_close(Gy, ref_y.numpy(), 0, 1e-12 * (1 + nuy.max()))
        rel_close(Gb, ref_b.numpy(), 0, 1e-12 * (1 + nub.max()))
        assert np.all(np.abs(Gy) <= nuy * (1 + 1e-12)) and np.all(np.abs(Gb) <= nub * (1 + 1e-12))
        cols = rng.permutation(N)[: max(1, N // 2)]
        assert np.array_equal(oracle.gauss_grad_y(x, y, b, g, sigma, cols=cols, lib=lib)[0], Gy[cols])
        assert np.array_equal(oracle.gauss_grad_b(x, y, g, sigma, cols=cols, lib=lib)[0], Gb[cols])


def pin_grad_y_finite_differences(lib=None):
    """Central differences of L(y) = sum_ie g_ie a_ie(y), all in double, match grad_y."""
    rng = np.random.default_rng(52)
    M, N, D, E = 30, 4, 3, 2
    x = rng.standard_normal((M, D)).astype(np.float32)
    y = dyadic(rng, (N, D), lo=-1, hi=1, step=1 / 16)
    b = rng.standard_normal((N, E)).astype(np.float32)
    g = rng.standard_normal((M, E)).astype(np.float32)
    sigma = 1.25
    Gy, nu = oracle.gauss_grad_y(x, y, b, g, sigma, lib=lib)
    h = np.float32(2.0 ** -10)            # y +- h stays exact in fp32
    for j in range(N):
        for d in range(D):
            yp, ym = y.copy(), y.copy()
            yp[j, d] += h
            ym[j, d] -= h
            ap, _ = oracle.gauss_sum(x, yp, b, sigma, lib=lib)
            am, _ = oracle.gauss_sum(x, ym, b, sigma, lib=lib)
            fd = ((ap - am) * g.astype(np.float64)).sum() / (2 * float(h))
            assert abs(fd - Gy[j, d]) <= 1e-5 * nu[j, d] + 1e-12, (j, d, fd, Gy[j, d], nu[j, d])


def pin_grad_b_linear(lib=None):
    """L = sum g * a is linear in b: a central difference with step 1 is exact up to rounding."""
    rng = np.random.default_rng(53)
    M, N, D, E = 20, 6, 3, 3
    x = rng.standard_normal((M, D)).astype(np.float32)
    y = rng.standard_normal((N, D)).astype(np.float32)
    b = dyadic(rng, (N, E), step=1 / 16)
    g = rng.standard_normal((M, E)).astype(np.float32)
    sigma = 1.1
    Gb, nu = oracle.gauss_grad_b(x, y, g, sigma, lib=lib)
    for j in range(N):
        for e in range(E):
            bp, bm = b.copy(), b.copy()
            bp[j, e] += 1
            bm[j, e] -= 1
            ap, _ = oracle.gauss_sum(x, y, bp, sigma, lib=lib)
            am, _ = oracle.gauss_sum(x, y, bm, sigma, lib=lib)
            fd = ((ap - am) * g.astype(np.float64)).sum() / 2
            assert abs(fd - Gb[j, e]) <= 1e-12 * (1 + nu[j, e]), (j, e, fd, Gb[j, e])


def pin_grad_pairing_and_balance(lib=None):
    """<Gb, b> = <g, a> (a is linear in b), and sum_i Gx_i + sum_j Gy_j = 0 (the kernel
    depends on x - y only, so moving every point together leaves L unchanged)."""
    rng = np.random.default_rng(54)
    for (M, N, D, E) in [(13, 21, 3, 1), (8, 30, 5, 2), (25, 7, 2, 3)]:
        sigma = 1.3
        x = rng.standard_normal((M, D)).astype(np.float32)
        y = rng.standard_normal((N, D)).astype(np.float32)
        b = rng.standard_normal((N, E)).astype(np.float32)
        g = rng.standard_normal((M, E)).astype(np.float32)
        a, n = oracle.gauss_sum(x, y, b, sigma, lib=lib)
        Gb, nub = oracle.gauss_grad_b(x, y, g, sigma, lib=lib)
        lhs = (Gb * b.astype(np.float64)).sum()
        rhs = (g.astype(np.float64) * a).sum()
        scale = (nub * np.abs(b)).sum() + (np.abs(g) * n).sum()
        assert abs(lhs - rhs) <= 1e-12 * scale, (lhs, rhs)
        Gx, nux = oracle.gauss_grad_x(x, y, b, g, sigma, lib=lib)
        Gy, nuy = oracle.gauss_grad_y(x, y, b, g, sigma, lib=lib)
        tot = Gx.sum(0) + Gy.sum(0)
        assert np.all(np.abs(tot) <= 1e-12 * (nux.sum(0) + nuy.sum(0))), tot


# --------------------------------------------------------------------------- kernel matrix, dense solve
def pin_matrix_brute_and_sum(lib=None):
    """The materialised kernel matrix equals numpy's, and K @ b equals the sum oracle."""
    rng = np.random.default_rng(61)
    for (M, N, D, E) in SHAPES[:6]:
        sigma = 0.8 * math.sqrt(D)
        x = rng.standard_normal((M, D)).astype(np.float32)
        y = rng.standard_normal((N, D)).astype(np.float32)
        b = rng.standard_normal((N, E)).astype(np.float32)
        K = oracle.gauss_matrix(x, y, sigma, lib=lib)
        rel_close(K, brute_K(x, y, sigma), 1e-14)
        a, n = oracle.gauss_sum(x, y, b, sigma, lib=lib)
        rel_close(K @ b.astype(np.float64), a, 0, 1e-12 * (1 + n.max()))


def pin_solve_closed_forms(lib=None):
    """(K + lam I) a = b: K = I for far-apart points gives b / (1 + lam); two points at
    squared distance d give the 2 x 2 inverse with k = exp(-d / sigma^2)."""
    rng = np.random.default_rng(62)
    x = (np.arange(12, dtype=np.float32)[:, None] * np.float32(100.0)).repeat(2, 1)
    b = rng.standard_normal((12, 2)).astype(np.float32)
    a = oracle.gauss_solve(x, b, 1.0, 0.25, lib=lib)
    rel_close(a, b.astype(np.float64) / 1.25, 1e-14)
    x2 = np.array([[0.0, 0.0], [0.75, 0.5]], np.float32)
    b2 = np.array([[1.0], [-2.0]], np.float32)
    sigma, lam = 0.9, 0.3
    k = math.exp(-(0.75 ** 2 + 0.5 ** 2) / sigma ** 2)
    det = (1 + lam) ** 2 - k ** 2
    expect = np.array([[((1 + lam) * 1.0 - k * -2.0) / det], [((1 + lam) * -2.0 - k * 1.0) / det]])
    rel_close(oracle.gauss_solve(x2, b2, sigma, lam, lib=lib), expect, 1e-13)


def pin_solve_residual(lib=None):
    """The dense solution leaves a residual at rounding level when the system is applied
    through the sum oracle (an independent route to K a)."""
    rng = np.random.default_rng(63)
    for (N, D, E, sigma, lam) in [(60, 3, 1, 0.5, 0.1), (40, 5, 2, 1.5, 1.0), (25, 2, 3, 0.3, 0.01)]:
        x = rng.standard_normal((N, D)).astype(np.float32)
        b = rng.standard_normal((N, E)).astype(np.float32)
        a = oracle.gauss_solve(x, b, sigma, lam, lib=lib)
        K = oracle.gauss_matrix(x, x, sigma, lib=lib)
        assert np.allclose(K, K.T, rtol=0, atol=0) and np.linalg.eigvalsh(K).min() > -1e-12
        Ka = np.stack([oracle.gauss_sum(x, x, a[:, e:e + 1].astype(np.float32), sigma, lib=lib)[0][:, 0]
                       for e in range(E)], 1)
        # a rounded to fp32 for the sum oracle: the residual is that rounding times (K + lam I)
        r = b - Ka - lam * a.astype(np.float32).astype(np.float64)
        bound = 2.0 ** -23 * (np.abs(K).sum(1, keepdims=True) + lam) * np.abs(a).max(0, keepdims=True)
        assert np.all(np.abs(r) <= bound + 1e-12), np.abs(r).max()


def pin_system_residual(lib=None, residual=None):
    """oracle.gauss_system_residual, the checker of the conjugate-gradient solver ([README]
    feature list: conjugate gradient solver for kriging), against facts that do not come from
    it: a = 0 leaves r = b exactly; far-apart points make K the identity, so r = b - (1 + lam) a
    (exact on dyadic values); the dense solution leaves a rounding-level residual; a row
    selection returns exactly those rows of the full residual.  ``residual`` replaces the
    helper (planted mistakes in a copy of it must fail here)."""
    res = residual or oracle.gauss_system_residual
    rng = np.random.default_rng(64)
    # a = 0: no product contributes
    x = rng.standard_normal((30, 3)).astype(np.float32)
    b = rng.standard_normal((30, 2)).astype(np.float32)
    r0 = res(x, b, np.zeros((30, 2), np.float32), 0.7, 0.5, lib=lib)
    assert r0.shape == (30, 2) and np.array_equal(r0, b.astype(np.float64))
    # K = I (points 100 apart, sigma 1: exp(-1e4) is exactly 0 in double), dyadic a, b, lam
    xf = (np.arange(16, dtype=np.float32)[:, None] * np.float32(100.0)).repeat(3, 1)
    af = dyadic(rng, (16, 2))
    bf = dyadic(rng, (16, 2))
    for lam in (0.25, 0.0, 3.0):
        rf = res(xf, bf, af, 1.0, lam, lib=lib)
        assert np.array_equal(rf, bf.astype(np.float64) - (1.0 + lam) * af.astype(np.float64)), lam
    # the dense solve, rounded to fp32, leaves a residual of fp32 rounding times (K + lam I)
    for (N, D, E, sigma, lam) in [(50, 3, 1, 0.6, 0.2), (35, 4, 2, 1.2, 2.0)]:
        xs = rng.standard_normal((N, D)).astype(np.float32)
        bs = rng.standard_normal((N, E)).astype(np.float32)
        a = oracle.gauss_solve(xs, bs, sigma, lam, lib=lib)
        K = brute_K(xs, xs, sigma)
        r = res(xs, bs, a.astype(np.float32), sigma, lam, lib=lib)
        bound = 2.0 ** -23 * (K.sum(1, keepdims=True) + lam) * np.abs(a).max(0, keepdims=True)
        assert r.shape == (N, E) and np.all(np.abs(r) <= bound + 1e-12), np.abs(r).max()
        # a residual that is not small: a perturbed solution; its residual is (K + lam I) delta
        delta = dyadic(rng, (N, E), -1.0, 1.0)
        a2 = (a.astype(np.float32) + delta).astype(np.float32)
        r2 = res(xs, bs, a2, sigma, lam, lib=lib)
        expect = bs.astype(np.float64) - (K + lam * np.eye(N)) @ a2.astype(np.float64)
        rel_close(r2, expect, 0, 1e-12 * (1 + np.abs(expect).max()))
        # rows: exactly the selected rows of the full call, in the given order
        rows = np.array([N - 1, 0, 7, 3], np.int64)
        full = res(xs, bs, a2, sigma, lam, lib=lib)
        sub = res(xs, bs, a2, sigma, lam, rows=rows, lib=lib)
        assert sub.shape == (4, E) and np.array_equal(sub, full[rows])


# --------------------------------------------------------------------------- block-sparse ranges
def random_ranges(rng, M, N, n_row_ranges, max_j_ranges, cover=False):
    """Disjoint row ranges (a partition of [0, M) when ``cover``, else with gaps), each meeting
    0..max_j_ranges random j ranges; returns (ranges_i, slices_i, redranges_j) and the mask."""
    cuts = np.sort(rng.choice(np.arange(1, M), size=min(n_row_ranges - 1, M - 1), replace=False)).tolist() \
        if M > 1 else []
    bounds = [0, *cuts, M]
    ranges_i, slices_i, redr = [], [], []
    mask = np.zeros((M, N), np.int64)
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        if not cover and rng.random() < 0.25:
            continue                                         # a gap: rows in no range
        for _ in range(int(rng.integers(0, max_j_ranges + 1))):
            a, c = sorted(rng.integers(0, N + 1, size=2).tolist())
            redr.append([a, c])
            mask[lo:hi, a:c] += 1
        ranges_i.append([lo, hi])
        slices_i.append(len(redr))
    return (np.array(ranges_i, np.int64).reshape(-1, 2), np.array(slices_i, np.int64),
            np.array(redr, np.int64).reshape(-1, 2), mask)


def pin_ranges_brute_mask(lib=None):
    """The block-sparse sum and LSE equal the dense formulas with a materialised pair mask
    (a pair listed twice counts twice); rows in no range get 0 and -inf."""
    rng = np.random.default_rng(71)
    for (M, N, D, E) in [(30, 40, 3, 1), (17, 50, 2, 2), (25, 9, 5, 3), (1, 1, 1, 1)]:
        sigma = 1.2
        x = rng.standard_normal((M, D)).astype(np.float32)
        y = rng.standard_normal((N, D)).astype(np.float32)
        b = rng.standard_normal((N, E)).astype(np.float32)
        ri, si, rj, mask = random_ranges(rng, M, N, 5, 3)
        a, n = oracle.gauss_sum_ranges(x, y, b, sigma, ri, si, rj, lib=lib)
        W = mask * brute_K(x, y, sigma)
        rel_close(a, W @ b.astype(np.float64), 0, 1e-12 * (1 + n.max()))
        rel_close(n, W @ np.abs(b.astype(np.float64)), 1e-12)
        l = oracle.gauss_lse_ranges(x, y, b, sigma, ri, si, rj, lib=lib)
        V = -brute_sqdist(x, y)[:, :, None] / sigma ** 2 + b.astype(np.float64)[None, :, :]
        ref = scipy.special.logsumexp(V, axis=1, b=np.broadcast_to(mask[:, :, None], V.shape))
        ref = np.where(mask.sum(1)[:, None] > 0, ref, -np.inf)
        fin = np.isfinite(ref)
        assert np.array_equal(fin, np.isfinite(l))
        rel_close(l[fin], ref[fin], 0, 1e-12 * (1 + np.abs(ref[fin]).max()) if fin.any() else 0)


def pin_ranges_dense_and_split(lib=None):
    """One row range meeting [0, N) is exactly the dense reduction; cutting a j range in two, or
    a row range in two with the same j list, changes nothing (same order, same terms)."""
    rng = np.random.default_rng(72)
    M, N, D, E = 23, 37, 3, 2
    x = rng.standard_normal((M, D)).astype(np.float32)
    y = rng.standard_normal((N, D)).astype(np.float32)
    b = rng.standard_normal((N, E)).astype(np.float32)
    a0, n0 = oracle.gauss_sum(x, y, b, 0.9, lib=lib)
    a1, n1 = oracle.gauss_sum_ranges(x, y, b, 0.9, [[0, M]], [1], [[0, N]], lib=lib)
    assert np.array_equal(a0, a1) and np.array_equal(n0, n1)
    assert np.array_equal(oracle.gauss_lse(x, y, b, 0.9, lib=lib),
                          oracle.gauss_lse_ranges(x, y, b, 0.9, [[0, M]], [1], [[0, N]], lib=lib))
    a2, _ = oracle.gauss_sum_ranges(x, y, b, 0.9, [[0, 9], [9, M]], [2, 4], [[0, 15], [15, N], [0, 15], [15, N]],
                                    lib=lib)
    assert np.array_equal(a0, a2)
    # an empty j list and a range list that skips rows
    a3, _ = oracle.gauss_sum_ranges(x, y, b, 0.9, [[2, 5], [7, 8]], [0, 1], [[4, 6]], lib=lib)
    assert not a3[[0, 1, 5, 6] + list(range(8, M))].any() and not a3[2:5].any() and a3[7].all()
    assert np.isneginf(oracle.gauss_lse_ranges(x, y, b, 0.9, [[2, 5]], [0], np.zeros((0, 2)), lib=lib)).all()


# --------------------------------------------------------------------------- max / argmax
def pin_max_brute(lib=None):
    """Max/ArgMax and Min/ArgMin of K b equal numpy's on the materialised product (first index
    on ties, forced with duplicated points and payloads); N = 0 gives -inf and -1."""
    rng = np.random.default_rng(81)
    for (M, N, D, E) in SHAPES:
        sigma = 0.9 * math.sqrt(D)
        x = rng.standard_normal((M, D)).astype(np.float32)
        y = rng.standard_normal((N, D)).astype(np.float32)
        b = rng.standard_normal((N, E)).astype(np.float32)
        if N >= 4:
            y[N - 1], b[N - 1] = y[0], b[0]          # exact ties: the smaller index wins
        P = brute_K(x, y, sigma)[:, :, None] * b.astype(np.float64)[None, :, :]
        v, i = oracle.gauss_max(x, y, b, sigma, 1, lib=lib)
        assert np.array_equal(i, P.argmax(1))
        rel_close(v, P.max(1), 1e-13)
        v, i = oracle.gauss_max(x, y, b, sigma, -1, lib=lib)
        assert np.array_equal(i, P.argmin(1))
        rel_close(-v, P.min(1), 1e-13)
    v, i = oracle.gauss_max(np.zeros((3, 2), np.float32), np.zeros((0, 2), np.float32), np.zeros((0, 1), np.float32),
                            1.0, lib=lib)
    assert np.isneginf(v).all() and (i == -1).all()


# --------------------------------------------------------------------------- Laplacian kernel
def pin_laplace_brute_and_limits(lib=None):
    """exp(-|x - y| / sigma) sums equal numpy's materialised product; x = y gives b; a very large
    sigma gives sum_j b_j; D = 1 on a sorted line is a geometric-series closed form."""
    rng = np.random.default_rng(91)
    for (M, N, D, E) in SHAPES:
        sigma = 0.7 * math.sqrt(D)
        x = rng.standard_normal((M, D)).astype(np.float32)
        y = rng.standard_normal((N, D)).astype(np.float32)
        b = rng.standard_normal((N, E)).astype(np.float32)
        a, n = oracle.laplace_sum(x, y, b, sigma, lib=lib)
        Kl = np.exp(-np.sqrt(brute_sqdist(x, y)) / sigma)
        rel_close(a, Kl @ b.astype(np.float64), 0, 1e-12 * (1 + n.max()))
    p = np.array([[0.25, -1.5]], np.float32)
    bb = np.array([[2.0, -3.0]], np.float32)
    rel_close(oracle.laplace_sum(p, p, bb, 0.3, lib=lib)[0], bb, 0)
    y = rng.standard_normal((40, 3)).astype(np.float32)
    b = rng.standard_normal((40, 1)).astype(np.float32)
    rel_close(oracle.laplace_sum(y[:5], y, b, 1e9, lib=lib)[0], np.full((5, 1), b.astype(np.float64).sum()), 1e-7)
    # points 0, h, 2h, ... on a line, b = 1: a_0 = sum_k q^k with q = exp(-h / sigma)
    h, sigma, n = 0.25, 0.8, 30
    line = (np.arange(n, dtype=np.float32) * np.float32(h))[:, None]
    q = math.exp(-h / sigma)
    a0 = oracle.laplace_sum(line[:1], line, np.ones((n, 1), np.float32), sigma, lib=lib)[0][0, 0]
    assert abs(a0 - (1 - q ** n) / (1 - q)) <= 1e-13 * a0


# --------------------------------------------------------------------------- kmin
def pin_kmin_argsort(lib=None):
    """K-min equals a stable argsort of the materialised distances (ties -> smaller j)."""
    rng = np.random.default_rng(41)
    for (M, N, D, _) in SHAPES:
        for K in sorted({1, min(N, 3), min(N, 10), N}):
            x = rng.standard_normal((M, D)).astype(np.float32)
            y = rng.standard_normal((N, D)).astype(np.float32)
            if N >= 4:                     # exact duplicates force distance ties
                y[N - 1] = y[1]
                y[N - 2] = y[0]
            d, idx = oracle.kmin(x, y, K, lib=lib)
            D2 = brute_sqdist(x, y)
            order = np.argsort(D2, axis=1, kind="stable")[:, :K]
            assert np.array_equal(idx, order), (M, N, D, K)
            assert np.array_equal(d, np.take_along_axis(D2, order, 1))


def pin_kmin_invariants(lib=None):
    """K = 1 is argmin; K = N is a permutation; returned distances recompute exactly."""
    rng = np.random.default_rng(42)
    x = rng.standard_normal((10, 3)).astype(np.float32)
    y = rng.standard_normal((50, 3)).astype(np.float32)
    d1, i1 = oracle.kmin(x, y, 1, lib=lib)
    D2 = brute_sqdist(x, y)
    assert np.array_equal(i1[:, 0], D2.argmin(1))
    dN, iN = oracle.kmin(x, y, 50, lib=lib)
    assert all(sorted(r) == list(range(50)) for r in iN.tolist())
    assert np.all(np.diff(dN, axis=1) >= 0)
    ii = np.repeat(np.arange(10), 50)
    again = oracle.sq_dist_pairs(x, y, ii, iN.ravel(), lib=lib)
    assert np.array_equal(again, dN.ravel())
    # x = y: the self-match is rank 0 at distance 0
    d0, i0 = oracle.kmin(y, y, 3, lib=lib)
    assert np.array_equal(i0[:, 0], np.arange(50)) and not d0[:, 0].any()


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
