"""GPU parity: the gfx950 kernels (through the C ABI) against the float64 oracle.

Small cases compare every output element and span several tiles, ragged
tails, both distance forms, forced j-splits and both row layouts.  The named
workloads run at full size in the launch configuration the library picks and
compare seeded samples of rows (each sampled row is exact: the oracle
evaluates it over all N).
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from parity import check_grad, check_kmin, check_lse, check_max, check_sum, dev, host

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import geometric_map_reduce_amd as gm
    from geometric_map_reduce_amd import workloads


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _options():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    for o in (gm.KEOPS_OPT_SPLIT_J, gm.KEOPS_OPT_FORM, gm.KEOPS_OPT_ROWS, gm.KEOPS_OPT_WG_TARGET, gm.KEOPS_OPT_MFMA):
        gm.keops_set_option(o, 0)
    yield
    for o in (gm.KEOPS_OPT_SPLIT_J, gm.KEOPS_OPT_FORM, gm.KEOPS_OPT_ROWS, gm.KEOPS_OPT_WG_TARGET, gm.KEOPS_OPT_MFMA):
        gm.keops_set_option(o, 0)


def rand_case(seed, M, N, D, E, scale=1.0):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((M, D)) * scale).astype(np.float32)
    y = (rng.standard_normal((N, D)) * scale).astype(np.float32)
    b = rng.standard_normal((N, E)).astype(np.float32)
    g = rng.standard_normal((M, E)).astype(np.float32)
    return x, y, b, g


# (M, N, D, E, sigma): tiles of 256 j, ragged tails, every compiled D group
SMALL = [
    (1, 1, 1, 1, 1.0), (2, 3, 3, 1, 0.7), (63, 65, 3, 1, 0.5), (64, 64, 2, 2, 1.0),
    (65, 257, 3, 1, 0.3), (255, 513, 5, 3, 1.5), (257, 1000, 8, 4, 2.0), (1000, 3001, 16, 1, 3.0),
    (300, 700, 4, 2, 0.8), (129, 600, 32, 1, 4.0), (70, 300, 50, 1, 5.0), (33, 250, 64, 2, 6.0),
    (20, 130, 100, 1, 8.0), (700, 1100, 6, 1, 1.2), (513, 2000, 7, 2, 0.9),
]


def _run_all(x, y, b, g, sigma):
    X, Y, B, G = dev(x), dev(y), dev(b), dev(g)
    a = gm.keops_gauss_sum(X, Y, B, sigma)
    l = gm.keops_gauss_lse(X, Y, B, sigma)
    gx = gm.keops_gauss_grad_x(X, Y, B, G, sigma)
    torch.cuda.synchronize()
    return host(a), host(l), host(gx)


def _check_all(x, y, b, g, sigma, res):
    a, l, gx = res
    a_ref, n_ref = oracle.gauss_sum(x, y, b, sigma)
    check_sum(a, a_ref, n_ref)
    check_lse(l, oracle.gauss_lse(x, y, b, sigma))
    G_ref, nu_ref = oracle.gauss_grad_x(x, y, b, g, sigma)
    check_grad(gx, G_ref, nu_ref)


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "M%d_N%d_D%d_E%d_s%g" % c)
def test_small_all_ops(case):
    M, N, D, E, sigma = case
    say(f"small case M={M} N={N} D={D} E={E} sigma={sigma}")
    x, y, b, g = rand_case(1000 + M + N + D, M, N, D, E)
    sigma = float(np.float32(sigma))
    _check_all(x, y, b, g, sigma, _run_all(x, y, b, g, sigma))


@pytest.mark.parametrize("form", [0, 1], ids=["auto", "direct"])
@pytest.mark.parametrize("split", [0, 1, 3, 7])
@pytest.mark.parametrize("rows", [1, 2], ids=["narrow", "wide"])
def test_forms_splits_layouts(form, split, rows):
    say(f"forced form={form} split={split} rows={rows}")
    # sigma = 0.4: one work-group beyond the expanded form's range (direct), one within
    for (M, N, D, E, sigma) in [(2100, 1900, 3, 1, 0.4), (600, 2500, 5, 2, 1.1), (3000, 700, 3, 1, 1.5)]:
        gm.keops_set_option(gm.KEOPS_OPT_FORM, form)
        gm.keops_set_option(gm.KEOPS_OPT_SPLIT_J, split)
        gm.keops_set_option(gm.KEOPS_OPT_ROWS, rows)
        x, y, b, g = rand_case(7 + D, M, N, D, E)
        _check_all(x, y, b, g, sigma, _run_all(x, y, b, g, sigma))


# few-rows layout (j per lane, rows in LDS): row groups of 16 with a ragged last
# group, steps of 1024 j with ragged tails, sigma = 0.05 puts the row group beyond
# the expanded form's range (direct-form fallback under the automatic form)
STREAM = [(1, 1, 3, 1, 1.0), (1, 5000, 3, 1, 0.3), (5, 1025, 1, 2, 0.7), (16, 3000, 3, 1, 0.1),
          (16, 3000, 3, 1, 0.05), (17, 4097, 8, 4, 1.5), (40, 10000, 5, 3, 0.9), (64, 2049, 2, 1, 2.0),
          (100, 3000, 3, 1, 0.5), (33, 70000, 4, 1, 0.2)]


@pytest.mark.parametrize("form", [0, 1], ids=["auto", "direct"])
@pytest.mark.parametrize("case", STREAM, ids=lambda c: "M%d_N%d_D%d_E%d_s%g" % c)
def test_stream_layout(case, form):
    M, N, D, E, sigma = case
    say(f"stream layout M={M} N={N} D={D} E={E} sigma={sigma} form={form}")
    x, y, b, _ = rand_case(300 + M + D, M, N, D, E)
    sigma = float(np.float32(sigma))
    a_ref, n_ref = oracle.gauss_sum(x, y, b, sigma)
    X, Y, B = dev(x), dev(y), dev(b)
    gm.keops_set_option(gm.KEOPS_OPT_ROWS, 3)
    gm.keops_set_option(gm.KEOPS_OPT_FORM, form)
    for target in (0, 1, 64):                 # one long j range per work-group, the default, many short
        gm.keops_set_option(gm.KEOPS_OPT_WG_TARGET, target)
        a = gm.keops_gauss_sum(X, Y, B, sigma)
        torch.cuda.synchronize()
        check_sum(host(a), a_ref, n_ref)


@pytest.mark.parametrize("form", [0, 1], ids=["auto", "direct"])
@pytest.mark.parametrize("case", STREAM, ids=lambda c: "M%d_N%d_D%d_E%d_s%g" % c)
def test_stream_layout_lse_grad(case, form):
    """LogSumExp and grad_x in the few-rows layout (online LogSumExp per lane; the
    gradient in the direct form) against the oracle, every row, for one long j range
    per work-group, the default, and many short ones."""
    M, N, D, E, sigma = case
    say(f"stream lse/grad M={M} N={N} D={D} E={E} sigma={sigma} form={form}")
    x, y, b, g = rand_case(400 + M + D, M, N, D, E)
    sigma = float(np.float32(sigma))
    l_ref = oracle.gauss_lse(x, y, b, sigma)
    G_ref, nu = oracle.gauss_grad_x(x, y, b, g, sigma)
    X, Y, B, Gt = dev(x), dev(y), dev(b), dev(g)
    gm.keops_set_option(gm.KEOPS_OPT_ROWS, 3)
    gm.keops_set_option(gm.KEOPS_OPT_FORM, form)
    for target in (0, 1, 64):
        gm.keops_set_option(gm.KEOPS_OPT_WG_TARGET, target)
        check_lse(host(gm.keops_gauss_lse(X, Y, B, sigma)), l_ref)
        check_grad(host(gm.keops_gauss_grad_x(X, Y, B, Gt, sigma)), G_ref, nu)


def _random_stream_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        cases.append((int(rng.integers(1, 65)), int(rng.integers(1, 40000)), int(rng.integers(1, 9)),
                      int(rng.integers(1, 5)), float(rng.choice([0.05, 0.1, 0.3, 1.0, 2.0])),
                      int(rng.choice([0, 1, 3, 7, 64])), int(rng.integers(0, 2))))
    return cases


@pytest.mark.parametrize("case", _random_stream_cases(24, 2024), ids=lambda c: "M%d_N%d_D%d_E%d_s%g_t%d_f%d" % c)
def test_stream_random_shapes(case):
    """Seeded random few-rows shapes (M up to 64, N up to 4e4, D 1-8, E 1-4, work-group
    targets from one chunk to many, both forms): sum, LogSumExp and grad_x against the
    oracle, every row.  Covers row-group counts and chunk counts that are not multiples
    of 8 in the XCD placement of the grid."""
    M, N, D, E, sigma, target, form = case
    say(f"stream random M={M} N={N} D={D} E={E} sigma={sigma} target={target} form={form}")
    sigma = float(np.float32(sigma))
    x, y, b, g = rand_case(500 + M + N, M, N, D, E)
    gm.keops_set_option(gm.KEOPS_OPT_WG_TARGET, target)
    gm.keops_set_option(gm.KEOPS_OPT_FORM, form)
    X, Y, B, Gt = dev(x), dev(y), dev(b), dev(g)
    a_ref, n_ref = oracle.gauss_sum(x, y, b, sigma)
    check_sum(host(gm.keops_gauss_sum(X, Y, B, sigma)), a_ref, n_ref)
    check_lse(host(gm.keops_gauss_lse(X, Y, B, sigma)), oracle.gauss_lse(x, y, b, sigma))
    G_ref, nu = oracle.gauss_grad_x(x, y, b, g, sigma)
    check_grad(host(gm.keops_gauss_grad_x(X, Y, B, Gt, sigma)), G_ref, nu)


@pytest.mark.parametrize("M", [1, 16, 40, 64])
def test_workload_few_rows_lse_grad_1M(M):
    """M in {1, 16, 40, 64} rows against N = 1e6 points (x, y ~ U[0,1)^3, b ~ N(0,1),
    sigma = 0.1): the sum, LogSumExp and grad_x, chosen automatically in the few-rows
    layout (up to four row groups sharing each chunk of j), every row against the
    oracle."""
    say(f"few rows sum/lse/grad M={M} N=1e6")
    x, y, b = workloads.make_points("uniform", M, 1_000_000, 3, 1, seed=20 + M)
    g = np.random.default_rng(M).standard_normal((M, 1)).astype(np.float32)
    X, Y, B, Gt = dev(x), dev(y), dev(b), dev(g)
    a_ref, n_ref = oracle.gauss_sum(x, y, b, 0.1)
    check_sum(host(gm.keops_gauss_sum(X, Y, B, 0.1)), a_ref, n_ref)
    check_lse(host(gm.keops_gauss_lse(X, Y, B, 0.1)), oracle.gauss_lse(x, y, b, 0.1))
    G_ref, nu = oracle.gauss_grad_x(x, y, b, g, 0.1)
    check_grad(host(gm.keops_gauss_grad_x(X, Y, B, Gt, 0.1)), G_ref, nu)


@pytest.mark.parametrize("M", [1, 16, 40])
def test_stream_far_rows_lse_grad(M):
    """Few-rows LogSumExp and grad_x with rows spread over 18 sigma and every y at one
    end: the far rows' terms are far below 2^-126, which the running maximum of the
    LogSumExp absorbs."""
    say(f"stream far rows lse/grad M={M}")
    x, y, b = _far_rows_case(491 + M, 1)
    x = x[np.argsort(x[:, 0])][np.linspace(0, x.shape[0] - 1, M).astype(int)]
    g = np.random.default_rng(M).standard_normal((M, 1)).astype(np.float32)
    gm.keops_set_option(gm.KEOPS_OPT_ROWS, 3)
    check_lse(host(gm.keops_gauss_lse(dev(x), dev(y), dev(b), 1.0)), oracle.gauss_lse(x, y, b, 1.0))
    G_ref, nu = oracle.gauss_grad_x(x, y, b, g, 1.0)
    check_grad(host(gm.keops_gauss_grad_x(dev(x), dev(y), dev(b), dev(g), 1.0)), G_ref, nu)


def test_far_from_origin_and_spread():
    """Data far from the origin (centring) and spread out (direct-form fallback)."""
    say("far/spread")
    rng = np.random.default_rng(5)
    for shift, scale, sigma in [(1000.0, 1.0, 0.5), (0.0, 30.0, 0.5), (-50.0, 5.0, 0.05)]:
        x = (rng.standard_normal((900, 3)) * scale + shift).astype(np.float32)
        y = np.concatenate([x[::3] + np.float32(0.01) * rng.standard_normal((300, 3)).astype(np.float32),
                            (rng.standard_normal((700, 3)) * scale + shift).astype(np.float32)])
        b = rng.standard_normal((y.shape[0], 1)).astype(np.float32)
        g = rng.standard_normal((900, 1)).astype(np.float32)
        _check_all(x, y, b, g, sigma, _run_all(x, y, b, g, sigma))


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "M%d_N%d_D%d_E%d_s%g" % c)
def test_small_transposed_grads(case):
    """grad_y and grad_b (reductions over i, one output per point y_j) on every small shape."""
    M, N, D, E, sigma = case
    say(f"transposed grads M={M} N={N} D={D} E={E} sigma={sigma}")
    x, y, b, g = rand_case(2000 + M + N + D, M, N, D, E)
    sigma = float(np.float32(sigma))
    X, Y, B, G = dev(x), dev(y), dev(b), dev(g)
    gy = gm.keops_gauss_grad_y(X, Y, B, G, sigma)
    gb = gm.keops_gauss_grad_b(X, Y, G, sigma)
    torch.cuda.synchronize()
    Gy_ref, nuy = oracle.gauss_grad_y(x, y, b, g, sigma)
    check_grad(host(gy), Gy_ref, nuy)
    Gb_ref, nub = oracle.gauss_grad_b(x, y, g, sigma)
    check_sum(host(gb), Gb_ref, nub, what="grad_b")


def test_transposed_grads_degenerate_and_balance():
    say("transposed grads: M = 0, N = 0, translation balance")
    x, y, b, g = rand_case(77, 0, 50, 3, 2)
    gy = gm.keops_gauss_grad_y(dev(np.zeros((0, 3), np.float32)), dev(y), dev(b), dev(np.zeros((0, 2), np.float32)), 1.0)
    gb = gm.keops_gauss_grad_b(dev(np.zeros((0, 3), np.float32)), dev(y), dev(np.zeros((0, 2), np.float32)), 1.0)
    torch.cuda.synchronize()
    assert not host(gy).any() and not host(gb).any() and gy.shape == (50, 3) and gb.shape == (50, 2)
    x, y, b, g = rand_case(78, 300, 500, 3, 1)
    X, Y, B, G = dev(x), dev(y), dev(b), dev(g)
    gx = host(gm.keops_gauss_grad_x(X, Y, B, G, 0.8)).astype(np.float64)
    gy = host(gm.keops_gauss_grad_y(X, Y, B, G, 0.8)).astype(np.float64)
    _, nux = oracle.gauss_grad_x(x, y, b, g, 0.8)
    _, nuy = oracle.gauss_grad_y(x, y, b, g, 0.8)
    # moving every point together leaves L unchanged: the two gradients balance
    assert np.all(np.abs(gx.sum(0) + gy.sum(0)) <= 1e-4 * (nux.sum(0) + nuy.sum(0)))


def _check_cg(x, b, sigma, lam, a, iters, rel, rtol, max_iter):
    """A conjugate-gradient solution against the dense float64 solve a*: the true residual
    (double, through the sum oracle) is within the stopping rule's reach, the reported
    residual agrees with it, and |a - a*| <= |r| / lam (K is positive semi-definite, so the
    smallest eigenvalue of K + lam I is at least lam)."""
    a = np.asarray(a, np.float64)
    a_star = oracle.gauss_solve(x, b, sigma, lam)
    r = oracle.gauss_system_residual(x, b, a.astype(np.float32), sigma, lam)
    nb = np.linalg.norm(b.astype(np.float64), axis=0)
    nr = np.linalg.norm(r, axis=0)
    rel_true = np.where(nb > 0, nr / np.maximum(nb, 1e-300), 0.0)
    assert iters <= max_iter
    assert np.all(np.abs(rel - rel_true) <= 1e-5 + 1e-2 * rel_true), (rel, rel_true)
    if iters < max_iter:
        assert np.all(rel_true <= 2 * rtol + 1e-5), (rel_true, rtol)
    err = np.linalg.norm(a - a_star, axis=0)
    assert np.all(err <= nr / lam * (1 + 1e-3) + 1e-6 * np.linalg.norm(a_star, axis=0)), (err, nr / lam)
    return rel_true


# (N, D, E, sigma, lambda, rtol)
CG_CASES = [(1, 3, 1, 1.0, 0.5, 1e-6), (50, 2, 1, 0.5, 0.1, 1e-6), (777, 3, 3, 0.3, 1.0, 1e-5),
            (3000, 3, 1, 0.1, 1.0, 1e-5), (2500, 5, 2, 1.0, 10.0, 1e-5), (1500, 64, 1, 8.0, 0.5, 1e-5)]


@pytest.mark.parametrize("case", CG_CASES, ids=lambda c: "N%d_D%d_E%d_s%g_l%g" % c[:5])
def test_cg_against_dense_solve(case):
    N, D, E, sigma, lam, rtol = case
    say(f"cg N={N} D={D} E={E} sigma={sigma} lambda={lam}")
    rng = np.random.default_rng(900 + N + D)
    x = rng.random((N, D)).astype(np.float32)
    b = rng.standard_normal((N, E)).astype(np.float32)
    sigma = float(np.float32(sigma))
    a, iters, rel = gm.keops_gauss_cg(dev(x), dev(b), sigma, lam, rtol=rtol, max_iter=2000)
    a2, iters2, rel2 = gm.keops_gauss_cg(dev(x), dev(b), sigma, lam, rtol=rtol, max_iter=2000)
    a, a2 = host(a), host(a2)
    assert iters == iters2 and np.array_equal(a, a2) and np.array_equal(rel, rel2)   # reproducible
    rel_true = _check_cg(x, b, sigma, lam, a, iters, rel, rtol, 2000)
    say(f"  iterations {iters}, relative residual {rel_true.max():.3g}")


def test_cg_edge_cases():
    say("cg edge cases: b = 0, max_iter = 0, one point, early stop")
    rng = np.random.default_rng(5)
    x = rng.random((200, 3)).astype(np.float32)
    b = np.zeros((200, 2), np.float32)
    a, iters, rel = gm.keops_gauss_cg(dev(x), dev(b), 0.2, 1.0)
    assert iters == 0 and not host(a).any() and not rel.any()
    b = rng.standard_normal((200, 2)).astype(np.float32)
    b[:, 1] = 0.0                                          # one zero column among others
    a, iters, rel = gm.keops_gauss_cg(dev(x), dev(b), 0.2, 1.0, rtol=1e-6)
    assert not host(a)[:, 1].any() and rel[1] == 0.0
    _check_cg(x, b, 0.2, 1.0, host(a), iters, rel, 1e-6, 1000)
    a, iters, rel = gm.keops_gauss_cg(dev(x), dev(b), 0.2, 1.0, max_iter=0)
    assert iters == 0 and not host(a).any()
    np.testing.assert_allclose(rel, [1.0, 0.0], rtol=1e-6)
    a, iters, rel = gm.keops_gauss_cg(dev(x), dev(b), 0.2, 1.0, max_iter=3)   # stops early: still bounded
    assert iters == 3
    _check_cg(x, b, 0.2, 1.0, host(a), iters, rel, 1e-6, 3)
    x1 = np.array([[0.3, -0.2, 0.5]], np.float32)
    b1 = np.array([[2.0, -1.0]], np.float32)
    a, iters, rel = gm.keops_gauss_cg(dev(x1), dev(b1), 1.0, 0.25)
    np.testing.assert_allclose(host(a), b1 / 1.25, rtol=1e-6)
    assert iters == 1


def _composed_reference(x, y, b, g, sigma, ri, si, rj, rows, op):
    """Oracle values of the block-sparse reduction at ``rows``: for each row range, the dense
    oracle over the concatenation of its j ranges (the definition restricted to kept pairs)."""
    M = x.shape[0]
    W = x.shape[1] if op == "grad" else b.shape[1]
    ref = np.zeros((len(rows), W))
    nu = np.zeros((len(rows), W))
    if op == "lse":
        ref[:] = -np.inf
    owner = np.full(M, -1)
    for c, (lo, hi) in enumerate(ri):
        owner[lo:hi] = c
    for c in range(len(ri)):
        sel = np.flatnonzero(owner[rows] == c)
        if not sel.size:
            continue
        J = np.concatenate([np.arange(a, e) for a, e in rj[(si[c - 1] if c else 0):si[c]]] + [np.zeros(0, np.int64)])
        if not J.size:
            continue
        r = rows[sel]
        if op == "sum":
            ref[sel], nu[sel] = oracle.gauss_sum(x, y[J], b[J], sigma, rows=r)
        elif op == "lse":
            ref[sel] = oracle.gauss_lse(x, y[J], b[J], sigma, rows=r)
        else:
            ref[sel], nu[sel] = oracle.gauss_grad_x(x, y[J], b[J], g, sigma, rows=r)
    return ref, nu


@pytest.mark.parametrize("form", [0, 1], ids=["auto", "direct"])
@pytest.mark.parametrize("split", [0, 1, 3])
@pytest.mark.parametrize("rows", [1, 2], ids=["narrow", "wide"])
def test_ranges_random(form, split, rows):
    """Random row ranges (with gaps) meeting random, possibly repeated, j ranges."""
    from oracle_pins import random_ranges
    say(f"ranges form={form} split={split} rows={rows}")
    for (M, N, D, E, sigma, nr) in [(700, 900, 3, 1, 0.6, 9), (3000, 2500, 3, 2, 0.4, 6), (257, 4100, 5, 1, 1.1, 4),
                                    (1, 1, 1, 1, 1.0, 1), (5000, 300, 2, 3, 0.8, 3)]:
        rng = np.random.default_rng(M + N + 17 * split)
        x, y, b, g = rand_case(M + N, M, N, D, E)
        ri, si, rj, _ = random_ranges(rng, M, N, nr, 4)
        X, Y, B, G = dev(x), dev(y), dev(b), dev(g)
        gm.keops_set_option(gm.KEOPS_OPT_FORM, form)
        gm.keops_set_option(gm.KEOPS_OPT_SPLIT_J, split)
        gm.keops_set_option(gm.KEOPS_OPT_ROWS, rows)
        a = host(gm.keops_gauss_sum_ranges(X, Y, B, sigma, ri, si, rj))
        l = host(gm.keops_gauss_lse_ranges(X, Y, B, sigma, ri, si, rj))
        gx = host(gm.keops_gauss_grad_x_ranges(X, Y, B, G, sigma, ri, si, rj))
        a_ref, n_ref = oracle.gauss_sum_ranges(x, y, b, sigma, ri, si, rj)
        check_sum(a, a_ref, n_ref, what="sum_ranges")
        check_lse(l, oracle.gauss_lse_ranges(x, y, b, sigma, ri, si, rj))
        G_ref, nu = _composed_reference(x, y, b, g, sigma, ri, si, rj, np.arange(M), "grad")
        check_grad(gx, G_ref, nu)


def test_ranges_cover_all_equals_dense():
    say("ranges covering every pair")
    x, y, b, g = rand_case(5, 2100, 1900, 3, 2)
    X, Y, B = dev(x), dev(y), dev(b)
    ri = np.array([[0, 700], [700, 2100]])
    si = np.array([2, 3])
    rj = np.array([[0, 1000], [1000, 1900], [0, 1900]])
    a = host(gm.keops_gauss_sum_ranges(X, Y, B, 0.5, ri, si, rj))
    a_ref, n_ref = oracle.gauss_sum(x, y, b, 0.5)
    check_sum(a, a_ref, n_ref)
    l = host(gm.keops_gauss_lse_ranges(X, Y, B, 0.5, ri, si, rj))
    check_lse(l, oracle.gauss_lse(x, y, b, 0.5))
    # no kept pair at all: 0 and -inf everywhere
    a0 = host(gm.keops_gauss_sum_ranges(X, Y, B, 0.5, ri, [0, 0], np.zeros((0, 2))))
    l0 = host(gm.keops_gauss_lse_ranges(X, Y, B, 0.5, ri, [0, 0], np.zeros((0, 2))))
    assert not a0.any() and np.isneginf(l0).all()


def _grid_ranges(x, y, voxel, sigma, eps):
    from geometric_map_reduce_amd import blocksparse as bs
    lx, ly = bs.grid_cluster(x, voxel), bs.grid_cluster(y, voxel)
    px, py = bs.sort_by_cluster(lx), bs.sort_by_cluster(ly)
    rx, cx, radx = bs.cluster_ranges_centroids(x[px], lx[px])
    ry, cy, rady = bs.cluster_ranges_centroids(y[py], ly[py])
    mask = bs.truncation_mask(cx, radx, cy, rady, bs.cutoff_for(sigma, eps))
    return px, py, bs.ranges_from_mask(mask, rx, ry), mask


def test_ranges_grid_truncation_1M():
    """M = N = 1e6 (D = 3, sigma = 0.1, U[0,1)^3) sorted into voxels of 0.1 with the eps = 1e-5
    truncation mask: sampled rows against the oracle over their kept pairs, and the truncation
    error against the dense oracle within eps * sum_j |b_j|."""
    w = workloads.WORKLOADS["sum_lse_1M"]
    say("block-sparse sum_lse_1M, voxel 0.1, eps 1e-5")
    x, y, b = workloads.make_inputs(w)
    px, py, (ri, si, rj), mask = _grid_ranges(x, y, 0.1, w.sigma, 1e-5)
    xs, ys, bs_ = x[px], y[py], b[py]
    X, Y, B = dev(xs), dev(ys), dev(bs_)
    a = host(gm.keops_gauss_sum_ranges(X, Y, B, w.sigma, ri, si, rj))
    l = host(gm.keops_gauss_lse_ranges(X, Y, B, w.sigma, ri, si, rj))
    rows = _sample(w.M, 256)
    a_ref, n_ref = _composed_reference(xs, ys, bs_, None, w.sigma, ri, si, rj, rows, "sum")
    check_sum(a[rows], a_ref, n_ref, what="sum_ranges")
    l_ref, _ = _composed_reference(xs, ys, bs_, None, w.sigma, ri, si, rj, rows, "lse")
    check_lse(l[rows], l_ref)
    full, _ = oracle.gauss_sum(xs, ys, bs_, w.sigma, rows=rows)
    bound = 1e-5 * np.abs(b.astype(np.float64)).sum() + 1e-4 * n_ref
    assert np.all(np.abs(a[rows] - full) <= bound)
    say(f"  kept cluster pairs {mask.mean():.3f}; worst truncation error {np.abs(a[rows] - full).max():.3g}")


def _run_max(x, y, b, sigma, rows=None):
    X, Y, B = dev(x), dev(y), dev(b)
    out = []
    for sign, fn in ((1, gm.keops_gauss_max), (-1, gm.keops_gauss_min)):
        v, i = fn(X, Y, B, sigma)
        torch.cuda.synchronize()
        v, i = host(v), host(i)
        r = np.arange(x.shape[0]) if rows is None else rows
        v_ref, i_ref = oracle.gauss_max(x, y, b, sigma, sign, rows=None if rows is None else rows)
        out.append(check_max(x, y, b, sigma, sign, r, v[r], i[r], v_ref, i_ref))
    return out


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "M%d_N%d_D%d_E%d_s%g" % c)
def test_small_max_min(case):
    M, N, D, E, sigma = case
    say(f"max/min M={M} N={N} D={D} E={E} sigma={sigma}")
    x, y, b, _ = rand_case(4000 + M + N + D, M, N, D, E)
    if N >= 4:
        y[N - 1], b[N - 1] = y[1], b[1]          # an exact tie: the smaller index
    _run_max(x, y, b, float(np.float32(sigma)))


@pytest.mark.parametrize("form", [0, 1], ids=["auto", "direct"])
@pytest.mark.parametrize("split", [0, 1, 5])
@pytest.mark.parametrize("rows", [1, 2], ids=["narrow", "wide"])
def test_max_forms_splits_layouts(form, split, rows):
    say(f"max forced form={form} split={split} rows={rows}")
    for (M, N, D, E, sigma) in [(2100, 1900, 3, 1, 0.4), (600, 2500, 5, 2, 1.1)]:
        gm.keops_set_option(gm.KEOPS_OPT_FORM, form)
        gm.keops_set_option(gm.KEOPS_OPT_SPLIT_J, split)
        gm.keops_set_option(gm.KEOPS_OPT_ROWS, rows)
        x, y, b, _ = rand_case(11 + D, M, N, D, E)
        _run_max(x, y, b, sigma)


def test_max_empty_and_far():
    say("max/min: N = 0, far data, all-negative payload")
    x = np.zeros((5, 3), np.float32)
    v, i = gm.keops_gauss_max(dev(x), dev(np.zeros((0, 3), np.float32)), dev(np.zeros((0, 2), np.float32)), 1.0)
    w, k = gm.keops_gauss_min(dev(x), dev(np.zeros((0, 3), np.float32)), dev(np.zeros((0, 2), np.float32)), 1.0)
    v, i, w, k = host(v), host(i), host(w), host(k)
    assert np.isneginf(v).all() and np.isposinf(w).all() and (i == -1).all() and (k == -1).all()
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((700, 3)) * 5 + 300).astype(np.float32)
    y = (rng.standard_normal((900, 3)) * 5 + 300).astype(np.float32)
    b = -np.abs(rng.standard_normal((900, 1))).astype(np.float32)
    _run_max(x, y, b, 0.7)


def test_workload_max_1M():
    w = workloads.WORKLOADS["sum_lse_1M"]
    say("workload sum_lse_1M: max/min")
    x, y, b = workloads.make_inputs(w)
    n = _run_max(x, y, b, w.sigma, rows=_sample(w.M, 256))
    say(f"  indices differing from the oracle's (near ties): {n}")


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "M%d_N%d_D%d_E%d_s%g" % c)
def test_small_laplace(case):
    M, N, D, E, sigma = case
    say(f"laplace M={M} N={N} D={D} E={E} sigma={sigma}")
    x, y, b, _ = rand_case(5000 + M + N + D, M, N, D, E)
    sigma = float(np.float32(sigma))
    a = host(gm.keops_laplace_sum(dev(x), dev(y), dev(b), sigma))
    a_ref, n_ref = oracle.laplace_sum(x, y, b, sigma)
    check_sum(a, a_ref, n_ref, what="laplace")


@pytest.mark.parametrize("split", [0, 1, 4])
@pytest.mark.parametrize("rows", [1, 2], ids=["narrow", "wide"])
def test_laplace_splits_layouts_far(split, rows):
    say(f"laplace split={split} rows={rows}")
    gm.keops_set_option(gm.KEOPS_OPT_SPLIT_J, split)
    gm.keops_set_option(gm.KEOPS_OPT_ROWS, rows)
    rng = np.random.default_rng(31 + split)
    for shift, scale, sigma in [(0.0, 1.0, 0.3), (500.0, 3.0, 0.8), (0.0, 20.0, 2.0)]:
        x = (rng.standard_normal((1500, 3)) * scale + shift).astype(np.float32)
        y = np.concatenate([x[::2] + np.float32(1e-3) * rng.standard_normal((750, 3)).astype(np.float32),
                            (rng.standard_normal((900, 3)) * scale + shift).astype(np.float32)])
        b = rng.standard_normal((y.shape[0], 2)).astype(np.float32)
        a = host(gm.keops_laplace_sum(dev(x), dev(y), dev(b), sigma))
        a_ref, n_ref = oracle.laplace_sum(x, y, b, sigma)
        check_sum(a, a_ref, n_ref, what="laplace")


def test_workload_laplace_1M():
    w = workloads.WORKLOADS["sum_lse_1M"]
    say("workload sum_lse_1M: Laplacian sum")
    x, y, b = workloads.make_inputs(w)
    a = host(gm.keops_laplace_sum(dev(x), dev(y), dev(b), w.sigma))
    rows = _sample(w.M, 256)
    a_ref, n_ref = oracle.laplace_sum(x, y, b, w.sigma, rows=rows)
    say(f"  max err / norm {check_sum(a[rows], a_ref, n_ref, what='laplace'):.3g}")


KMIN_SMALL = [(1, 1, 1, 1), (5, 40, 3, 10), (300, 1000, 3, 10), (257, 513, 2, 16), (100, 3000, 4, 32),
              (70, 600, 8, 7), (64, 300, 16, 5), (40, 500, 32, 10), (30, 200, 50, 3), (25, 300, 64, 10),
              (10, 128, 100, 2), (200, 900, 5, 1), (129, 129, 3, 12),
              # matrix-core prefilter shapes: several twelve-wave work-groups with ragged rows
              # and j, eight waves of three tiles, K = N, N below one 16-j step, D = 100 at K = 1
              (800, 1000, 64, 4), (500, 777, 50, 12), (20, 16, 64, 16), (33, 7, 32, 7), (400, 300, 100, 1)]


@pytest.mark.parametrize("case", KMIN_SMALL, ids=lambda c: "M%d_N%d_D%d_K%d" % c)
def test_kmin_small(case):
    M, N, D, K = case
    say(f"kmin M={M} N={N} D={D} K={K}")
    rng = np.random.default_rng(M * 7 + N + D)
    x = rng.standard_normal((M, D)).astype(np.float32)
    y = rng.standard_normal((N, D)).astype(np.float32)
    if N > 4:
        y[N - 1] = y[0]                       # an exact distance tie: smaller index first
    for split in (0, 3):
        gm.keops_set_option(gm.KEOPS_OPT_SPLIT_J, split)
        d, i = gm.keops_kmin(dev(x), dev(y), K)
        torch.cuda.synchronize()
        d_ref, i_ref = oracle.kmin(x, y, K)
        check_kmin(x, y, np.arange(M), host(d), host(i), d_ref, i_ref)


@pytest.mark.parametrize("D", [3, 50])
def test_kmeans_assignment(D):
    """k-means assignment (the pages' argmin reduction): 200,000 points of a 16-component
    mixture against 64 centroids (a few j tiles, every row block of the grid), K = 1,
    on the VALU kernel (D = 3) and the matrix-core prefilter (D = 50); 4,096 sampled
    rows against the oracle, and every index a valid centroid."""
    say(f"k-means assignment M=200000 N=64 D={D}")
    x, _, _ = workloads.make_points("mixture16", 200_000, 1, D, 1, seed=70 + D)
    rng = np.random.default_rng(71 + D)
    cent = x[rng.choice(x.shape[0], 64, replace=False)] + np.float32(0.01) * rng.standard_normal((64, D)).astype(np.float32)
    cent = np.ascontiguousarray(cent, dtype=np.float32)
    d, i = gm.keops_kmin(dev(x), dev(cent), 1)
    torch.cuda.synchronize()
    d, i = host(d), host(i)
    assert ((i >= 0) & (i < 64)).all()
    rows = _sample(x.shape[0], 4096)
    d_ref, i_ref = oracle.kmin(x[rows], cent, 1)
    check_kmin(x, cent, rows, d[rows], i[rows], d_ref, i_ref)


def test_kmin_self_and_permutation():
    say("kmin self-match and K = N")
    rng = np.random.default_rng(9)
    y = rng.standard_normal((16, 3)).astype(np.float32)
    d, i = gm.keops_kmin(dev(y), dev(y), 16)
    torch.cuda.synchronize()
    d, i = host(d), host(i)
    assert (i[:, 0] == np.arange(16)).all() and (d[:, 0] == 0).all()
    assert all(sorted(r) == list(range(16)) for r in i.tolist())


# few-rows K-min (lanes own j): (M, N, D, K), rows from one to a full 64, ragged row
# groups and chunks, K = 32 (two rows per group), N below one step and K = N
KMIN_FEW = [(1, 5000, 3, 10), (3, 1000, 1, 1), (16, 20037, 3, 10), (40, 7777, 8, 16), (64, 3000, 2, 32),
            (17, 300, 5, 7), (5, 10, 3, 10), (6, 2049, 4, 15), (64, 70000, 7, 2)]


@pytest.mark.parametrize("split", [0, 1, 5, 16])
@pytest.mark.parametrize("case", KMIN_FEW, ids=lambda c: "M%d_N%d_D%d_K%d" % c)
def test_kmin_few_rows(case, split):
    """The few-rows K-min equals the row-per-lane kernel bit for bit (both insert the same
    direct-form fp32 distances by (d^2, j)) and matches the oracle."""
    M, N, D, K = case
    say(f"kmin few rows M={M} N={N} D={D} K={K} split={split}")
    rng = np.random.default_rng(M * 13 + N + D * 7 + K)
    x = rng.standard_normal((M, D)).astype(np.float32)
    y = rng.standard_normal((N, D)).astype(np.float32)
    if N > 4:
        y[N - 1] = y[1]                       # an exact tie across the j range
    X, Y = dev(x), dev(y)
    gm.keops_set_option(gm.KEOPS_OPT_ROWS, 3)
    gm.keops_set_option(gm.KEOPS_OPT_SPLIT_J, split)
    d, i = gm.keops_kmin(X, Y, K)
    gm.keops_set_option(gm.KEOPS_OPT_ROWS, 1)
    gm.keops_set_option(gm.KEOPS_OPT_SPLIT_J, 0)
    d1, i1 = gm.keops_kmin(X, Y, K)
    d, i, d1, i1 = host(d), host(i), host(d1), host(i1)
    assert np.array_equal(i, i1) and np.array_equal(d.view(np.uint32), d1.view(np.uint32))
    d_ref, i_ref = oracle.kmin(x, y, K)
    check_kmin(x, y, np.arange(M), d, i, d_ref, i_ref)


@pytest.mark.parametrize("K", [1, 10, 32])
@pytest.mark.parametrize("split", [0, 3])
def test_kmin_few_rows_ties(K, split):
    """Integer coordinates on a 3^3 grid: distances are exact in fp32 and nearly every
    one is shared by hundreds of j, so each work-group's candidate set fills and the
    order among equal distances decides every slot.  The picks must be the oracle's
    exactly: ascending (d^2, j)."""
    say(f"kmin few rows ties K={K} split={split}")
    rng = np.random.default_rng(77 + K)
    M, N, D = 24, 40000, 3
    x = rng.integers(0, 3, (M, D)).astype(np.float32)
    y = rng.integers(0, 3, (N, D)).astype(np.float32)
    gm.keops_set_option(gm.KEOPS_OPT_ROWS, 3)
    gm.keops_set_option(gm.KEOPS_OPT_SPLIT_J, split)
    d, i = gm.keops_kmin(dev(x), dev(y), K)
    d, i = host(d), host(i)
    d_ref, i_ref = oracle.kmin(x, y, K)
    assert np.array_equal(i, i_ref)
    assert np.array_equal(d.astype(np.float64), d_ref)


@pytest.mark.parametrize("K", [1, 5])
def test_kmin_few_rows_nonfinite(K):
    """Non-finite coordinates: a NaN row and an infinite row get no neighbour (+inf, -1);
    y points with a NaN or an infinite coordinate are never picked; the few-rows and
    row-per-lane layouts agree bit for bit, and the finite rows match the oracle run on
    the finite points alone."""
    say(f"kmin few rows non-finite K={K}")
    rng = np.random.default_rng(808 + K)
    M, N, D = 6, 5000, 3
    x = rng.standard_normal((M, D)).astype(np.float32)
    y = rng.standard_normal((N, D)).astype(np.float32)
    x[2, 0] = np.nan
    x[4, 1] = np.inf
    bad = np.array([10, 20, 30, 4999])
    y[10, 1] = np.nan
    y[20, 0] = np.inf
    y[30, 2] = -np.inf
    y[4999] = np.nan
    X, Y = dev(x), dev(y)
    gm.keops_set_option(gm.KEOPS_OPT_ROWS, 3)
    d, i = gm.keops_kmin(X, Y, K)
    gm.keops_set_option(gm.KEOPS_OPT_ROWS, 1)
    d1, i1 = gm.keops_kmin(X, Y, K)
    d, i, d1, i1 = host(d), host(i), host(d1), host(i1)
    assert np.array_equal(i, i1) and np.array_equal(d.view(np.uint32), d1.view(np.uint32))
    for r in (2, 4):
        assert (i[r] == -1).all() and np.isinf(d[r]).all() and (d[r] > 0).all()
    good = np.setdiff1d(np.arange(N), bad)
    assert not np.isin(i, bad).any()
    rows = np.array([0, 1, 3, 5])
    d_ref, i_ref = oracle.kmin(x[rows], y[good], K)
    check_kmin(x[rows], y[good], np.arange(len(rows)), d[rows], np.searchsorted(good, i[rows]), d_ref, i_ref)


@pytest.mark.parametrize("rows", [0, 1], ids=["auto", "row_per_lane"])
@pytest.mark.parametrize("M,D", [(6, 3), (600, 3), (600, 64)])
def test_nonfinite_rows_leave_others_exact(M, D, rows):
    """A NaN row and a row with an infinite coordinate share their work-group (or row
    group) with finite rows: the finite rows' sum, LogSumExp, grad_x, Max and K-min
    must still match the oracle (work-group centres and range checks take finite
    coordinates only).  D = 64 runs the matrix-core kernels."""
    say(f"non-finite rows M={M} D={D} rows={rows}")
    rng = np.random.default_rng(909 + M + D)
    N, K = 3000, 4
    sigma = 0.7 * np.sqrt(D / 3.0)
    x = rng.standard_normal((M, D)).astype(np.float32)
    y = rng.standard_normal((N, D)).astype(np.float32)
    b = rng.standard_normal((N, 1)).astype(np.float32)
    g = rng.standard_normal((M, 1)).astype(np.float32)
    x[1, 0] = np.nan
    x[3, 2] = np.inf
    fin = np.setdiff1d(np.arange(M), [1, 3])
    X, Y, B, G = dev(x), dev(y), dev(b), dev(g)
    gm.keops_set_option(gm.KEOPS_OPT_ROWS, rows)
    a = host(gm.keops_gauss_sum(X, Y, B, sigma))
    a_ref, n_ref = oracle.gauss_sum(x[fin], y, b, sigma)
    check_sum(a[fin], a_ref, n_ref)
    l = host(gm.keops_gauss_lse(X, Y, B, sigma))
    check_lse(l[fin], oracle.gauss_lse(x[fin], y, b, sigma))
    gr = host(gm.keops_gauss_grad_x(X, Y, B, G, sigma))
    gr_ref, nu = oracle.gauss_grad_x(x[fin], y, b, g[fin], sigma)
    check_grad(gr[fin], gr_ref, nu)
    v, vi = gm.keops_gauss_max(X, Y, B, sigma)
    v_ref, vi_ref = oracle.gauss_max(x[fin], y, b, sigma, 1)
    check_max(x[fin], y, b, sigma, 1, np.arange(len(fin)), host(v)[fin], host(vi)[fin], v_ref, vi_ref)
    d, i = gm.keops_kmin(X, Y, K)
    d, i = host(d), host(i)
    d_ref, i_ref = oracle.kmin(x[fin], y, K)
    check_kmin(x[fin], y, np.arange(len(fin)), d[fin], i[fin], d_ref, i_ref)
    for r in (1, 3):
        assert (i[r] == -1).all() and np.isinf(d[r]).all()


@pytest.mark.parametrize("spike", [0.0, 12.0, 40.0])
def test_stream_lse_shift_and_cap(spike):
    """Few-rows LogSumExp's per-work-group shift comes from the first step's largest b:
    a b far above it later in the chunk (40) sends the work-group to the online pass,
    one within the cap (12) stays on the shifted pass; both must match the oracle."""
    say(f"stream lse shift cap spike={spike}")
    rng = np.random.default_rng(1401)
    M, N, D, sigma = 12, 300_000, 3, 0.1
    x = rng.uniform(0, 1, (M, D)).astype(np.float32)
    y = rng.uniform(0, 1, (N, D)).astype(np.float32)
    b = rng.standard_normal((N, 1)).astype(np.float32)
    if spike:
        b[rng.integers(N // 2, N, 40), 0] = spike
    gm.keops_set_option(gm.KEOPS_OPT_ROWS, 3)
    l = host(gm.keops_gauss_lse(dev(x), dev(y), dev(b), sigma))
    check_lse(l, oracle.gauss_lse(x, y, b, sigma))


@pytest.mark.parametrize("rows", [0, 1], ids=["auto", "row_per_lane"])
@pytest.mark.parametrize("M,D", [(6, 3), (600, 3), (600, 64)])
def test_lse_minus_inf_payloads(M, D, rows):
    """LogSumExp with log-weights b = -inf: those j drop out (the result equals the
    oracle over the other j), and where every b is -inf every row is -inf."""
    say(f"lse -inf payloads M={M} D={D} rows={rows}")
    rng = np.random.default_rng(1303 + M + D)
    N = 3000
    sigma = 0.7 * np.sqrt(D / 3.0)
    x = rng.standard_normal((M, D)).astype(np.float32)
    y = rng.standard_normal((N, D)).astype(np.float32)
    b = rng.standard_normal((N, 1)).astype(np.float32)
    drop = rng.random(N) < 0.3
    b[drop] = -np.inf
    gm.keops_set_option(gm.KEOPS_OPT_ROWS, rows)
    l = host(gm.keops_gauss_lse(dev(x), dev(y), dev(b), sigma))
    keep = ~drop
    check_lse(l, oracle.gauss_lse(x, y[keep], b[keep], sigma))
    b_all = np.full((N, 1), -np.inf, np.float32)
    l_all = host(gm.keops_gauss_lse(dev(x), dev(y), dev(b_all), sigma))
    assert np.all(l_all == -np.inf)


@pytest.mark.parametrize("K", [3, 10, 32])
def test_kmin_few_rows_many_chunks(K):
    """700 chunks: pass 2's threads each merge two or three partial lists, some of
    whose tails rank after the K entries already kept."""
    say(f"kmin few rows 700 chunks K={K}")
    rng = np.random.default_rng(330 + K)
    M, N, D = 5, 300_000, 3
    x = rng.standard_normal((M, D)).astype(np.float32)
    y = rng.standard_normal((N, D)).astype(np.float32)
    X, Y = dev(x), dev(y)
    gm.keops_set_option(gm.KEOPS_OPT_ROWS, 3)
    gm.keops_set_option(gm.KEOPS_OPT_SPLIT_J, 700)
    d, i = gm.keops_kmin(X, Y, K)
    gm.keops_set_option(gm.KEOPS_OPT_ROWS, 1)
    gm.keops_set_option(gm.KEOPS_OPT_SPLIT_J, 0)
    d1, i1 = gm.keops_kmin(X, Y, K)
    d, i, d1, i1 = host(d), host(i), host(d1), host(i1)
    assert np.array_equal(i, i1) and np.array_equal(d.view(np.uint32), d1.view(np.uint32))
    d_ref, i_ref = oracle.kmin(x, y, K)
    check_kmin(x, y, np.arange(M), d, i, d_ref, i_ref)


@pytest.mark.parametrize("M", [1, 16, 64])
def test_workload_kmin_few_rows_1M(M):
    """Few-rows K-min at N = 1e6 (D = 3, K = 10) in the launch configuration the library
    picks: every row against the oracle over all j."""
    say(f"kmin few rows M={M} N=1e6")
    rng = np.random.default_rng(600 + M)
    x = rng.standard_normal((M, 3)).astype(np.float32)
    y = rng.standard_normal((1_000_000, 3)).astype(np.float32)
    d, i = gm.keops_kmin(dev(x), dev(y), 10)
    d_ref, i_ref = oracle.kmin(x, y, 10)
    check_kmin(x, y, np.arange(M), host(d), host(i), d_ref, i_ref)


@pytest.mark.parametrize("E", [1, 2])
@pytest.mark.parametrize("rows", [1, 2], ids=["narrow", "wide"])
@pytest.mark.parametrize("split", [0, 1, 3])
def test_lse_fixed_shift_and_fixup(split, rows, E):
    """LogSumExp rows spread over 18 sigma, still inside one work-group's expanded-form
    range, with every y at one end: rows near the y take the fixed per-row shift; for the
    far ones every term underflows there, so they are flagged and recomputed by the fix-up
    launch with a running maximum."""
    say(f"lse fixed shift / fix-up split={split} rows={rows} E={E}")
    rng = np.random.default_rng(91 + E)
    M, N, sigma = 1500, 2000, 1.0
    x = np.zeros((M, 3), np.float32)
    x[:, 0] = rng.uniform(-9.0, 9.0, M)
    x[:, 1:] = 0.1 * rng.standard_normal((M, 2))
    y = np.zeros((N, 3), np.float32)
    y[:, 0] = -9.0 + 0.5 * rng.random(N)
    y[:, 1:] = 0.3 * rng.standard_normal((N, 2))
    b = rng.standard_normal((N, E)).astype(np.float32)
    gm.keops_set_option(gm.KEOPS_OPT_SPLIT_J, split)
    gm.keops_set_option(gm.KEOPS_OPT_ROWS, rows)
    l = host(gm.keops_gauss_lse(dev(x), dev(y), dev(b), sigma))
    l_ref = oracle.gauss_lse(x, y, b, sigma)
    assert l_ref.min() < -250.0 and l_ref.max() > -5.0      # both regimes present
    check_lse(l, l_ref)


def _far_rows_case(seed, E):
    """Rows spread over 18 sigma along x0, inside one work-group's expanded-form range,
    with every y at the x0 = -9 end: the far rows' values fall to 1e-30 and below."""
    rng = np.random.default_rng(seed)
    M, N = 1500, 2000
    x = np.zeros((M, 3), np.float32)
    x[:, 0] = rng.uniform(-9.0, 9.0, M)
    x[:, 1:] = 0.1 * rng.standard_normal((M, 2))
    y = np.zeros((N, 3), np.float32)
    y[:, 0] = -9.0 + 0.5 * rng.random(N)
    y[:, 1:] = 0.3 * rng.standard_normal((N, 2))
    b = rng.standard_normal((N, E)).astype(np.float32)
    return x, y, b


@pytest.mark.parametrize("E", [1, 2])
@pytest.mark.parametrize("rows", [1, 2], ids=["narrow", "wide"])
@pytest.mark.parametrize("split", [0, 1, 3])
def test_sum_far_rows(split, rows, E):
    """Sum rows 7-9 sigma from every y inside an expanded-form work-group: their terms lie
    below that form's floor, so they must come out of the direct form, not as 0."""
    say(f"sum far rows split={split} rows={rows} E={E}")
    x, y, b = _far_rows_case(191 + E, E)
    gm.keops_set_option(gm.KEOPS_OPT_SPLIT_J, split)
    gm.keops_set_option(gm.KEOPS_OPT_ROWS, rows)
    a = host(gm.keops_gauss_sum(dev(x), dev(y), dev(b), 1.0))
    a_ref, n_ref = oracle.gauss_sum(x, y, b, 1.0)
    assert ((n_ref > 1e-30) & (n_ref < 1e-20)).sum() > 20       # rows in the floor's range exist
    check_sum(a, a_ref, n_ref)


SIGN_PATTERNS = {"all_pos": 1, "all_neg": 2, "one_pos_per_tile": 3, "zeros_and_neg": 4}


@pytest.mark.parametrize("pattern", list(SIGN_PATTERNS))
@pytest.mark.parametrize("split", [0, 3])
def test_sign_classes_and_read_ahead(pattern, split):
    """Sum, LogSumExp and the Laplacian sum over payloads that leave one class of
    the sign-split tile empty, or one group long, in the 256-j tiles, over a
    ragged j range: the loops that read the next group's records ahead start,
    end and re-read the last group at every class boundary."""
    say(f"sign classes {pattern} split={split}")
    rng = np.random.default_rng(40 + SIGN_PATTERNS[pattern] * 7 + split)
    M, N = 700, 256 * 5 + 37
    x = rng.uniform(0, 1, (M, 3)).astype(np.float32)
    y = rng.uniform(0, 1, (N, 3)).astype(np.float32)
    mag = rng.uniform(0.5, 2.0, (N, 1))
    b = -mag
    if pattern == "all_pos":
        b = mag
    elif pattern == "one_pos_per_tile":
        b[::256] = mag[::256]
    elif pattern == "zeros_and_neg":
        b[rng.random(N) < 0.5] = 0.0
    b = b.astype(np.float32)
    sigma = 0.2
    gm.keops_set_option(gm.KEOPS_OPT_SPLIT_J, split)
    a = host(gm.keops_gauss_sum(dev(x), dev(y), dev(b), sigma))
    a_ref, n_ref = oracle.gauss_sum(x, y, b, sigma)
    check_sum(a, a_ref, n_ref)
    lap = host(gm.keops_laplace_sum(dev(x), dev(y), dev(b), sigma))
    lap_ref, lap_n = oracle.laplace_sum(x, y, b, sigma)
    check_sum(lap, lap_ref, lap_n, what="laplace")
    lse = host(gm.keops_gauss_lse(dev(x), dev(y), dev(b), sigma))
    check_lse(lse, oracle.gauss_lse(x, y, b, sigma))


@pytest.mark.parametrize("E", [1, 2])
@pytest.mark.parametrize("split", [0, 1, 3])
def test_grad_far_rows(split, E):
    """grad_x of rows 7-9 sigma from every y inside an expanded-form work-group."""
    say(f"grad_x far rows split={split} E={E}")
    x, y, b = _far_rows_case(291 + E, E)
    g = np.random.default_rng(5).standard_normal((x.shape[0], E)).astype(np.float32)
    gm.keops_set_option(gm.KEOPS_OPT_SPLIT_J, split)
    G = host(gm.keops_gauss_grad_x(dev(x), dev(y), dev(b), dev(g), 1.0))
    G_ref, nu = oracle.gauss_grad_x(x, y, b, g, 1.0)
    check_grad(G, G_ref, nu)


@pytest.mark.parametrize("split", [0, 1, 3])
def test_max_far_rows(split):
    """Max / ArgMax of rows 7-9 sigma from every y inside an expanded-form work-group."""
    say(f"max far rows split={split}")
    x, y, b = _far_rows_case(391, 1)
    gm.keops_set_option(gm.KEOPS_OPT_SPLIT_J, split)
    v, i = gm.keops_gauss_max(dev(x), dev(y), dev(b), 1.0)
    v_ref, i_ref = oracle.gauss_max(x, y, b, 1.0, 1)
    check_max(x, y, b, 1.0, 1, np.arange(x.shape[0]), host(v), host(i), v_ref, i_ref)


@pytest.mark.parametrize("M", [3, 16, 40])
def test_stream_far_rows(M):
    """Few-rows layout: rows spread over 18 sigma with every y at one end."""
    say(f"stream far rows M={M}")
    x, y, b = _far_rows_case(491 + M, 1)
    x = x[np.argsort(x[:, 0])][np.linspace(0, x.shape[0] - 1, M).astype(int)]
    gm.keops_set_option(gm.KEOPS_OPT_ROWS, 3)
    a = host(gm.keops_gauss_sum(dev(x), dev(y), dev(b), 1.0))
    a_ref, n_ref = oracle.gauss_sum(x, y, b, 1.0)
    check_sum(a, a_ref, n_ref)


def test_lse_large_payload():
    """b up to about 90: the bound G + (max b) log2 e rules the fixed shift out and the
    running maximum is used throughout."""
    say("lse large payload")
    x, y, b, _ = rand_case(5, 700, 900, 3, 2)
    b = (b * np.float32(30.0)).astype(np.float32)
    assert b.max() * np.log2(np.e) > 120
    for split in (0, 3):
        gm.keops_set_option(gm.KEOPS_OPT_SPLIT_J, split)
        check_lse(host(gm.keops_gauss_lse(dev(x), dev(y), dev(b), 0.8)), oracle.gauss_lse(x, y, b, 0.8))


def test_empty_and_degenerate():
    say("empty / degenerate sizes")
    x = dev(np.ones((5, 3), np.float32))
    y0 = torch.empty((0, 3), device="cuda")
    b0 = torch.empty((0, 2), device="cuda")
    assert (host(gm.keops_gauss_sum(x, y0, b0, 1.0)) == 0).all()
    assert np.isneginf(host(gm.keops_gauss_lse(x, y0, b0, 1.0))).all()
    g = dev(np.ones((5, 2), np.float32))
    assert (host(gm.keops_gauss_grad_x(x, y0, b0, g, 1.0)) == 0).all()
    x0 = torch.empty((0, 3), device="cuda")
    out = gm.keops_gauss_sum(x0, dev(np.ones((4, 3), np.float32)), dev(np.ones((4, 1), np.float32)), 1.0)
    assert out.shape == (0, 1)
    with pytest.raises(gm.KeopsError):
        gm.keops_kmin(x, dev(np.ones((3, 3), np.float32)), 4)         # K > N
    with pytest.raises(gm.KeopsError):
        gm.keops_gauss_sum(x, dev(np.ones((4, 3), np.float32)), dev(np.ones((4, 1), np.float32)), 0.0)
    with pytest.raises(gm.KeopsError):
        gm.keops_gauss_sum(dev(np.ones((5, 9), np.float32)), dev(np.ones((4, 9), np.float32)),
                           dev(np.ones((4, 1), np.float32)), 1.0)      # D = 9 not compiled


def test_single_point_identity():
    """M = N = 1, x = y: a = b (K = 1) and LSE = b."""
    say("single point")
    x = dev(np.float32([[0.3, -1.2, 2.5]]))
    b = dev(np.float32([[1.75]]))
    assert host(gm.keops_gauss_sum(x, x.clone(), b, 0.37))[0, 0] == np.float32(1.75)
    assert abs(host(gm.keops_gauss_lse(x, x.clone(), b, 0.37))[0, 0] - 1.75) <= 1e-6


def test_determinism_stream_and_out():
    """Bitwise-equal reruns; a non-default stream; caller-owned out and offset views."""
    say("determinism / stream / out")
    x, y, b, g = rand_case(3, 3000, 5000, 3, 1)
    X, Y, B = dev(x), dev(y), dev(b)
    a1 = host(gm.keops_gauss_sum(X, Y, B, 0.3))
    a2 = host(gm.keops_gauss_sum(X, Y, B, 0.3))
    assert np.array_equal(a1, a2)
    s = torch.cuda.Stream()
    out = torch.full((3000, 1), float("nan"), device="cuda")
    with torch.cuda.stream(s):
        gm.keops_gauss_sum(X, Y, B, 0.3, out=out)
    s.synchronize()
    assert np.array_equal(host(out), a1)
    # views whose data pointer is 4-byte but not 16-byte aligned
    Xv = torch.cat([torch.zeros(1, device="cuda"), X.ravel()])[1:].view(3000, 3)
    assert Xv.data_ptr() % 16 != 0
    a3 = host(gm.keops_gauss_sum(Xv, Y, B, 0.3))
    assert np.array_equal(a3, a1)


# ----------------------------------------------------------------------------- named workloads
def _sample(M, n):
    return workloads.sample_rows(M, n)


def test_workload_sum_1k():
    w = workloads.WORKLOADS["sum_1k"]
    say(f"workload {w.name}")
    x, y, b = workloads.make_inputs(w)
    a = host(gm.keops_gauss_sum(dev(x), dev(y), dev(b), w.sigma))
    a_ref, n_ref = oracle.gauss_sum(x, y, b, w.sigma)
    check_sum(a, a_ref, n_ref)


def test_workload_sum_grad_10k():
    w = workloads.WORKLOADS["sum_grad_10k"]
    say(f"workload {w.name}")
    x, y, b = workloads.make_inputs(w)
    X, Y, B = dev(x), dev(y), dev(b)
    a = gm.keops_gauss_sum(X, Y, B, w.sigma)
    a_ref, n_ref = oracle.gauss_sum(x, y, b, w.sigma)
    check_sum(host(a), a_ref, n_ref)
    # gated grad: both sides get the same fp32 cotangent g = 2 a_oracle
    g = (2.0 * a_ref).astype(np.float32)
    G = host(gm.keops_gauss_grad_x(X, Y, B, dev(g), w.sigma))
    G_ref, nu_ref = oracle.gauss_grad_x(x, y, b, g, w.sigma)
    check_grad(G, G_ref, nu_ref)
    # end-to-end chain g = 2 a_gpu (as autograd of (a**2).sum() would produce)
    G2 = host(gm.keops_gauss_grad_x(X, Y, B, 2.0 * a, w.sigma))
    G2_ref, nu2 = oracle.gauss_grad_x(x, y, b, (2.0 * host(a)).astype(np.float32), w.sigma)
    check_grad(G2, G2_ref, nu2)


@pytest.mark.parametrize("op", ["sum", "lse"])
def test_workload_sum_lse_1M(op):
    """M = N = 1e6, D = 3, sigma = 0.1: 4,096 seeded rows, each over all 1e6 j."""
    w = workloads.WORKLOADS["sum_lse_1M"]
    say(f"workload {w.name}: {op}")
    x, y, b = workloads.make_inputs(w)
    X, Y, B = dev(x), dev(y), dev(b)
    rows = _sample(w.M, 4096)
    if op == "sum":
        a = host(gm.keops_gauss_sum(X, Y, B, w.sigma))
        a_ref, n_ref = oracle.gauss_sum(x, y, b, w.sigma, rows=rows)
        err = check_sum(a[rows], a_ref, n_ref)
    else:
        l = host(gm.keops_gauss_lse(X, Y, B, w.sigma))
        err = check_lse(l[rows], oracle.gauss_lse(x, y, b, w.sigma, rows=rows))
    say(json.dumps({"workload": w.name, "op": op, "rows_checked": len(rows), "max_err": err}))


def test_workload_solver_matvec():
    w = workloads.WORKLOADS["solver_matvec_100k_x_10M"]
    say(f"workload {w.name}")
    x, y, b = workloads.make_inputs(w)
    X, Y, B = dev(x), dev(y), dev(b)
    a = host(gm.keops_gauss_sum(X, Y, B, w.sigma))
    del X, Y, B
    torch.cuda.empty_cache()
    rows = _sample(w.M, 512)
    a_ref, n_ref = oracle.gauss_sum(x, y, b, w.sigma, rows=rows)
    err = check_sum(a[rows], a_ref, n_ref)
    say(json.dumps({"workload": w.name, "rows_checked": len(rows), "sum_max_norm_err": err}))


def test_workload_stream_16_x_100M():
    """Few rows, 1e8 j: every row against the oracle, in the launch the library picks."""
    w = workloads.WORKLOADS["stream_16_x_100M"]
    say(f"workload {w.name}")
    x, y, b = workloads.make_inputs(w)
    a = gm.keops_gauss_sum(dev(x), dev(y), dev(b), w.sigma)
    torch.cuda.synchronize()
    a_ref, n_ref = oracle.gauss_sum(x, y, b, w.sigma)
    err = check_sum(host(a), a_ref, n_ref)
    say(f"  max err / norm {err:.3g}")


def test_workload_kmin10_16_x_100M():
    """Few-rows K-min at 1e8 j: every row against the oracle, in the launch the library picks."""
    w = workloads.WORKLOADS["kmin10_16_x_100M"]
    say(f"workload {w.name}")
    x, y, _ = workloads.make_inputs(w)
    d, i = gm.keops_kmin(dev(x), dev(y), w.K)
    d_ref, i_ref = oracle.kmin(x, y, w.K)
    nswap = check_kmin(x, y, np.arange(w.M), host(d), host(i), d_ref, i_ref)
    say(json.dumps({"workload": w.name, "rows_checked": w.M, "near_tie_swaps": nswap}))


def test_workload_transposed_grads_1M():
    """grad_y and grad_b at M = N = 1e6 (D = 3, sigma = 0.1), sampled points against the oracle."""
    w = workloads.WORKLOADS["sum_lse_1M"]
    say("workload sum_lse_1M: grad_y, grad_b")
    x, y, b = workloads.make_inputs(w)
    g = np.random.default_rng(3).standard_normal((w.M, w.E)).astype(np.float32)
    X, Y, B, G = dev(x), dev(y), dev(b), dev(g)
    gy = host(gm.keops_gauss_grad_y(X, Y, B, G, w.sigma))
    gb = host(gm.keops_gauss_grad_b(X, Y, G, w.sigma))
    cols = _sample(w.N, 192)
    Gy_ref, nuy = oracle.gauss_grad_y(x, y, b, g, w.sigma, cols=cols)
    Gb_ref, nub = oracle.gauss_grad_b(x, y, g, w.sigma, cols=cols)
    say(f"  grad_y max err/nu {check_grad(gy[cols], Gy_ref, nuy):.3g}; "
        f"grad_b {check_sum(gb[cols], Gb_ref, nub, what='grad_b'):.3g}")


def test_workload_krige_100k():
    """CG at N = 1e5: the oracle recomputes sampled rows of the true residual in double; their
    scaled root-mean-square matches the reported norm, which meets the stopping rule."""
    w = workloads.WORKLOADS["krige_100k"]
    say(f"workload {w.name}")
    x, _, b = workloads.make_inputs(w)
    rtol = 1e-4
    a, iters, rel = gm.keops_gauss_cg(dev(x), dev(b), w.sigma, w.lam, rtol=rtol, max_iter=1000)
    a = host(a)
    rows = _sample(w.N, 512)
    r = oracle.gauss_system_residual(x, b, a, w.sigma, w.lam, rows=rows)
    est = np.sqrt((r ** 2).mean() * w.N) / np.linalg.norm(b.astype(np.float64))
    say(f"  iterations {iters}, reported {rel[0]:.3g}, sampled estimate {est:.3g}")
    assert iters < 1000 and rel[0] <= 2 * rtol
    assert 0.5 * rel[0] - 1e-6 <= est <= 2.0 * rel[0] + 1e-6


@pytest.mark.parametrize("name", ["kmin10_1M_d3", "kmin10_1M_d64"])
def test_workload_kmin(name):
    """K-min at M = N = 1e6: 4,096 seeded rows at D = 3, 2,048 at D = 64, each over all 1e6 j."""
    w = workloads.WORKLOADS[name]
    say(f"workload {w.name}")
    x, y, _ = workloads.make_inputs(w)
    d, i = gm.keops_kmin(dev(x), dev(y), w.K)
    d, i = host(d), host(i)
    rows = _sample(w.M, 4096 if w.D <= 8 else 2048)
    d_ref, i_ref = oracle.kmin(x, y, w.K, rows=rows)
    nswap = check_kmin(x, y, rows, d[rows], i[rows], d_ref, i_ref)
    say(json.dumps({"workload": w.name, "rows_checked": len(rows), "near_tie_swaps": nswap}))


# ----------------------------------------------------------------------------- MFMA path
@pytest.mark.parametrize("D", [32, 50, 64, 100])
@pytest.mark.parametrize("E", [1, 3])
def test_mfma_vs_valu(D, E):
    """fp32-MFMA cross term (automatic at D >= 32), the VALU expanded form (matrix cores
    switched off) and the VALU direct form (forced) all match the oracle; the deviation
    between the MFMA and VALU paths is reported."""
    M, N, sigma = 700, 2300, 0.9 * np.sqrt(D / 3.0)
    say(f"mfma vs valu D={D} E={E}")
    x, y, b, _ = rand_case(50 + D + E, M, N, D, E, scale=1.0)
    X, Y, B = dev(x), dev(y), dev(b)
    a_ref, n_ref = oracle.gauss_sum(x, y, b, float(np.float32(sigma)))
    a_mfma = host(gm.keops_gauss_sum(X, Y, B, sigma))
    gm.keops_set_option(gm.KEOPS_OPT_MFMA, 1)
    a_vexp = host(gm.keops_gauss_sum(X, Y, B, sigma))
    gm.keops_set_option(gm.KEOPS_OPT_MFMA, 0)
    gm.keops_set_option(gm.KEOPS_OPT_FORM, 1)
    a_valu = host(gm.keops_gauss_sum(X, Y, B, sigma))
    e1 = check_sum(a_mfma, a_ref, n_ref, what="sum (mfma)")
    e2 = check_sum(a_valu, a_ref, n_ref, what="sum (valu direct)")
    e3 = check_sum(a_vexp, a_ref, n_ref, what="sum (valu expanded)")
    dev_paths = float(np.max(np.abs(a_mfma - a_valu) / np.maximum(n_ref, 1e-300)))
    say(json.dumps({"D": D, "E": E, "mfma_err": e1, "valu_err": e2, "valu_expanded_err": e3,
                    "mfma_vs_valu": dev_paths}))


@pytest.mark.parametrize("D", [32, 50, 64, 100])
@pytest.mark.parametrize("E", [1, 3])
@pytest.mark.parametrize("op", ["lse", "grad_x"])
def test_mfma_lse_grad_vs_valu(op, D, E):
    """LogSumExp and grad_x with the fp32-MFMA cross term (automatic at D >= 32; grad_x
    up to D = 64) and on the VALU (matrix cores switched off) both match the oracle."""
    M, N, sigma = 700, 2300, 0.9 * np.sqrt(D / 3.0)
    say(f"mfma {op} vs valu D={D} E={E}")
    x, y, b, g = rand_case(150 + D + E, M, N, D, E, scale=1.0)
    X, Y, B, G = dev(x), dev(y), dev(b), dev(g)
    s32 = float(np.float32(sigma))
    run = (lambda: gm.keops_gauss_lse(X, Y, B, sigma)) if op == "lse" else \
        (lambda: gm.keops_gauss_grad_x(X, Y, B, G, sigma))
    r_mfma = host(run())
    gm.keops_set_option(gm.KEOPS_OPT_MFMA, 1)
    r_valu = host(run())
    if op == "lse":
        ref = oracle.gauss_lse(x, y, b, s32)
        e1, e2 = check_lse(r_mfma, ref), check_lse(r_valu, ref)
    else:
        G_ref, nu = oracle.gauss_grad_x(x, y, b, g, s32)
        e1, e2 = check_grad(r_mfma, G_ref, nu), check_grad(r_valu, G_ref, nu)
    say(json.dumps({"op": op, "D": D, "E": E, "mfma_err": e1, "valu_err": e2}))


@pytest.mark.parametrize("split", [0, 1, 4])
@pytest.mark.parametrize("op", ["lse", "grad_x"])
def test_mfma_lse_grad_mixed_blocks(op, split):
    """One call where some work-groups stay on the matrix cores and others go to the
    direct-form VALU kernel: a row block spread beyond the expansion's range bound, and
    (LogSumExp) rows so far from every y that their terms flush to zero, which the
    work-group's underflow check hands over."""
    say(f"mfma {op} mixed blocks split={split}")
    rng = np.random.default_rng(78)
    D, E, sigma = 50, 2, 0.6
    x = (rng.standard_normal((700, D)) * 0.05).astype(np.float32)
    x[256:512] *= np.float32(40.0)                 # second row block: beyond the range bound
    x[600:610] += np.float32(1.2)                  # third block: ten rows far from every y
    y = np.concatenate([x[:600:2] + np.float32(0.01) * rng.standard_normal((300, D)).astype(np.float32),
                        (rng.standard_normal((900, D)) * 0.05).astype(np.float32)])
    b = rng.standard_normal((y.shape[0], E)).astype(np.float32)
    g = rng.standard_normal((x.shape[0], E)).astype(np.float32)
    gm.keops_set_option(gm.KEOPS_OPT_SPLIT_J, split)
    s32 = float(np.float32(sigma))
    if op == "lse":
        l = host(gm.keops_gauss_lse(dev(x), dev(y), dev(b), sigma))
        ref = oracle.gauss_lse(x, y, b, s32)
        assert np.all(ref[600:610] < -50.0)        # the far rows' terms are far below 2^-126
        check_lse(l, ref)
    else:
        G = host(gm.keops_gauss_grad_x(dev(x), dev(y), dev(b), dev(g), sigma))
        G_ref, nu = oracle.gauss_grad_x(x, y, b, g, s32)
        check_grad(G, G_ref, nu)


@pytest.mark.parametrize("split", [0, 1, 4])
def test_mfma_mixed_blocks(split):
    """Row blocks within the expansion's range run on MFMA, the others on the direct-form
    VALU kernel, in one call (256-row blocks: the second block is spread out)."""
    say(f"mfma mixed blocks split={split}")
    rng = np.random.default_rng(77)
    D, sigma = 50, 0.6
    x = (rng.standard_normal((700, D)) * 0.05).astype(np.float32)
    x[256:512] *= np.float32(40.0)                 # second row block: far beyond the range bound
    y = np.concatenate([x[::2] + np.float32(0.01) * rng.standard_normal((350, D)).astype(np.float32),
                        (rng.standard_normal((900, D)) * 0.05).astype(np.float32)])
    b = rng.standard_normal((y.shape[0], 2)).astype(np.float32)
    gm.keops_set_option(gm.KEOPS_OPT_SPLIT_J, split)
    a = host(gm.keops_gauss_sum(dev(x), dev(y), dev(b), sigma))
    a_ref, n_ref = oracle.gauss_sum(x, y, b, float(np.float32(sigma)))
    check_sum(a, a_ref, n_ref)


@pytest.mark.parametrize("D", [50, 64])
def test_kmin_mfma_unaligned_y(D):
    """y one float past a 16-byte boundary (the ABI asks for 4-byte alignment only): the
    split-bf16 K-min reads y with scalar loads then, and must still equal the VALU
    kernel bit for bit and match the oracle."""
    say(f"kmin mfma unaligned y D={D}")
    rng = np.random.default_rng(1500 + D)
    M, N, K = 500, 2000, 10
    x = rng.standard_normal((M, D)).astype(np.float32)
    y = rng.standard_normal((N, D)).astype(np.float32)
    buf = torch.empty(N * D + 4, dtype=torch.float32, device="cuda")
    Y = buf[1:1 + N * D].view(N, D)
    Y.copy_(torch.from_numpy(y))
    assert Y.data_ptr() % 16 == 4
    X = dev(x)
    d1, i1 = gm.keops_kmin(X, Y, K)
    gm.keops_set_option(gm.KEOPS_OPT_MFMA, 1)
    d2, i2 = gm.keops_kmin(X, Y, K)
    gm.keops_set_option(gm.KEOPS_OPT_MFMA, 0)
    d1, i1, d2, i2 = host(d1), host(i1), host(d2), host(i2)
    assert np.array_equal(i1, i2) and np.array_equal(d1.view(np.int32), d2.view(np.int32))
    d_ref, i_ref = oracle.kmin(x, y, K)
    check_kmin(x, y, np.arange(M), d1, i1, d_ref, i_ref)


@pytest.mark.parametrize("D,K,data", [(32, 10, "mix"), (50, 3, "mix"), (64, 10, "mix"), (64, 16, "mix"), (100, 1, "mix"),
                                       (100, 10, "mix"), (64, 1, "mix"), (64, 32, "mix"), (64, 10, "dups"),
                                       (100, 16, "dups"), (32, 13, "dups"), (64, 10, "far"), (50, 4, "far"),
                                       (100, 3, "mix"), (32, 32, "dups"), (100, 32, "mix"), (50, 32, "far")])
def test_kmin_mfma_equals_valu(D, K, data):
    """Both MFMA-prefiltered K-min forms (split bf16, the default, and fp32) and the
    VALU K-min return the direct-form fp32 K-min: identical indices and
    bitwise-identical distances; all match the oracle.
    "dups": y holds 100 points, each 30 times at scattered j, so every row's K
    smallest are exact ties, spread over the lane groups that share a threshold,
    and only the smallest j among the copies may be returned.  "far": the
    mixture moved 300 units off the origin in every coordinate."""
    say(f"kmin mfma == valu D={D} K={K} data={data}")
    rng = np.random.default_rng(D * 100 + K)
    centres = rng.uniform(-5, 5, (16, D))
    x = (centres[rng.integers(0, 16, 600)] + 0.5 * rng.standard_normal((600, D))).astype(np.float32)
    if data == "dups":
        base = (centres[rng.integers(0, 16, 100)] + 0.5 * rng.standard_normal((100, D))).astype(np.float32)
        y = base[rng.permutation(np.repeat(np.arange(100), 30))]
    else:
        y = (centres[rng.integers(0, 16, 3000)] + 0.5 * rng.standard_normal((3000, D))).astype(np.float32)
        y[2999] = y[5]                               # an exact tie
    if data == "far":
        x, y = x + np.float32(300.0), y + np.float32(300.0)
    X, Y = dev(x), dev(y)
    d1, i1 = gm.keops_kmin(X, Y, K)
    gm.keops_set_option(gm.KEOPS_OPT_MFMA, 2)        # fp32-MFMA prefilter
    d4, i4 = gm.keops_kmin(X, Y, K)
    gm.keops_set_option(gm.KEOPS_OPT_MFMA, 1)        # matrix cores off: the VALU kernel
    d3, i3 = gm.keops_kmin(X, Y, K)
    gm.keops_set_option(gm.KEOPS_OPT_MFMA, 0)
    gm.keops_set_option(gm.KEOPS_OPT_FORM, 1)        # forces the VALU kernel
    d2, i2 = gm.keops_kmin(X, Y, K)
    d1, i1, d2, i2, d3, i3 = host(d1), host(i1), host(d2), host(i2), host(d3), host(i3)
    d4, i4 = host(d4), host(i4)
    assert np.array_equal(i3, i2) and np.array_equal(d3.view(np.int32), d2.view(np.int32))
    assert np.array_equal(i4, i2) and np.array_equal(d4.view(np.int32), d2.view(np.int32))
    d_ref, i_ref = oracle.kmin(x, y, K)
    check_kmin(x, y, np.arange(600), d2, i2, d_ref, i_ref)   # VALU path
    check_kmin(x, y, np.arange(600), d1, i1, d_ref, i_ref)   # MFMA path
    assert np.array_equal(i1, i2)
    assert np.array_equal(d1.view(np.int32), d2.view(np.int32))
