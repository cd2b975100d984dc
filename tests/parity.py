"""Shared helpers of the GPU parity tests: device transfer and the acceptance checks.

Acceptance (fp32 GPU results against the float64 oracle):
  sum    |a - a*| <= 1e-4 * n        n = sum_j |K_ij b_j|        (per row and column)
  lse    |l - l*| <= 1e-4 + 2^-21 |l*|   (1e-4 absolute: every term is positive, so
                                      a relative 1e-4 on the sum is 1e-4 on its log;
                                      plus 8 fp32 ulps of the output itself, which an
                                      fp32 result of magnitude |l*| cannot beat)
  grad   |G - G*| <= 1e-4 * nu       nu = sum_j |(2/sigma^2) K <g,b> (x - y)|
  max    |max - max*| <= 2e-5 |max*| + 1e-37; an index other than the oracle's is
         accepted when its exact product is within that tolerance of the maximum
  kmin   indices distinct and in range; each pick equals the oracle's or its
         distance is within 1e-5 relative of the oracle's k-th distance (near
         ties); returned distances non-decreasing and within
         1e-4 * d + 1e-6 * (|x|^2 + |y|^2) of the exact distance of the pick.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

SUM_RTOL = 1e-4
LSE_ATOL = 1e-4
LSE_RTOL = 2.0 ** -21
GRAD_RTOL = 1e-4
KMIN_TIE_RTOL = 1e-5


def dev(a, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host(t):
    return t.detach().cpu().numpy()


def check_sum(a_gpu, a_ref, n_ref, rtol=SUM_RTOL, what="sum"):
    a_gpu = np.asarray(a_gpu, np.float64).reshape(a_ref.shape)
    err = np.abs(a_gpu - a_ref)
    bound = rtol * n_ref + 1e-37
    bad = ~(err <= bound)
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tol; worst ratio "
                           f"{np.nanmax(err / bound):.3g} at {np.argwhere(bad)[:3].tolist()}")
    return float(np.max(err / np.maximum(n_ref, 1e-300))) if err.size else 0.0


def check_lse(l_gpu, l_ref, atol=LSE_ATOL, rtol=LSE_RTOL):
    l_gpu = np.asarray(l_gpu, np.float64).reshape(l_ref.shape)
    both_inf = np.isneginf(l_gpu) & np.isneginf(l_ref)
    with np.errstate(invalid="ignore"):
        err = np.where(both_inf, 0.0, np.abs(l_gpu - l_ref))
    bad = ~(err <= atol + rtol * np.where(both_inf, 0.0, np.abs(l_ref)))
    assert not bad.any(), f"lse: {bad.sum()} outside tol; max err {np.nanmax(err):.3g}"
    return float(err.max()) if err.size else 0.0


def check_grad(G_gpu, G_ref, nu_ref, rtol=GRAD_RTOL):
    return check_sum(G_gpu, G_ref, nu_ref, rtol, what="grad_x")


MAX_RTOL = 2e-5


def check_max(x, y, b, sigma, sign, rows, v_gpu, i_gpu, v_ref, i_ref, rtol=MAX_RTOL):
    """Max/ArgMax (sign = +1) or Min/ArgMin (sign = -1) of K b against the oracle's signed maximum
    v_ref = max_j sign K_ij b_je with index i_ref: the value within rtol (plus a floor below the
    smallest normal fp32), and each index either the oracle's or one whose exact product is
    within the same tolerance of the maximum (near ties)."""
    s = sign * np.asarray(v_gpu, np.float64).reshape(v_ref.shape)
    i_gpu = np.asarray(i_gpu).reshape(i_ref.shape)
    tol = rtol * np.abs(v_ref) + 1e-37
    both_inf = np.isneginf(s) & np.isneginf(v_ref)
    with np.errstate(invalid="ignore"):
        err = np.where(both_inf, 0.0, np.abs(s - v_ref))
    assert np.all(err <= tol), f"max: worst {np.nanmax(err / tol):.3g} x tol"
    N = y.shape[0]
    diff = np.argwhere(i_gpu != i_ref)
    for r, e in diff:
        j = int(i_gpu[r, e])
        assert 0 <= j < N, (r, e, j)
        d2 = oracle.sq_dist_pairs(x, y, np.array([rows[r]]), np.array([j]))[0]
        exact = sign * np.exp(-d2 / float(sigma) ** 2) * float(b[j, e])
        assert abs(exact - v_ref[r, e]) <= tol[r, e], (r, e, j, exact, v_ref[r, e])
    return len(diff)


def check_kmin(x, y, rows, d_gpu, i_gpu, d_ref, i_ref):
    """Check GPU K-min picks of the given rows against the oracle's (d_ref, i_ref)."""
    d_gpu = np.asarray(d_gpu, np.float64)
    i_gpu = np.asarray(i_gpu, np.int64)
    n_rows, K = d_ref.shape
    N = y.shape[0]
    assert d_gpu.shape == (n_rows, K) and i_gpu.shape == (n_rows, K)
    assert (i_gpu >= 0).all() and (i_gpu < N).all(), "index out of range"
    s = np.sort(i_gpu, axis=1)
    assert (np.diff(s, axis=1) != 0).all(), "repeated index in a row"
    assert (np.diff(d_gpu, axis=1) >= 0).all(), "distances not ascending"
    ii = np.repeat(rows, K)
    exact = oracle.sq_dist_pairs(x, y, ii, i_gpu.ravel()).reshape(n_rows, K)
    # (2) each pick is the oracle's, or a near tie of the oracle's k-th distance
    same = i_gpu == i_ref
    tie = np.abs(exact - d_ref) <= KMIN_TIE_RTOL * d_ref
    bad = ~(same | tie)
    assert not bad.any(), (f"kmin: {bad.sum()} picks differ beyond near ties, first at "
                           f"{np.argwhere(bad)[:3].tolist()}")
    # (3) returned distances match the exact distance of the pick
    nx = (x[rows].astype(np.float64) ** 2).sum(1)[:, None]
    ny = (y[i_gpu.ravel()].astype(np.float64) ** 2).sum(1).reshape(n_rows, K)
    floor = 1e-4 * exact + 1e-6 * (nx + ny)
    assert (np.abs(d_gpu - exact) <= floor).all(), "returned distance off its pick's distance"
    return int((~same).sum())
