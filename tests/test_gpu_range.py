"""GPU range checks: payloads and cotangents far from 1, rows far from every point, and
block-sparse launches over far pairs, against the float64 oracle.

The expanded distance form shifts every exponent so that edge rows keep their terms in
range, and the direct form adds a fixed offset; both scale the fp32 accumulators by up to
2^64.  Each work-group checks its own rows after its j loop (underflow: results below the
floor's reach; overflow: non-finite results from finite inputs) and runs its j range once
more in the direct form with an offset sized from the payloads it saw.  These cases drive
each check in every layout: both forms, with and without j-splits, the few-rows layout and
block-sparse ranges.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from parity import check_grad, check_lse, check_max, check_sum, dev, host

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import geometric_map_reduce_amd as gm

OPTS = ("KEOPS_OPT_SPLIT_J", "KEOPS_OPT_FORM", "KEOPS_OPT_ROWS", "KEOPS_OPT_WG_TARGET", "KEOPS_OPT_MFMA")


@pytest.fixture(autouse=True)
def _options():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    for o in OPTS:
        gm.keops_set_option(getattr(gm, o), 0)
    yield
    for o in OPTS:
        gm.keops_set_option(getattr(gm, o), 0)


def say(msg):
    print(msg, flush=True)


def big_case(seed, M=700, N=1500, D=3, E=1, bscale=1e20):
    """x, y ~ N(0, 1) and b ~ N(0, 1) * bscale: true sums near 1e23, far inside fp32, while an
    accumulator scaled by 2^64 would reach 1e42."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, D)).astype(np.float32)
    y = rng.standard_normal((N, D)).astype(np.float32)
    b = (rng.standard_normal((N, E)) * bscale).astype(np.float32)
    return x, y, b


def far_rows(seed, E=1, M=1500, N=2000):
    """Rows spread over 18 sigma along x0 with every y at the x0 = -9 end (sigma = 1): the far
    rows' sums fall to 1e-30 and below, under the expanded form's floor."""
    rng = np.random.default_rng(seed)
    x = np.zeros((M, 3), np.float32)
    x[:, 0] = rng.uniform(-9.0, 9.0, M)
    x[:, 1:] = 0.1 * rng.standard_normal((M, 2))
    y = np.zeros((N, 3), np.float32)
    y[:, 0] = -9.0 + 0.5 * rng.random(N)
    y[:, 1:] = 0.3 * rng.standard_normal((N, 2))
    b = rng.standard_normal((N, E)).astype(np.float32)
    return x, y, b


@pytest.mark.parametrize("E", [1, 2])
@pytest.mark.parametrize("form", [0, 1])
@pytest.mark.parametrize("split", [0, 3])
def test_sum_grad_large_payload(split, form, E):
    """b ~ 1e20: sums near 1e23 must come out finite and within tolerance."""
    say(f"large payload sum/grad split={split} form={form} E={E}")
    x, y, b = big_case(11 + E, E=E)
    g = np.random.default_rng(12).standard_normal((x.shape[0], E)).astype(np.float32)
    gm.keops_set_option(gm.KEOPS_OPT_SPLIT_J, split)
    gm.keops_set_option(gm.KEOPS_OPT_FORM, form)
    a = host(gm.keops_gauss_sum(dev(x), dev(y), dev(b), 1.0))
    a_ref, n_ref = oracle.gauss_sum(x, y, b, 1.0)
    assert n_ref.max() > 1e22
    check_sum(a, a_ref, n_ref)
    G = host(gm.keops_gauss_grad_x(dev(x), dev(y), dev(b), dev(g), 1.0))
    G_ref, nu = oracle.gauss_grad_x(x, y, b, g, 1.0)
    check_grad(G, G_ref, nu)


@pytest.mark.parametrize("split", [0, 3])
def test_grad_large_cotangent_small_sigma(split):
    """g ~ 1e20 and sigma = 0.05 (the factor 2/sigma^2 = 800): the gradient's bound includes both."""
    say(f"large cotangent split={split}")
    rng = np.random.default_rng(21)
    x = (0.05 * rng.standard_normal((500, 3))).astype(np.float32)
    y = (0.05 * rng.standard_normal((900, 3))).astype(np.float32)
    b = rng.standard_normal((900, 1)).astype(np.float32)
    g = (rng.standard_normal((500, 1)) * 1e20).astype(np.float32)
    gm.keops_set_option(gm.KEOPS_OPT_SPLIT_J, split)
    G = host(gm.keops_gauss_grad_x(dev(x), dev(y), dev(b), dev(g), 0.05))
    G_ref, nu = oracle.gauss_grad_x(x, y, b, g, 0.05)
    assert nu.max() > 1e22
    check_grad(G, G_ref, nu)


@pytest.mark.parametrize("sign", [1, -1])
@pytest.mark.parametrize("form", [0, 1])
@pytest.mark.parametrize("split", [0, 3])
def test_max_large_payload(split, form, sign):
    """Max / Min of K b with b ~ 1e30: values near 1e30 in a 2^64-scaled fp32 would overflow."""
    say(f"large payload max split={split} form={form} sign={sign}")
    x, y, b = big_case(31, bscale=1e30)
    gm.keops_set_option(gm.KEOPS_OPT_SPLIT_J, split)
    gm.keops_set_option(gm.KEOPS_OPT_FORM, form)
    fn = gm.keops_gauss_max if sign > 0 else gm.keops_gauss_min
    v, i = fn(dev(x), dev(y), dev(b), 1.0)
    v_ref, i_ref = oracle.gauss_max(x, y, b, 1.0, sign)
    check_max(x, y, b, 1.0, sign, np.arange(x.shape[0]), host(v), host(i), v_ref, i_ref)


@pytest.mark.parametrize("split", [0, 3])
def test_laplace_large_payload(split):
    """Laplacian sum (always the direct form, offset 2^64) with b ~ 1e20."""
    say(f"large payload laplace split={split}")
    x, y, b = big_case(41)
    gm.keops_set_option(gm.KEOPS_OPT_SPLIT_J, split)
    a = host(gm.keops_laplace_sum(dev(x), dev(y), dev(b), 1.0))
    a_ref, n_ref = oracle.laplace_sum(x, y, b, 1.0)
    check_sum(a, a_ref, n_ref, what="laplace")


@pytest.mark.parametrize("form", [0, 1])
@pytest.mark.parametrize("M", [3, 16, 40])
def test_stream_large_payload(M, form):
    """Few-rows layout (j per lane) with b ~ 1e20, both forms."""
    say(f"large payload stream M={M} form={form}")
    x, y, b = big_case(51 + M, M=M, N=5000)
    gm.keops_set_option(gm.KEOPS_OPT_ROWS, 3)
    gm.keops_set_option(gm.KEOPS_OPT_FORM, form)
    a = host(gm.keops_gauss_sum(dev(x), dev(y), dev(b), 1.0))
    a_ref, n_ref = oracle.gauss_sum(x, y, b, 1.0)
    check_sum(a, a_ref, n_ref)


@pytest.mark.parametrize("split", [0, 3])
def test_far_rows_large_payload(split):
    """Far rows and b ~ 1e20 together: the same work-group meets the floor and the range."""
    say(f"far rows large payload split={split}")
    x, y, b = far_rows(61)
    b = (b * np.float32(1e20)).astype(np.float32)
    gm.keops_set_option(gm.KEOPS_OPT_SPLIT_J, split)
    a = host(gm.keops_gauss_sum(dev(x), dev(y), dev(b), 1.0))
    a_ref, n_ref = oracle.gauss_sum(x, y, b, 1.0)
    check_sum(a, a_ref, n_ref)


@pytest.mark.parametrize("E", [1, 2])
@pytest.mark.parametrize("split", [0, 3])
def test_ranges_far_rows_one_range(split, E):
    """Block-sparse launches with one range that keeps every pair of far-rows data: the same
    result as the dense reductions (sum, LogSumExp, grad_x), far rows included."""
    say(f"ranges far rows split={split} E={E}")
    x, y, b = far_rows(71 + E, E)
    g = np.random.default_rng(72).standard_normal((x.shape[0], E)).astype(np.float32)
    M, N = x.shape[0], y.shape[0]
    ri, si, rj = np.array([[0, M]]), np.array([1]), np.array([[0, N]])
    gm.keops_set_option(gm.KEOPS_OPT_SPLIT_J, split)
    X, Y, B = dev(x), dev(y), dev(b)
    a = host(gm.keops_gauss_sum_ranges(X, Y, B, 1.0, ri, si, rj))
    a_ref, n_ref = oracle.gauss_sum(x, y, b, 1.0)
    assert ((n_ref > 1e-30) & (n_ref < 1e-20)).sum() > 20       # rows under the floor exist
    check_sum(a, a_ref, n_ref)
    check_lse(host(gm.keops_gauss_lse_ranges(X, Y, B, 1.0, ri, si, rj)), oracle.gauss_lse(x, y, b, 1.0))
    G = host(gm.keops_gauss_grad_x_ranges(X, Y, B, dev(g), 1.0, ri, si, rj))
    G_ref, nu = oracle.gauss_grad_x(x, y, b, g, 1.0)
    check_grad(G, G_ref, nu)


def test_ranges_large_payload():
    """Block-sparse sum with b ~ 1e20 over random ranges that split the rows and the j."""
    say("ranges large payload")
    x, y, b = big_case(81)
    M, N = x.shape[0], y.shape[0]
    ri = np.array([[0, 300], [300, M]])
    si = np.array([2, 3])
    rj = np.array([[0, 800], [900, N], [100, 1200]])
    a = host(gm.keops_gauss_sum_ranges(dev(x), dev(y), dev(b), 1.0, ri, si, rj))
    a_ref, n_ref = oracle.gauss_sum_ranges(x, y, b, 1.0, ri, si, rj)
    check_sum(a, a_ref, n_ref)
