"""keops_gauss_sum_noalloc: the Gaussian sum with its workspace in the library's fixed
device scratch, through the C ABI, against keops_gauss_sum on the same inputs (and both
against the float64 oracle).  Two calls in a row on one GPU, the second smaller, so the
second reuses the scratch the first left behind; a shape whose usual split-j partials do
not fit (fewer splits, same results to the tolerance); the few-rows and the MFMA layouts.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from parity import check_sum, dev, host

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import geometric_map_reduce_amd as gm
    from geometric_map_reduce_amd import binding, workloads


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    for o in (gm.KEOPS_OPT_SPLIT_J, gm.KEOPS_OPT_FORM, gm.KEOPS_OPT_ROWS, gm.KEOPS_OPT_WG_TARGET, gm.KEOPS_OPT_MFMA):
        gm.keops_set_option(o, 0)


def case(seed, M, N, D, E, scale=1.0):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((M, D)) * scale).astype(np.float32)
    y = (rng.standard_normal((N, D)) * scale).astype(np.float32)
    b = rng.standard_normal((N, E)).astype(np.float32)
    return x, y, b


def both(x, y, b, sigma):
    X, Y, B = dev(x), dev(y), dev(b)
    a_na = binding.keops_gauss_sum_noalloc(X, Y, B, sigma)
    torch.cuda.synchronize()
    a = binding.keops_gauss_sum(X, Y, B, sigma)
    torch.cuda.synchronize()
    return host(a_na), host(a)


def oracle_rows(x, y, b, sigma, n=300, seed=1):
    rows = workloads.sample_rows(x.shape[0], min(n, x.shape[0]), seed=seed)
    ref, nrm = oracle.gauss_sum(x, y, b, sigma, rows=rows)
    return rows, ref, nrm


def test_two_calls_second_smaller():
    """Same launch plan as keops_gauss_sum (the partials fit): identical bits, both calls."""
    for seed, (M, N, D, E, sigma) in enumerate([(20000, 30000, 3, 2, 0.5), (700, 1100, 3, 1, 0.7)]):
        print(f"no-alloc call {seed}: M={M} N={N} D={D} E={E}", flush=True)
        x, y, b = case(100 + seed, M, N, D, E)
        a_na, a = both(x, y, b, sigma)
        assert np.array_equal(a_na, a)
        rows, ref, nrm = oracle_rows(x, y, b, sigma)
        check_sum(a_na[rows], ref, nrm)


def test_fewer_splits_when_partials_do_not_fit():
    """M = 200k, N = 100k, E = 4: the usual plan's partials need about 270 MB, so the call
    takes as many j-splits as 64 MiB holds; the results agree to the tolerance."""
    M, N, D, E, sigma = 200_000, 100_000, 3, 4, 0.3
    print(f"no-alloc capped splits: M={M} N={N} E={E}", flush=True)
    x, y, b = case(7, M, N, D, E)
    a_na, a = both(x, y, b, sigma)
    rows, ref, nrm = oracle_rows(x, y, b, sigma, n=200)
    check_sum(a_na[rows], ref, nrm)
    check_sum(a[rows], ref, nrm)
    _, nrm_all = oracle.gauss_sum(x, y, b, sigma, rows=rows)
    assert np.all(np.abs(a_na[rows] - a[rows]) <= 2e-4 * nrm_all + 1e-37)
    # and a smaller call right after, on the scratch this one filled
    x2, y2, b2 = case(8, 3000, 5000, D, 1)
    a_na2, a2 = both(x2, y2, b2, sigma)
    assert np.array_equal(a_na2, a2)


@pytest.mark.parametrize("M", [3, 40])
def test_few_rows_layout(M):
    print(f"no-alloc few rows M={M}", flush=True)
    x, y, b = case(9 + M, M, 200_000, 3, 1)
    a_na, a = both(x, y, b, 0.5)
    assert np.array_equal(a_na, a)
    ref, nrm = oracle.gauss_sum(x, y, b, 0.5)
    check_sum(a_na, ref, nrm)


def test_mfma_layout():
    print("no-alloc D=50", flush=True)
    x, y, b = case(11, 3000, 20000, 50, 1, scale=1 / np.sqrt(50))
    a_na, a = both(x, y, b, 1.0)
    assert np.array_equal(a_na, a)
    rows, ref, nrm = oracle_rows(x, y, b, 1.0)
    check_sum(a_na[rows], ref, nrm)
