"""Host-side block-sparse preparation (grid clusters, ranges, truncation mask) and the
range validation of the C ABI; no GPU needed."""
import ctypes
import math
import os

import numpy as np
import pytest

from geometric_map_reduce_amd import blocksparse as bs


def test_grid_cluster_and_ranges():
    rng = np.random.default_rng(0)
    p = rng.random((2000, 3)).astype(np.float32)
    lab = bs.grid_cluster(p, 0.25)
    cells = np.floor(p.astype(np.float64) / 0.25).astype(np.int64)
    # same label <=> same voxel
    for a, b in rng.integers(0, 2000, size=(500, 2)):
        assert (lab[a] == lab[b]) == bool(np.all(cells[a] == cells[b]))
    perm = bs.sort_by_cluster(lab)
    ps, ls = p[perm], lab[perm]
    ranges, cen, rad = bs.cluster_ranges_centroids(ps, ls)
    assert ranges[0, 0] == 0 and ranges[-1, 1] == 2000 and np.all(ranges[1:, 0] == ranges[:-1, 1])
    for c, (lo, hi) in enumerate(ranges):
        assert np.all(ls[lo:hi] == ls[lo])
        np.testing.assert_allclose(cen[c], ps[lo:hi].astype(np.float64).mean(0), rtol=1e-12)
        d = np.sqrt(((ps[lo:hi] - cen[c]) ** 2).sum(1))
        assert np.all(d <= rad[c] + 1e-12) and np.isclose(d.max(), rad[c])


def test_truncation_mask_is_conservative():
    """Every pair of points closer than the cutoff lies in a kept cluster pair."""
    rng = np.random.default_rng(1)
    x = rng.random((600, 3)).astype(np.float32)
    y = rng.random((700, 3)).astype(np.float32)
    sigma, eps = 0.1, 1e-3
    cut = bs.cutoff_for(sigma, eps)
    assert math.isclose(math.exp(-(cut / sigma) ** 2), eps, rel_tol=1e-12)
    px, py = bs.sort_by_cluster(bs.grid_cluster(x, 0.2)), bs.sort_by_cluster(bs.grid_cluster(y, 0.2))
    xs, ys = x[px], y[py]
    rx, cx, radx = bs.cluster_ranges_centroids(xs, bs.grid_cluster(x, 0.2)[px])
    ry, cy, rady = bs.cluster_ranges_centroids(ys, bs.grid_cluster(y, 0.2)[py])
    mask = bs.truncation_mask(cx, radx, cy, rady, cut)
    ri, si, rj = bs.ranges_from_mask(mask, rx, ry)
    kept = np.zeros((600, 700), bool)
    for c, (lo, hi) in enumerate(ri):
        for k in range(si[c - 1] if c else 0, si[c]):
            kept[lo:hi, rj[k, 0]:rj[k, 1]] = True
    d = np.sqrt(((xs[:, None, :].astype(np.float64) - ys[None].astype(np.float64)) ** 2).sum(-1))
    assert np.all(kept[d < cut]) and 0 < kept.mean() < 1
    # the ranges reproduce the cluster mask exactly, with no j listed twice
    cl = np.zeros((len(rx), len(ry)), bool)
    for c in range(len(rx)):
        for k in range(si[c - 1] if c else 0, si[c]):
            cl[c, np.flatnonzero((ry[:, 0] >= rj[k, 0]) & (ry[:, 1] <= rj[k, 1]))] = True
    assert np.array_equal(cl, mask)


FAKE = ctypes.c_void_p(0x10000)
FAKE2 = ctypes.c_void_p(0x20000000)


@pytest.fixture(scope="module")
def L():
    from geometric_map_reduce_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("library not built")
    return binding.lib()


def _call(L, ri, si, rj, M=10, N=20):
    ri = np.ascontiguousarray(ri, np.int64).reshape(-1, 2)
    si = np.ascontiguousarray(si, np.int64).ravel()
    rj = np.ascontiguousarray(rj, np.int64).reshape(-1, 2)
    hp = lambda a: a.ctypes.data_as(ctypes.c_void_p) if a.size else None  # noqa: E731
    return L.keops_gauss_sum_ranges(FAKE, FAKE2, FAKE2, M, N, 3, 1, 1.0, hp(ri), ri.shape[0], hp(si), hp(rj),
                                    rj.shape[0], ctypes.c_void_p(0x900000), None)


@pytest.mark.parametrize("ri,si,rj", [
    ([[0, 11]], [1], [[0, 5]]),             # row range beyond M
    ([[5, 3]], [1], [[0, 5]]),              # reversed row range
    ([[0, 6], [5, 10]], [1, 1], [[0, 5]]),  # overlapping row ranges
    ([[0, 5], [5, 10]], [1, 0], [[0, 5]]),  # decreasing slices
    ([[0, 5]], [2], [[0, 5]]),              # slice beyond the j ranges
    ([[0, 5]], [1], [[0, 21]]),             # j range beyond N
    ([[0, 5]], [1], [[-1, 3]]),             # negative j
])
def test_ranges_validation(L, ri, si, rj):
    assert _call(L, ri, si, rj) == -1


def test_ranges_empty_is_valid_on_host(L):
    # M = 0 with no ranges: nothing to do, no device work
    assert L.keops_gauss_sum_ranges(None, FAKE2, FAKE2, 0, 20, 3, 1, 1.0, None, 0, None, None, 0, None, None) == 0
