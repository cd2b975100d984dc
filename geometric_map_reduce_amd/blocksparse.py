"""Host-side preparation of block-sparse reductions: grid clusters, their ranges
and the truncation mask, in the range format of ``keops_gauss_*_ranges``.

KeOps pages: "Kernel Operations on the GPU, with Autodiff, without Memory
Overflows" §3 "Applications" (cluster-wise block-sparsity for large kernel
linear systems) and §4 (the block-sparse truncation rule); the README feature
list (an interface for block-sparse and coarse-to-fine strategies).

The steps, all on host arrays (numpy), done once per point set:

1. ``grid_cluster``: one label per point, the index of its cubic voxel of side
   ``voxel`` among the occupied voxels (in lexicographic voxel order).
2. ``sort_by_cluster``: a stable permutation that makes every cluster a
   contiguous run of points; the caller reorders x, y, b with it (and maps the
   results back with its inverse).
3. ``cluster_ranges_centroids``: the [start, end) range of every cluster in the
   sorted order, its centroid and its radius (largest distance of a member to
   the centroid).
4. ``truncation_mask``: keep the cluster pair (I, J) unless every pair of
   their points is at least ``cutoff`` apart, judged by
   |c_I - c_J| - r_I - r_J >= cutoff; ``cutoff_for`` gives the distance beyond
   which exp(-d^2 / sigma^2) <= eps.  A dropped pair (i, j) therefore has
   K_ij <= eps, and a row's truncation error is at most eps * sum_j |b_j|.
5. ``ranges_from_mask``: the row ranges, slice ends and j ranges of the kept
   cluster pairs, merging j clusters that are adjacent in the sorted order.

The reductions themselves run on the GPU; nothing here touches the results.
"""
from __future__ import annotations

import math

import numpy as np


def grid_cluster(points: np.ndarray, voxel: float) -> np.ndarray:
    """int64 label per point: the rank of its voxel floor(p / voxel) among the occupied ones."""
    p = np.asarray(points, np.float64)
    if p.ndim != 2:
        raise ValueError("points must be [N, D]")
    if not voxel > 0:
        raise ValueError("voxel must be positive")
    cells = np.floor(p / float(voxel)).astype(np.int64)
    if cells.shape[0] == 0:
        return np.zeros(0, np.int64)
    cells -= cells.min(0)
    span = cells.max(0) + 1
    if np.prod(span.astype(np.float64)) < 2.0 ** 62:
        # one integer key per voxel, in the same lexicographic order as the cells
        key = np.zeros(cells.shape[0], np.int64)
        for d in range(cells.shape[1]):
            key = key * span[d] + cells[:, d]
        _, labels = np.unique(key, return_inverse=True)
    else:
        _, labels = np.unique(cells, axis=0, return_inverse=True)
    return labels.reshape(-1).astype(np.int64)


def sort_by_cluster(labels: np.ndarray) -> np.ndarray:
    """Stable permutation perm such that labels[perm] is non-decreasing."""
    return np.argsort(np.asarray(labels, np.int64), kind="stable")


def cluster_ranges_centroids(points_sorted: np.ndarray, labels_sorted: np.ndarray):
    """(ranges [C, 2] int64, centroids [C, D] float64, radii [C] float64) of the clusters of points
    already sorted by label (labels_sorted non-decreasing)."""
    p = np.asarray(points_sorted, np.float64)
    lab = np.asarray(labels_sorted, np.int64)
    if lab.size and np.any(np.diff(lab) < 0):
        raise ValueError("labels must be sorted")
    starts = np.flatnonzero(np.r_[True, lab[1:] != lab[:-1]]) if lab.size else np.zeros(0, np.int64)
    ends = np.r_[starts[1:], lab.size].astype(np.int64)
    ranges = np.stack([starts, ends], 1).astype(np.int64)
    counts = (ends - starts).astype(np.float64)
    sums = np.add.reduceat(p, starts, axis=0) if lab.size else np.zeros((0, p.shape[1]))
    centroids = sums / counts[:, None] if lab.size else sums
    seg = np.repeat(np.arange(len(starts)), (ends - starts))
    d = np.sqrt(((p - centroids[seg]) ** 2).sum(1)) if lab.size else np.zeros(0)
    radii = np.zeros(len(starts))
    np.maximum.at(radii, seg, d)
    return ranges, centroids, radii


def cutoff_for(sigma: float, eps: float) -> float:
    """The distance d with exp(-d^2 / sigma^2) = eps: pairs farther apart have K_ij <= eps."""
    if not (0 < eps < 1):
        raise ValueError("eps must be in (0, 1)")
    return float(sigma) * math.sqrt(math.log(1.0 / eps))


def truncation_mask(centroids_i, radii_i, centroids_j, radii_j, cutoff: float) -> np.ndarray:
    """bool [CI, CJ]: True where the cluster pair may hold a pair of points closer than cutoff."""
    ci = np.asarray(centroids_i, np.float64)
    cj = np.asarray(centroids_j, np.float64)
    d2 = ((ci[:, None, :] - cj[None, :, :]) ** 2).sum(-1)
    gap = np.sqrt(d2) - np.asarray(radii_i)[:, None] - np.asarray(radii_j)[None, :]
    return gap < float(cutoff)


def ranges_from_mask(mask: np.ndarray, ranges_i: np.ndarray, ranges_j: np.ndarray):
    """(ranges_i, slices_i, redranges_j) of the kept cluster pairs.  Row ranges are the row
    clusters; each one's j ranges are its kept j clusters, runs of consecutive clusters merged
    into one range (they are contiguous in the sorted order)."""
    mask = np.asarray(mask, bool)
    ri = np.asarray(ranges_i, np.int64).reshape(-1, 2)
    rj = np.asarray(ranges_j, np.int64).reshape(-1, 2)
    if mask.shape != (ri.shape[0], rj.shape[0]):
        raise ValueError("mask must be [row clusters, j clusters]")
    slices, red = [], []
    for row in mask:
        kept = np.flatnonzero(row)
        if kept.size:
            breaks = np.flatnonzero(np.diff(kept) != 1)
            first = np.r_[kept[0], kept[breaks + 1]]
            last = np.r_[kept[breaks], kept[-1]]
            red.extend(zip(rj[first, 0].tolist(), rj[last, 1].tolist()))
        slices.append(len(red))
    return (ri.copy(), np.asarray(slices, np.int64), np.asarray(red, np.int64).reshape(-1, 2))
