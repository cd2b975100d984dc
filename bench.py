#!/usr/bin/env python
"""Benchmark of the Gaussian kernel mat-vec on one MI355X.

Default workload (one "step" = one call of the whole hot path on resident
inputs): the Gaussian kernel sum a_i = sum_j exp(-|x_i - y_j|^2 / sigma^2) b_j
at M = N = 1,000,000, D = 3, E = 1, sigma = 0.1, x, y ~ U[0,1)^3,
b ~ N(0, 1), seed 0 -- the shape of the KeOps paper's benchmark (M = N
points in dimension 3; timings quoted up to N = 1M).

Prints ONE JSON line:
  value         G pair-evaluations per second (M*N / time per step)
  roofline      fp32 VALU roofline of the pair-evaluation kernel: algorithmic
                flops per launch (12 per pair at D = 3, E = 1) / the kernel's
                average duration, measured here with HIP events recorded by
                the library around each launch on the call's stream;
                traffic = HBM bytes per launch from the recorded rocprofv3
                counter runs (null when the kernel sources changed since)
  cpu_baseline  the float64 oracle timed on this host's cores over a bounded
                sample of rows (each row over all N), scaled to pair-evals/s
Other workloads (--workload) print the same fields for their own op; the
few-rows sum (--workload stream: 16 rows against 1e8 points) is bound by
streaming y and b from HBM and reports its roofline in GB/s against 8 TB/s.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Gaussian kernel mat-vec G pair-evals/s @ M=N=1M,D=3; % fp32 VALU peak"
PEAK_FP32_TFLOPS = 157.3          # MI355X fp32 vector peak, and fp32 MFMA (dense) peak
PEAK_BF16_TFLOPS = 2500.0         # MI355X bf16 MFMA (dense) peak
PAGES_PAIRS_PER_S_1M = 1e12 / 1.38  # the pages' KeOps timing at N = 1M (hardware not stated)

# (op, workload name, algorithmic flops per pair)
#  sum: 3D + 1 + 2E (D subtractions, D squares, D-1 adds, 1 scale, 1 exp, E multiply-adds)
#  lse: 3D + 5 (distance 3D-1, scale, +b, max, -m, exp, add)
#  grad: 5D + 2E + 1;  kmin: 3D (distance 3D-1, compare)
BENCHES = {
    "sum": ("sum", "sum_lse_1M"),
    "lse": ("lse", "sum_lse_1M"),
    "grad": ("grad_x", "sum_grad_10k"),
    "grad_y": ("grad_y", "sum_lse_1M"),
    "grad_b": ("grad_b", "sum_lse_1M"),
    "sum10k": ("sum", "sum_grad_10k"),
    "sum1k": ("sum", "sum_1k"),
    "solver": ("sum", "solver_matvec_100k_x_10M"),
    "solver_lse": ("lse", "solver_matvec_100k_x_10M"),
    "solver_grad": ("grad_x", "solver_matvec_100k_x_10M"),
    "kmin3": ("kmin", "kmin10_1M_d3"),
    "kmin64": ("kmin", "kmin10_1M_d64"),
    "stream": ("sum", "stream_16_x_100M"),
    "stream_lse": ("lse", "stream_16_x_100M"),
    "stream_grad": ("grad_x", "stream_16_x_100M"),
    "stream_kmin": ("kmin", "kmin10_16_x_100M"),
    "cg": ("cg", "krige_100k"),
    "sum_bs": ("sum_ranges", "sum_lse_1M"),
    "max": ("max", "sum_lse_1M"),
    "laplace": ("laplace", "sum_lse_1M"),
}
BS_VOXEL, BS_EPS = 0.1, 1e-5       # block-sparse bench: voxel side and truncation threshold
CG_RTOL = 1e-4
PEAK_HBM_GBS = 8000.0             # MI355X HBM3E peak
STREAM_MAX_ROWS = 64              # the library's few-rows layout (j per lane), D <= 8


def flops_per_pair(op, D, E):
    return {"sum": 3 * D + 1 + 2 * E, "cg": 3 * D + 1 + 2 * E, "sum_ranges": 3 * D + 1 + 2 * E,
            "max": 3 * D + 1 + 2 * E, "laplace": 3 * D + 2 + 2 * E, "lse": 3 * D + 5, "grad_x": 5 * D + 2 * E + 1, "grad_y": 5 * D + 2 * E + 1,
            "grad_b": 3 * D + 1 + 2 * E, "kmin": 3 * D}[op]


def uses_mfma(op, D):
    """Ops whose pair map runs the -2<x, y> cross term on MFMA (D >= 32)."""
    return D >= 32 and op in ("sum", "lse", "kmin", "grad_x")


STREAM_KERNELS = {"sum": "gauss_stream_kernel", "lse": "gauss_stream_lse_kernel",
                  "grad_x": "gauss_stream_grad_kernel", "kmin": "kmin_stream_kernel"}


def is_stream(op, M, D):
    """At few rows the sum, LogSumExp, grad_x and K-min run the j-per-lane kernels, whose
    floor is streaming y (and b) from HBM once."""
    return op in STREAM_KERNELS and M <= STREAM_MAX_ROWS and D <= 8


def roofline_of(op, M, D, E):
    """(bound, algorithmic units per pair, kernel name) of the dominant pass-1 kernel.
    MFMA sum and LogSumExp: the contraction <x~, y~> of 2D flops per pair against the
    fp32 matrix peak (the per-pair exp and accumulate are VALU work on top).  MFMA
    grad_x: that contraction and the weighted sum of y, 4D flops per pair.  MFMA K-min: the distance's
    contraction, 2D algorithmic flops per pair, against the peak of the bf16 matrix pipe
    the split-bf16 prefilter runs on (it executes three bf16 products, 6D flops, reported
    beside it).  Few-rows kernels: HBM bytes, priced per launch (y and b read once)
    rather than per pair."""
    if is_stream(op, M, D):
        return "hbm", None, STREAM_KERNELS[op]
    if uses_mfma(op, D):
        if op == "sum":
            return "mfma", 2 * D, "gauss_mfma_kernel<sum>"
        if op == "lse":
            return "mfma", 2 * D, "gauss_mfma_kernel<lse>"
        if op == "grad_x":
            return "mfma", 4 * D, "gauss_mfma_grad_kernel"
        return "mfma_bf16", 2 * D, "kmin_mfma_split_kernel"
    # the transposed gradients run the row kernels with y as the rows
    kop = {"grad_y": "grad_x", "grad_b": "sum", "cg": "sum", "sum_ranges": "sum"}.get(op, op)
    if op == "laplace":
        return "alu", flops_per_pair(op, D, E), "laplace_sum (gauss_valu_kernel<OP_LAPLACE>)"
    name = "kmin_valu_kernel" if op == "kmin" else f"gauss_valu_kernel<{kop}>"
    return "alu", flops_per_pair(op, D, E), name


def stream_bytes(w, op="sum"):
    """Algorithmic HBM bytes of one few-rows launch: the inputs read once, the outputs
    written once (K-min reads no b and writes K fp32 distances and int64 indices per row;
    grad_x also reads the cotangent [M, E] and writes [M, D])."""
    if op == "kmin":
        return 4 * (w.N * w.D + w.M * w.D) + 12 * w.M * w.K
    extra = w.M * w.E + w.M * w.D if op == "grad_x" else w.M * w.E
    return 4 * (w.N * (w.D + w.E) + w.M * w.D + extra)


# sources that define each benchmarked kernel and its launch plan
_COMMON_SRC = ["common.h", "launch.h", "keops_api.cpp"]
KERNEL_SOURCES = {
    "sum": ["gauss_kernel.h", "dispatch_gauss.h", "gauss_sum_small.hip"],
    "lse": ["gauss_kernel.h", "dispatch_gauss.h", "gauss_lse_small.hip"],
    "grad_x": ["gauss_kernel.h", "dispatch_gauss.h", "gauss_grad_small.hip"],
    "kmin": ["kmin_kernel.h", "dispatch_kmin.h", "kmin_d1_4.hip"],
    "kmin_split": ["kmin_kernel.h", "kmin_mfma_split.h", "kmin_mfma_split.hip"],
    "stream": ["gauss_stream.h", "gauss_stream.hip"],
    "stream_ops": ["gauss_stream_ops.h", "gauss_stream_ops.hip"],
    "kmin_stream": ["kmin_kernel.h", "kmin_stream.h", "kmin_stream.hip"],
}
# the kernel whose HBM traffic each workload records (rocprofv3's kernel name)
TRAFFIC_KERNELS = {
    "sum": ("sum", "gauss_valu_kernel<0, 3, 1, 2>"),
    "stream": ("stream", "gauss_stream_kernel<3, 1, 16>"),
    "kmin64": ("kmin_split", "kmin_mfma_split_kernel<64, 10>"),
    "stream_kmin": ("kmin_stream", "kmin_stream_kernel<3, 10, 4>"),
}
COPY_KNOWN_KIB = 262144.0          # the calibration copy reads and writes 256 MiB per launch


def kernel_source_hash(op):
    """sha256 over the sources of one op's pass-1 kernel (traffic is void once they change)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "geometric_map_reduce_amd", "csrc")
    for f in sorted(_COMMON_SRC + KERNEL_SOURCES[op]):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def recorded_traffic(bench_name, op):
    """HBM bytes per launch from profiles/traffic_<bench>.json if it matches the current sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{bench_name}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_sources_sha256") != kernel_source_hash(op):
        return None
    return rec.get("hbm_bytes_per_launch")


def _counter_per_dispatch(csv_path, kernel):
    """Per-dispatch sums (over XCDs and instances) of the one counter in a rocprofv3
    --pmc CSV, for the dispatches whose kernel name contains ``kernel``."""
    import csv
    agg = {}
    with open(csv_path) as fh:
        for r in csv.DictReader(fh):
            if kernel in r["Kernel_Name"]:
                agg[r["Dispatch_Id"]] = agg.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return [agg[k] for k in sorted(agg, key=int)]


def record_traffic(workload, fetch_csv, write_csv, cal_fetch_csv, cal_write_csv):
    """Write profiles/traffic_<workload>.json from four rocprofv3 --pmc runs (FETCH_SIZE and
    WRITE_SIZE, each of this workload and of --workload copycal).  The counters read KiB
    per dispatch; each is scaled by what it reads for the copy kernel of known size (the
    copy's first dispatch, a warm-up that also pages in, is left out)."""
    import statistics
    src_key, kernel = TRAFFIC_KERNELS[workload]
    cf = _counter_per_dispatch(cal_fetch_csv, "elementwise")[1:]
    cw = _counter_per_dispatch(cal_write_csv, "elementwise")[1:]
    f = _counter_per_dispatch(fetch_csv, kernel)
    w = _counter_per_dispatch(write_csv, kernel)
    if not (cf and cw and f and w):
        raise SystemExit(f"no dispatches of {kernel!r} or of the copy kernel in the given CSVs")
    ff, wf = COPY_KNOWN_KIB / statistics.mean(cf), COPY_KNOWN_KIB / statistics.mean(cw)
    fb, wb = round(statistics.mean(f) * 1024 * ff), round(statistics.mean(w) * 1024 * wf)
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    rec = json.load(open(path)) if os.path.exists(path) else {}
    rec.update({
        "kernel": rec.get("kernel", kernel),
        "fetch_size_kib_per_dispatch": f,
        "write_size_kib_per_dispatch": w,
        "copy_calibration": {"kernel": "torch neg elementwise, 256 MiB read + 256 MiB written",
                             "fetch_size_kib": cf, "write_size_kib": cw,
                             "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)},
        "hbm_fetch_bytes_per_launch": fb,
        "hbm_write_bytes_per_launch": wb,
        "hbm_bytes_per_launch": fb + wb,
        "kernel_sources_sha256": kernel_source_hash(src_key),
    })
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps({"workload": workload, "kernel": kernel, "hbm_fetch_bytes": fb, "hbm_write_bytes": wb,
                      "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)}))


def run_op(gm, op, X, Y, B, G, sigma, K, out, lam=0.0, ranges=None):
    if op == "sum_ranges":
        return gm.keops_gauss_sum_ranges(X, Y, B, sigma, *ranges, out=out)
    if op == "cg":
        return gm.keops_gauss_cg(X, B, sigma, lam, rtol=CG_RTOL, max_iter=1000, out=out)
    if op == "sum":
        return gm.keops_gauss_sum(X, Y, B, sigma, out=out)
    if op == "max":
        return gm.keops_gauss_max(X, Y, B, sigma, out=out[0], out_idx=out[1])
    if op == "laplace":
        return gm.keops_laplace_sum(X, Y, B, sigma, out=out)
    if op == "lse":
        return gm.keops_gauss_lse(X, Y, B, sigma, out=out)
    if op == "grad_x":
        return gm.keops_gauss_grad_x(X, Y, B, G, sigma, out=out)
    if op == "grad_y":
        return gm.keops_gauss_grad_y(X, Y, B, G, sigma, out=out)
    if op == "grad_b":
        return gm.keops_gauss_grad_b(X, Y, G, sigma, out=out)
    return gm.keops_kmin(X, Y, K, out_d=out[0], out_idx=out[1])


def block_sparse_setup(x, y, b, sigma):
    """Sort x, y (and b) by voxel clusters and build the truncation ranges (host preparation,
    outside the timed region).  Returns the permuted inputs, the ranges and the kept pairs."""
    import numpy as np

    from geometric_map_reduce_amd import blocksparse as bs
    lx, ly = bs.grid_cluster(x, BS_VOXEL), bs.grid_cluster(y, BS_VOXEL)
    px, py = bs.sort_by_cluster(lx), bs.sort_by_cluster(ly)
    rx, cx, radx = bs.cluster_ranges_centroids(x[px], lx[px])
    ry, cy, rady = bs.cluster_ranges_centroids(y[py], ly[py])
    mask = bs.truncation_mask(cx, radx, cy, rady, bs.cutoff_for(sigma, BS_EPS))
    ri, si, rj = bs.ranges_from_mask(mask, rx, ry)
    starts = np.r_[0, si[:-1]]
    tj = np.array([(rj[s:e, 1] - rj[s:e, 0]).sum() for s, e in zip(starts, si)], np.int64)
    kept = int(((ri[:, 1] - ri[:, 0]) * tj).sum())
    return x[px], y[py], b[py], (ri, si, rj), kept


def cpu_baseline(op, w, x, y, b, g, target_s, gpu_out, ranges=None):
    import numpy as np

    import oracle
    from geometric_map_reduce_amd import workloads

    def call(rows):
        t0 = time.perf_counter()
        if op == "sum_ranges":      # the oracle sum of each sampled row over its kept j ranges
            ri, si, rj = ranges
            owner = np.zeros(w.M, np.int64)
            for c, (lo, hi) in enumerate(ri):
                owner[lo:hi] = c
            res = (np.zeros((len(rows), w.E)), np.zeros((len(rows), w.E)))
            for c in np.unique(owner[rows]):
                sel = np.flatnonzero(owner[rows] == c)
                J = np.concatenate([np.arange(a, e) for a, e in rj[(si[c - 1] if c else 0):si[c]]])
                res[0][sel], res[1][sel] = oracle.gauss_sum(x, y[J], b[J], w.sigma, rows=rows[sel])
            return time.perf_counter() - t0, res
        if op == "sum":
            res = oracle.gauss_sum(x, y, b, w.sigma, rows=rows)
        elif op == "max":
            res = oracle.gauss_max(x, y, b, w.sigma, 1, rows=rows)
        elif op == "laplace":
            res = oracle.laplace_sum(x, y, b, w.sigma, rows=rows)
        elif op == "cg":        # the solver's work is its products K p: the sum oracle on x
            res = oracle.gauss_sum(x, x, b, w.sigma, rows=rows)
        elif op == "lse":
            res = oracle.gauss_lse(x, y, b, w.sigma, rows=rows)
        elif op == "grad_x":
            res = oracle.gauss_grad_x(x, y, b, g, w.sigma, rows=rows)
        elif op == "grad_y":
            res = oracle.gauss_grad_y(x, y, b, g, w.sigma, cols=rows)
        elif op == "grad_b":
            res = oracle.gauss_grad_b(x, y, g, w.sigma, cols=rows)
        else:
            res = oracle.kmin(x, y, w.K, rows=rows)
        return time.perf_counter() - t0, res

    # outputs per row i, or per point j for the transposed gradients
    n_out, n_red = (w.N, w.M) if op in ("grad_y", "grad_b") else (w.M, w.N)
    probe = workloads.sample_rows(n_out, min(n_out, 64), seed=2)
    t_probe, _ = call(probe)
    per_row = max(t_probe / len(probe), 1e-9)
    n = int(min(n_out, max(64, target_s / per_row)))
    rows = workloads.sample_rows(n_out, n, seed=1)
    t, res = call(rows)
    pairs = len(rows) * n_red
    if op == "sum_ranges":
        ri, si, rj = ranges
        per_c = np.array([(rj[s:e, 1] - rj[s:e, 0]).sum() for s, e in zip(np.r_[0, si[:-1]], si)])
        owner = np.zeros(w.M, np.int64)
        for c, (lo, hi) in enumerate(ri):
            owner[lo:hi] = c
        pairs = int(per_c[owner[rows]].sum())
    base = {"value": pairs / t / 1e9, "unit": "G pair-evals/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": (f"{len(rows)} seeded points j x all {w.M} i" if op in ("grad_y", "grad_b") else
                       f"{len(rows)} seeded rows x their kept j ({pairs} pairs)" if op == "sum_ranges" else
                       f"{len(rows)} seeded rows x all {w.N} j") + f" (float64 C/OpenMP oracle), {t:.1f} s"}
    # the same rows double as a spot check of the GPU result
    check = None
    if op == "cg":
        check = None
    elif op == "max":
        ref, _ = res
        gpu = gpu_out[rows].reshape(ref.shape).astype(np.float64)
        check = {"rows": len(rows), "max_rel_err": float(np.max(np.abs(gpu - ref) / np.maximum(np.abs(ref), 1e-300)))}
    elif op in ("sum", "grad_x", "grad_y", "grad_b", "sum_ranges", "laplace"):
        ref, nrm = res
        gpu = gpu_out[rows].reshape(ref.shape).astype(np.float64)
        check = {"rows": len(rows), "max_err_over_norm": float(np.max(np.abs(gpu - ref) / np.maximum(nrm, 1e-300)))}
    elif op == "lse":
        check = {"rows": len(rows), "max_abs_err": float(np.max(np.abs(gpu_out[rows].astype(np.float64) - res)))}
    elif op == "kmin":
        # index lists equal to the oracle's, or differing only among candidates whose
        # distances lie within 1e-5 relative of each other (near ties)
        d_ref, i_ref = res
        d_gpu, i_gpu = gpu_out
        i_gpu = i_gpu[rows]
        same = np.all(i_gpu == i_ref, axis=1)
        swaps = bad = 0
        for r in np.flatnonzero(~same):
            dx = ((x[rows[r]].astype(np.float64) - y[i_gpu[r]].astype(np.float64)) ** 2).sum(axis=1)
            if np.all(np.abs(np.sort(dx) - d_ref[r]) <= 1e-5 * np.maximum(d_ref[r], 1e-30)):
                swaps += 1
            else:
                bad += 1
        check = {"rows": len(rows), "exact_rows": int(same.sum()), "near_tie_swaps": swaps, "mismatches": bad}
    return base, check


def copy_calibration(torch, args):
    """A plain streaming kernel of known traffic (read 256 MiB, write 256 MiB), run under the
    same rocprofv3 counters as the hot kernel to scale FETCH_SIZE / WRITE_SIZE into bytes."""
    n = 64 << 20
    src = torch.ones(n, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(args.warmup + args.steps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"workload": "copycal", "kernel": "torch neg (elementwise)", "launches": args.warmup + args.steps,
                      "read_bytes_per_launch": 4 * n, "write_bytes_per_launch": 4 * n}), flush=True)


MICRO_PROBES = ["fma", "add", "exp", "fma_exp", "mfma_f32", "mfma_bf16", "mfma_fma_wave", "mfma_exp_wave",
                "split_mfma", "split_valu", "split_both", "pair_valu", "pair_mfma", "bank_free", "bank_two",
                "bank_three"]


def micro_rates(torch):
    """Instruction rates of the chip (geometric_map_reduce_amd/micro/rates.hip): for each probe
    the kernel time, the engine clock it ran at, the cycles one SIMD spends per wave64
    instruction of each kind, and for the pair probes the Gaussian pair-evaluations per second.
    Prints one JSON line."""
    import ctypes

    from geometric_map_reduce_amd import build as gbuild
    lib = ctypes.CDLL(gbuild.MICRO_LIB)
    lib.keops_micro_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_float),
                                    ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    assert lib.keops_micro_count() == len(MICRO_PROBES)
    torch.cuda.init()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    simds = 4 * cus
    kinds = ["fma", "add", "exp", "mfma_f32", "mfma_bf16"]
    res = {}
    for pid, name in enumerate(MICRO_PROBES):
        threads = 512 if name.startswith("split") else 256
        blocks = cus * (4 if threads == 512 else 8)
        iters = 64 if name.startswith("pair") else 2048
        for _ in range(2):              # the first launch also loads the code object
            ms, mhz = ctypes.c_float(0), ctypes.c_double(0)
            cnt = (ctypes.c_double * 8)()
            rc = lib.keops_micro_run(pid, blocks, iters, ctypes.byref(ms), ctypes.byref(mhz), cnt)
            if rc != 0:
                raise RuntimeError(f"micro probe {name}: status {rc}")
        t = ms.value * 1e-3
        simd_cycles = t * mhz.value * 1e6 * simds      # SIMD-cycles available during the launch
        waves = cnt[5]
        r = {"ms": round(ms.value, 4), "clock_mhz": round(mhz.value, 1), "blocks": blocks, "threads": threads,
             "iters": iters}
        instr = {k: cnt[q] * waves for q, k in enumerate(kinds) if cnt[q] > 0}
        # cycles of one SIMD per wave64 instruction, all kinds of the probe together
        tot = sum(instr.values())
        if tot:
            r["wave_instr"] = {k: v for k, v in instr.items()}
            r["simd_cycles_per_wave_instr"] = round(simd_cycles / tot, 3)
            if len(instr) == 1:
                k = next(iter(instr))
                per_s = instr[k] * 64 / t
                if k.startswith("mfma"):
                    flops = (16 * 16 * 4 * 2 if k == "mfma_f32" else 16 * 16 * 32 * 2) * instr[k] / t
                    r["tflops"] = round(flops / 1e12, 2)
                else:
                    r["lane_ops_per_s"] = float(f"{per_s:.4g}")
        if cnt[6]:
            pairs = cnt[6] / t
            r["pairs_per_s"] = float(f"{pairs:.4g}")
            r["equiv_12flop_tflops"] = round(12 * pairs / 1e12, 2)
            r["frac_fp32_vector_peak"] = round(12 * pairs / (PEAK_FP32_TFLOPS * 1e12), 4)
            r["simd_cycles_per_64_pairs"] = round(simd_cycles / (cnt[6] / 64), 3)
        res[name] = r
    # HBM read rate: a 1.6 GB buffer read once per launch (the few-rows workload's y and
    # b), grid-stride and one contiguous chunk per work-group, best of five launches
    lib.keops_micro_hbm.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                    ctypes.POINTER(ctypes.c_float)]
    n = 400_000_000
    buf = torch.ones(n, device="cuda:0")
    hbm = {}
    for mode, label in ((0, "grid_stride"), (1, "chunk_per_wg")):
        for blocks in (1024, 2048, 4096, 8192, 16384):
            sink = torch.empty(blocks * 256, device="cuda:0")
            best = None
            for _ in range(6):
                ms = ctypes.c_float(0)
                if lib.keops_micro_hbm(ctypes.c_void_p(buf.data_ptr()), n, ctypes.c_void_p(sink.data_ptr()),
                                       blocks, mode, ctypes.byref(ms)) != 0:
                    raise RuntimeError("keops_micro_hbm failed")
                best = ms.value if best is None else min(best, ms.value)
            hbm[f"{label}_{blocks}"] = {"ms": round(best, 4), "GB_s": round(4 * n / (best * 1e-3) / 1e9, 1)}
    res["hbm_read"] = hbm
    print(json.dumps({"workload": "micro", "cus": cus, "probes": res}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="sum", choices=sorted(BENCHES) + ["copycal", "micro"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--record-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="no GPU: write profiles/traffic_<workload>.json from rocprofv3 --pmc CSVs")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(args.workload, *args.record_traffic)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}): this engine "
              "has no multi-GPU path; the one-GPU throughput is the reported value.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.workload == "copycal":
        copy_calibration(torch, args)
        return
    if args.workload == "micro":
        micro_rates(torch)
        return

    import geometric_map_reduce_amd as gm
    from geometric_map_reduce_amd import workloads

    op, wname = BENCHES[args.workload]
    w = workloads.WORKLOADS[wname]
    x, y, b = workloads.make_inputs(w)
    ranges, kept = None, None
    if op == "sum_ranges":
        x, y, b, ranges, kept = block_sparse_setup(x, y, b, w.sigma)
    dev = torch.device("cuda:0")
    X, Y = torch.from_numpy(x).to(dev), torch.from_numpy(y).to(dev)
    B = torch.from_numpy(b).to(dev) if b is not None else None
    g = None
    G = None
    if op in ("grad_x", "grad_y", "grad_b"):
        g = np.random.default_rng(3).standard_normal((w.M, w.E)).astype(np.float32)
        G = torch.from_numpy(g).to(dev)
    if op == "kmin":
        out = (torch.empty((w.M, w.K), device=dev), torch.empty((w.M, w.K), device=dev, dtype=torch.int64))
    elif op == "cg":
        out = torch.empty((w.N, w.E), device=dev)
    elif op == "max":
        out = (torch.empty((w.M, w.E), device=dev), torch.empty((w.M, w.E), device=dev, dtype=torch.int64))
    elif op in ("grad_y", "grad_b"):
        out = torch.empty((w.N, w.D if op == "grad_y" else w.E), device=dev)
    else:
        out = torch.empty((w.M, w.D if op == "grad_x" else w.E), device=dev)

    for _ in range(args.warmup):
        run_op(gm, op, X, Y, B, G, w.sigma, w.K, out, w.lam, ranges)
    torch.cuda.synchronize()

    gm.keops_set_option(gm.KEOPS_OPT_PROFILE, 1)
    gm.keops_profile_read()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    solves = []
    for _ in range(args.steps):
        solves.append(run_op(gm, op, X, Y, B, G, w.sigma, w.K, out, w.lam, ranges))
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gm.keops_set_option(gm.KEOPS_OPT_PROFILE, 0)
    kern_ms, launches = gm.keops_profile_read()
    ms_step = ev0.elapsed_time(ev1) / args.steps

    pairs = w.M * w.N
    cg_info = None
    if op == "cg":
        # one step = one whole solve; its pair-evaluations are those of its products K p
        # (iterations + 1 for the final residual), every one N x N
        iters = solves[-1][1]
        cg_info = {"iterations": iters, "rel_residual": float(solves[-1][2].max()), "rtol": CG_RTOL,
                   "products_per_solve": iters + 1}
        pairs = (iters + 1) * w.N * w.N
    bs_info = None
    if op == "sum_ranges":
        # kept pairs only; the dense-equivalent rate is reported beside it
        bs_info = {"voxel": BS_VOXEL, "eps": BS_EPS, "kept_pairs": kept, "kept_fraction": round(kept / pairs, 4),
                   "dense_equivalent_G_pair_evals_per_s": round(pairs / (ms_step * 1e-3) / 1e9, 1)}
        pairs = kept
    value = pairs / (ms_step * 1e-3) / 1e9
    bound, fpp, kname = roofline_of(op, w.M, w.D, w.E)
    kern_avg_ms = kern_ms / max(launches, 1)
    src_key = ({"sum": "stream", "kmin": "kmin_stream"}.get(op, "stream_ops") if bound == "hbm"
               else "kmin_split" if bound == "mfma_bf16" and op == "kmin"
               else {"grad_y": "grad_x", "grad_b": "sum"}.get(op, op))
    traffic = recorded_traffic(args.workload, src_key)
    if bound == "hbm":
        achieved = stream_bytes(w, op) / (kern_avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic}
        kinfo = {"bytes_per_launch": stream_bytes(w, op)}
    else:
        per_launch = w.N * w.N if op == "cg" else pairs
        achieved = fpp * per_launch / (kern_avg_ms * 1e-3) / 1e12
        peak = PEAK_BF16_TFLOPS if bound == "mfma_bf16" else PEAK_FP32_TFLOPS
        roof = {"bound": "mfma" if bound == "mfma_bf16" else bound, "achieved": round(achieved, 3), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic}
        kinfo = {"flops_per_pair": fpp}
        if bound == "mfma_bf16":
            # what the split-bf16 prefilter executes: three bf16 products over D, 6D flops per pair
            kinfo["executed_flops_per_pair"] = 6 * w.D
            kinfo["executed_TFLOP_s"] = round(6 * w.D * per_launch / (kern_avg_ms * 1e-3) / 1e12, 3)

    res = {
        "metric": METRIC if args.workload == "sum" else f"{op} G pair-evals/s @ {w.name}",
        "value": round(value, 3),
        "unit": "G pair-evals/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / (PAGES_PAIRS_PER_S_1M / 1e9), 3) if args.workload == "sum" else None,
        "dtype": "f32",
        "data": "synthetic",
        "config": dict(w.describe(), op=op, seed=0),
        "roofline": roof,
        "kernel": dict({"name": kname, "avg_ms": round(kern_avg_ms, 4), "launches": launches}, **kinfo),
        "wall_s_timed": round(wall, 3),
    }
    if cg_info is not None:
        res["solver"] = cg_info
    if bs_info is not None:
        res["block_sparse"] = bs_info
    if not args.no_cpu_baseline:
        gpu_out = ((out[0].cpu().numpy(), out[1].cpu().numpy()) if op == "kmin"
                   else (out[0] if op == "max" else out).cpu().numpy())
        base, check = cpu_baseline(op, w, x, y, b, g, args.cpu_seconds, gpu_out, ranges)
        res["cpu_baseline"] = base
        if check is not None:
            res["check"] = check
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
