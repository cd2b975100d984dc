// kmin_kernel.h -- pass-1 kernel of the K-min reduction with indices on
// gfx950 VALU (KeOps pages: "Kernel Operations on the GPU, with Autodiff,
// without Memory Overflows" §2, argmin / argKmin; KeOps README feature list,
// "ArgMin ... or K-min reductions").
//
// Each lane keeps, for each of its R rows, a sorted register list of the K
// best (d^2, j) pairs.  The pair loop has two stages:
//   1. prefilter in the expanded form u = |y_c|^2 - 2<x_c, y_c> = d^2 - |x_c|^2
//      (centred coordinates, three FMAs at D = 3), compared against the
//      current K-th distance plus a bound on the rounding error of u;
//   2. only for candidates that pass: the exact direct-form fp32 distance
//      sum_k (x_k - y_k)^2 from raw coordinates, and insertion when it beats
//      the K-th entry.  Insertion is a branch-free shift network over K.
// The filter never rejects a pair whose direct distance would be inserted
// (the margin bounds the rounding of both forms), so the result is exactly
// that of a direct-form K-min in fp32.  Ties keep the smaller j first: j
// increases within a split and the insertion test is strict.
#pragma once

#include "common.h"

namespace kmi {

template <int D, int K>
struct KminShape {
  static constexpr int NV = (D + 1 + 3) / 4;   // centred y and |y_c|^2
  static constexpr int NR = (D + 3) / 4;       // raw y
  static constexpr int BYTES_PER_J = (NV + NR) * 16;
  static constexpr int TJ = (2 * 256 * BYTES_PER_J <= 49152) ? 256
                          : (2 * 128 * BYTES_PER_J <= 49152) ? 128
                          : (2 * 64 * BYTES_PER_J <= 49152) ? 64 : 32;
  // rows per lane: the most (up to 4) that keep the kernel within 128 VGPRs, i.e.
  // four waves per SIMD.  The register model 30 + R (2K + 3D + 8) follows the
  // compiled counts (e.g. D = 3, K = 10: 66 / 102 / 132 VGPRs for R = 1 / 2 / 3);
  // at that shape R = 2 (4 waves) ran 8 % faster than R = 3 (3 waves) and 11 %
  // faster than R = 1 (7 waves).
  static constexpr int R0 = (124 - 30) / (2 * K + 3 * D + 8);
  static constexpr int R = R0 < 1 ? 1 : (R0 > 4 ? 4 : R0);
};

// Rounding-error bound of the prefilter, as a multiple of (|x_c| + |y_c|)^2.
__device__ __forceinline__ float kmin_margin_coef(int D) { return (4.0f * D + 32.0f) * 5.9604645e-8f; }

template <int K>
__device__ __forceinline__ void kmin_insert(float (&bd)[K], int (&bi)[K], float v, int j) {
  // new list = first K of (old list with (v, j) inserted after every entry <= v);
  // pure selects, no branches
#pragma unroll
  for (int k = K - 1; k > 0; --k) {
    const bool shift = v < bd[k - 1];
    const bool here = v < bd[k];
    const float nd = shift ? bd[k - 1] : (here ? v : bd[k]);
    const int ni = shift ? bi[k - 1] : (here ? j : bi[k]);
    bd[k] = nd;
    bi[k] = ni;
  }
  const bool first = v < bd[0];
  bd[0] = first ? v : bd[0];
  bi[0] = first ? j : bi[0];
}

// Insertion by (d, j) lexicographic order into a sorted list whose empty slots
// carry j < 0 and rank last; an entry with j < 0 is not inserted.  Used to merge
// lists built over disjoint j sets.  Pure selects over bitwise boolean logic (a
// short-circuit formulation of the K = 1 case was lowered with the partner's
// values lost on this toolchain).
template <int K>
__device__ __forceinline__ void kmin_insert_lex(float (&bd)[K], int (&bi)[K], float v, int j) {
  const bool invalid = j < 0;   // ranks after every slot, so nothing moves
  bool before[K];
#pragma unroll
  for (int k = 0; k < K; ++k)
    before[k] = invalid | ((bi[k] >= 0) & ((bd[k] < v) | ((bd[k] == v) & (bi[k] < j))));
#pragma unroll
  for (int k = K - 1; k > 0; --k) {
    const float nd = !before[k - 1] ? bd[k - 1] : (!before[k] ? v : bd[k]);
    const int ni = !before[k - 1] ? bi[k - 1] : (!before[k] ? j : bi[k]);
    bd[k] = nd;
    bi[k] = ni;
  }
  bd[0] = before[0] ? bd[0] : v;
  bi[0] = before[0] ? bi[0] : j;
}

template <int D, int K, int R>
__global__ __launch_bounds__(kThreads) void kmin_valu_kernel(KminArgs a) {
  using S = KminShape<D, K>;
  constexpr int NV = S::NV, NR = S::NR, TJ = S::TJ;
  __shared__ float4 sRec[2][TJ * NV];
  __shared__ float4 sRaw[2][TJ * NR];
  __shared__ float sRed[2 * D * (kThreads / kWave) + 8];

  const int tid = threadIdx.x;
  const int wid = tid / kWave, lane = tid & (kWave - 1);
  const int64_t row0 = (int64_t)blockIdx.x * (kThreads * R);
  const int64_t M = a.M, N = a.N;

  float xr[R][D];
  bool valid[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t i = row0 + (int64_t)r * kThreads + tid;
    valid[r] = i < M;
#pragma unroll
    for (int k = 0; k < D; ++k) xr[r][k] = valid[r] ? a.x[i * D + k] : 0.0f;
  }
  float cen[D];
  {
    float lo[D], hi[D];
#pragma unroll
    for (int k = 0; k < D; ++k) {
      lo[k] = INFINITY;
      hi[k] = -INFINITY;
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (valid[r] && isfinite(xr[r][k])) { lo[k] = fminf(lo[k], xr[r][k]); hi[k] = fmaxf(hi[k], xr[r][k]); }
      lo[k] = wave_min(lo[k]);
      hi[k] = wave_max(hi[k]);
    }
    if (lane == 0) {
#pragma unroll
      for (int k = 0; k < D; ++k) { sRed[(2 * k) * 4 + wid] = lo[k]; sRed[(2 * k + 1) * 4 + wid] = hi[k]; }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < D; ++k) {
      float l = sRed[(2 * k) * 4], h = sRed[(2 * k + 1) * 4];
#pragma unroll
      for (int w = 1; w < kThreads / kWave; ++w) {
        l = fminf(l, sRed[(2 * k) * 4 + w]);
        h = fmaxf(h, sRed[(2 * k + 1) * 4 + w]);
      }
      // finite coordinates only (an infinite one would make every row's centred
      // coordinates infinite); 0 where the work-group has none
      cen[k] = l <= h ? 0.5f * l + 0.5f * h : 0.0f;
    }
  }
  // -2 * centred coordinates, |x_c|^2, |x_c|
  float xm[R][D], nx[R], ax[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float n = 0.0f;
#pragma unroll
    for (int k = 0; k < D; ++k) {
      const float c = xr[r][k] - cen[k];
      xm[r][k] = -2.0f * c;
      n = fmaf(c, c, n);
    }
    nx[r] = n;
    ax[r] = sqrtf(n);
  }
  const float mcoef = kmin_margin_coef(D);

  float bd[R][K];
  int bi[R][K];
  float thr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    thr[r] = INFINITY;
#pragma unroll
    for (int k = 0; k < K; ++k) { bd[r][k] = INFINITY; bi[r][k] = -1; }
  }

  const int64_t jb = (int64_t)blockIdx.y * a.j_per_split;
  const int64_t je = (jb + a.j_per_split < N) ? jb + a.j_per_split : N;

  float ry[D];
  auto load_raw = [&](int64_t jt) {
    const int64_t j = jt + tid;
    const bool ok = (tid < TJ) && (j < je);
#pragma unroll
    for (int k = 0; k < D; ++k) ry[k] = ok ? a.y[j * D + k] : 0.0f;
    return ok;
  };
  auto stage = [&](int buf, bool ok) {
    if (tid >= TJ) return;
    float rec[4 * NV], raw[4 * NR];
    float ny = 0.0f;
#pragma unroll
    for (int q = 0; q < 4 * NV; ++q) rec[q] = 0.0f;
#pragma unroll
    for (int q = 0; q < 4 * NR; ++q) raw[q] = 0.0f;
#pragma unroll
    for (int k = 0; k < D; ++k) {
      const float c = ry[k] - cen[k];
      rec[k] = c;
      ny = fmaf(c, c, ny);
      raw[k] = ry[k];
    }
    rec[D] = ok ? ny : INFINITY;   // padded j: u = +inf never passes the filter
#pragma unroll
    for (int v = 0; v < NV; ++v)
      sRec[buf][tid * NV + v] = make_float4(rec[4 * v], rec[4 * v + 1], rec[4 * v + 2], rec[4 * v + 3]);
#pragma unroll
    for (int v = 0; v < NR; ++v)
      sRaw[buf][tid * NR + v] = make_float4(raw[4 * v], raw[4 * v + 1], raw[4 * v + 2], raw[4 * v + 3]);
  };

  if (jb < je) {
    bool ok = load_raw(jb);
    stage(0, ok);
  }
  __syncthreads();
  int buf = 0;
  for (int64_t jt = jb; jt < je; jt += TJ) {
    const bool has_next = jt + TJ < je;
    bool ok_next = false;
    if (has_next) ok_next = load_raw(jt + TJ);
    const int cnt = (int)(((je - jt < TJ ? je - jt : TJ) + 3) & ~3);
    const float4 *rec = sRec[buf];
    const float4 *raw = sRaw[buf];
    // Records of a group of 4 j live in registers: two buffers, each read from
    // LDS one group ahead of its use (wrapping inside the tile past its end, where
    // the values are never used).
    auto read_group = [&](float4 (&g)[4][NV], int jj) {
      const int jw = jj & (TJ - 1);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < NV; ++v) g[u][v] = rec[(jw + u) * NV + v];
    };
    // Filter 4 j x R rows; one wave-level branch for the whole group.  Per row the
    // least of the 4 prefilter values (v_min3 + v_min) is compared once, and the
    // lane masks are ORed in scalar registers: the CU's one scalar unit, shared by
    // its four SIMDs, sees one OR per row per group instead of one per pair.
    auto filter_group = [&](auto &&fetch, int jj) {
      float t[4][R];
      uint64_t hit = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float yv[4 * NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const float4 q = fetch(u, v);
          yv[4 * v] = q.x; yv[4 * v + 1] = q.y; yv[4 * v + 2] = q.z; yv[4 * v + 3] = q.w;
        }
#pragma unroll
        for (int r = 0; r < R; ++r) t[u][r] = yv[D];
#pragma unroll
        for (int k = 0; k < D; ++k)
#pragma unroll
          for (int r = 0; r < R; ++r) t[u][r] = fmaf(xm[r][k], yv[k], t[u][r]);
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        // NaN values drop out of fminf, as they fail the compare
        const float lo = fminf(fminf(t[0][r], t[1][r]), fminf(t[2][r], t[3][r]));
        hit |= __builtin_amdgcn_ballot_w64(lo < thr[r]);
      }
      if (hit) {   // wave-uniform
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
          for (int r = 0; r < R; ++r) {
            // compare again here (an opaque copy of t): keeping the loop's compare
            // results alive across the branch costs more VALU work than redoing it
            float tt = t[u][r];
            asm volatile("" : "+v"(tt));
            if (tt < thr[r]) {
              float yr[4 * NR];
#pragma unroll
              for (int v = 0; v < NR; ++v) {
                const float4 q = raw[(jj + u) * NR + v];
                yr[4 * v] = q.x; yr[4 * v + 1] = q.y; yr[4 * v + 2] = q.z; yr[4 * v + 3] = q.w;
              }
              float d2 = 0.0f;
#pragma unroll
              for (int k = 0; k < D; ++k) { const float d = xr[r][k] - yr[k]; d2 = fmaf(d, d, d2); }
              if (d2 < bd[r][K - 1]) {
                kmin_insert<K>(bd[r], bi[r], d2, (int)(jt + jj + u));
                const float kth = bd[r][K - 1];
                const float s = 2.0f * ax[r] + sqrtf(kth);
                thr[r] = (kth - nx[r]) + mcoef * s * s;   // +inf while the list is not full
              }
            }
          }
        }
      }
    };
    if constexpr (NV > 4) {
      // records of D > 15: read from LDS where they are used (two register buffers of
      // four such records spilled hundreds of registers at D = 50)
      for (int jj = 0; jj < cnt; jj += 4)
        filter_group([&](int u, int v) { return rec[(jj + u) * NV + v]; }, jj);
    } else {
      float4 ga[4][NV], gb[4][NV];
      read_group(ga, 0);
      for (int jj = 0; jj < cnt; jj += 8) {
        read_group(gb, jj + 4);
        filter_group([&](int u, int v) { return ga[u][v]; }, jj);
        if (jj + 4 < cnt) {   // wave-uniform
          read_group(ga, jj + 8);
          filter_group([&](int u, int v) { return gb[u][v]; }, jj + 4);
        }
      }
    }
    if (has_next) stage(buf ^ 1, ok_next);
    __syncthreads();
    buf ^= 1;
  }

  const bool partial = a.nsplit > 1;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (!valid[r]) continue;
    const int64_t i = row0 + (int64_t)r * kThreads + tid;
    if (partial) {
      const int64_t base = ((int64_t)blockIdx.y * M + i) * K;
#pragma unroll
      for (int k = 0; k < K; ++k) { a.out_d[base + k] = bd[r][k]; a.part_idx[base + k] = bi[r][k]; }
    } else {
#pragma unroll
      for (int k = 0; k < K; ++k) { a.out_d[i * K + k] = bd[r][k]; a.out_idx[i * K + k] = (int64_t)bi[r][k]; }
    }
  }
}

template <int D, int K>
void launch_kmin_t(dim3 grid, const KminArgs &a, hipStream_t st) {
  hipLaunchKernelGGL((kmin_valu_kernel<D, K, KminShape<D, K>::R>), grid, dim3(kThreads), 0, st, a);
}

}  // namespace kmi
