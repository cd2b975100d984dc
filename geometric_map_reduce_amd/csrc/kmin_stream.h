// kmin_stream.h -- pass-1 kernel of the K-min reduction for few rows and many j
// (KeOps pages: "Kernel Operations on the GPU, with Autodiff, without Memory
// Overflows" §2, argKmin; the Falkon issue "Transparent interface for
// billion-scale matrices": M much smaller than N).
//
// With a few dozen query rows the row-per-lane kernel leaves most lanes without a
// row.  Here lanes own j: each lane walks its j of the work-group's chunk in
// increasing order (J of them per step, loaded together), computes the exact
// direct-form fp32 distance to each of the MR rows of its row group (held in
// registers; the same arithmetic as every other K-min kernel), and keeps a sorted
// K-list per row in registers.
//
// A candidate is inserted only below a bound on the row's K-th distance over the
// wave, refreshed whenever a list changes: the least of the lanes' K-th entries
// and the K-th smallest of the lanes' first entries (in both cases K entries lie at
// or below it, all from earlier steps, so with smaller j: a candidate at or above
// it ranks after K others and cannot be among the row's K smallest by (d^2, j)).
// The test is made once per row and step on the least of the lane's J distances,
// as one wave-level branch.
//
// Merge: T = the least of two bounds on the work-group's K-th distance, the least
// K-th entry of a lane and, per wave, the K-th smallest of the lanes' first
// entries (K lanes hold an entry at or below it).  The work-group's K best entries
// all lie at or below T, and each lane contributes at most K of them, so they fit
// a 256 K buffer in LDS.  Every candidate's rank is the count of candidates before
// it in (d^2, j) order (the j are distinct); ranks below K go to their slots.  The
// partial list per row goes to the split-j pass 2, which merges the chunks.
#pragma once

#include "common.h"
#include "kmin_kernel.h"

namespace kmi {

// Rows per row group: the K-lists take MR x 2K registers.
constexpr int kmin_stream_rows(int K) { return K <= 16 ? 4 : 2; }
// j per lane per step, loaded together.
constexpr int kmin_stream_j(int D) { return D <= 4 ? 8 : 4; }

// Work-group w -> (row group, chunk).  When the chunk count is a multiple of 8,
// the row groups of one chunk get consecutive ids among those with w % 8 equal,
// which the dispatcher places on one XCD (ids go round-robin over the eight), so
// the chunk's y comes from that XCD's L2 after the first row group reads it.
__device__ __forceinline__ void kmin_stream_place(int64_t w, int64_t G, int64_t C, int64_t &rg, int64_t &c) {
  if ((C & 7) == 0) {
    const int64_t xcd = w & 7, k = w >> 3;
    rg = k % G;
    c = (k / G) * 8 + xcd;
  } else {
    rg = w % G;
    c = w / G;
  }
}

// Ascending bitonic sort of one value per lane over the 64 lanes of a wave.
__device__ __forceinline__ float wave_sort_asc(float v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int k = 2; k <= kWave; k <<= 1)
#pragma unroll
    for (int h = k >> 1; h > 0; h >>= 1) {
      const float p = __shfl_xor(v, h);
      const bool take_min = ((lane & h) == 0) == ((lane & k) == 0);
      v = take_min ? fminf(v, p) : fmaxf(v, p);
    }
  return v;
}

// LDS of the work-group merge below.
template <int K>
struct KminMergeLds {
  uint64_t cand[kThreads * K];   // (d^2 bits << 32) | j; d^2 >= +0, so key order = (d^2, j) order
  uint64_t top[K];
  float red[kThreads / kWave];
  int count;                     // 0 on entry (set before the caller's first barrier)
};

// The K smallest by (d^2, j) of the union of the threads' sorted lists (empty slots
// carry j < 0 and come last; the j of different threads are distinct), into s.top;
// returns how many the union holds (slots from there on are empty).  The bound T
// and the ranking are those described at the top of this file.  Every thread of
// the work-group calls it; s.count is 0 again after the caller's next barrier.
template <int K>
__device__ int block_kmin_merge(const float (&bd)[K], const int (&bi)[K], KminMergeLds<K> &s) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const float tw = fminf(wave_min(bd[K - 1]), __shfl(wave_sort_asc(bd[0]), K - 1));
  if (lane == 0) s.red[wid] = tw;
  __syncthreads();   // s.red written; the previous call's readers of s.cand and s.top are done
  float T = s.red[0];
#pragma unroll
  for (int w = 1; w < kThreads / kWave; ++w) T = fminf(T, s.red[w]);
  int n = 0;   // a prefix of the sorted list
#pragma unroll
  for (int q = 0; q < K; ++q) n += (bi[q] >= 0 && bd[q] <= T) ? 1 : 0;
  const int off = n > 0 ? atomicAdd(&s.count, n) : 0;
#pragma unroll
  for (int q = 0; q < K; ++q)
    if (q < n) s.cand[off + q] = ((uint64_t)__float_as_uint(bd[q]) << 32) | (uint32_t)bi[q];
  __syncthreads();
  const int nc = s.count;
  for (int t = tid; t < nc; t += kThreads) {
    const uint64_t key = s.cand[t];
    int rank = 0;
    for (int u = 0; u < nc; ++u) rank += s.cand[u] < key ? 1 : 0;
    if (rank < K) s.top[rank] = key;
  }
  __syncthreads();
  if (tid == 0) s.count = 0;   // every thread read it before the barrier above
  return nc;
}

template <int D, int K, int MR>
__global__ __launch_bounds__(kThreads) void kmin_stream_kernel(KminArgs a) {
  constexpr int J = kmin_stream_j(D);
  __shared__ float sRow[MR * D];
  __shared__ KminMergeLds<K> sm;

  const int tid = threadIdx.x;
  const int64_t M = a.M, N = a.N;
  const int64_t G = (M + MR - 1) / MR;
  int64_t rg, c;
  kmin_stream_place(blockIdx.x, G, a.nsplit, rg, c);
  const int64_t r0 = rg * MR;
  const int nr = (int)((M - r0) < MR ? (M - r0) : MR);   // >= 1 by the grid
  for (int f = tid; f < MR * D; f += kThreads) {
    const int i = f / D;
    sRow[f] = i < nr ? a.x[(r0 + i) * D + (f - i * D)] : 0.0f;
  }
  if (tid == 0) sm.count = 0;
  __syncthreads();
  float xr[MR][D];
#pragma unroll
  for (int r = 0; r < MR; ++r)
#pragma unroll
    for (int k = 0; k < D; ++k) xr[r][k] = sRow[r * D + k];

  float bd[MR][K];
  int bi[MR][K];
#pragma unroll
  for (int r = 0; r < MR; ++r)
#pragma unroll
    for (int k = 0; k < K; ++k) { bd[r][k] = INFINITY; bi[r][k] = -1; }
  float thr[MR];   // the least of the wave's K-th distances per row
#pragma unroll
  for (int r = 0; r < MR; ++r) thr[r] = INFINITY;

  const int64_t jb = c * a.j_per_split;
  const int64_t je = (jb + a.j_per_split < N) ? jb + a.j_per_split : N;
  // The trip count is the same for every lane (the wave-wide minima need them all).
  // A step's J loads are issued together; past je the chunk's last j is read again
  // (always in bounds) and its distance set to +inf.  (Carrying the next step's y
  // in a second register set ran slower at every shape tried: it needs J = 4 to
  // keep three waves per SIMD.)
  for (int64_t j0 = jb; j0 < je; j0 += (int64_t)kThreads * J) {
    const bool full = j0 + (int64_t)kThreads * J <= je;   // uniform
    float y[J][D];
#pragma unroll
    for (int u = 0; u < J; ++u) {
      const int64_t j = j0 + tid + (int64_t)u * kThreads;
      const int64_t jc = j < je ? j : je - 1;
#pragma unroll
      for (int k = 0; k < D; ++k) y[u][k] = a.y[jc * D + k];
    }
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      if (r < nr) {   // uniform
        float d2[J];
#pragma unroll
        for (int u = 0; u < J; ++u) {
          d2[u] = 0.0f;
#pragma unroll
          for (int k = 0; k < D; ++k) {
            const float d = xr[r][k] - y[u][k];
            d2[u] = fmaf(d, d, d2[u]);
          }
        }
        if (!full) {
#pragma unroll
          for (int u = 0; u < J; ++u)
            if (j0 + tid + (int64_t)u * kThreads >= je) d2[u] = INFINITY;
        }
        // one wave-level test per row and step: the scalar unit, shared by the CU's
        // four SIMDs, sees a branch per J pairs instead of one per pair
        const float lim = fminf(thr[r], bd[r][K - 1]);
        float mn = d2[0];
#pragma unroll
        for (int u = 1; u < J; ++u) mn = fminf(mn, d2[u]);
        if (__any(mn < lim)) {
#pragma unroll
          for (int u = 0; u < J; ++u)
            if (d2[u] < lim) kmin_insert<K>(bd[r], bi[r], d2[u], (int)(j0 + tid + (int64_t)u * kThreads));
          // the lists changed: refresh the bound (every lane is active here)
          thr[r] = fminf(thr[r], fminf(wave_min(bd[r][K - 1]), __shfl(wave_sort_asc(bd[r][0]), K - 1)));
        }
      }
    }
  }

  // ---- merge, one row at a time
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    if (r >= nr) break;   // uniform
    const int nc = block_kmin_merge<K>(bd[r], bi[r], sm);
    if (tid < K) {
      const int64_t base = (c * M + r0 + r) * K + tid;
      const bool has = tid < nc;
      const uint64_t key = has ? sm.top[tid] : 0;
      a.out_d[base] = has ? __uint_as_float((uint32_t)(key >> 32)) : INFINITY;
      a.part_idx[base] = has ? (int32_t)(uint32_t)key : -1;
    }
  }
}

// Pass 2 for few rows: one work-group per row; thread t merges the partial lists of
// chunks t, t + 256, ... by (d^2, j), then the work-group merge picks the K best.
// Empty slots come out as (+inf, -1).
template <int K>
__global__ __launch_bounds__(kThreads) void kmin_stream_combine_kernel(const float *__restrict__ pd,
                                                                       const int32_t *__restrict__ pi, int nsplit,
                                                                       int64_t M, float *__restrict__ out_d,
                                                                       int64_t *__restrict__ out_i) {
  __shared__ KminMergeLds<K> sm;
  const int64_t i = blockIdx.x;
  if (threadIdx.x == 0) sm.count = 0;   // the merge's first barrier comes before any use
  float bd[K];
  int bi[K];
#pragma unroll
  for (int q = 0; q < K; ++q) { bd[q] = INFINITY; bi[q] = -1; }
  for (int sp = threadIdx.x; sp < nsplit; sp += kThreads) {
    const int64_t base = ((int64_t)sp * M + i) * K;
    for (int q = 0; q < K; ++q) {
      const int j = pi[base + q];
      const float v = pd[base + q];
      // the rest of this sorted list is empty, or ranks after the K kept entries
      if (j < 0 || (bi[K - 1] >= 0 && (v > bd[K - 1] || (v == bd[K - 1] && j > bi[K - 1])))) break;
      kmin_insert_lex<K>(bd, bi, v, j);
    }
  }
  const int nc = block_kmin_merge<K>(bd, bi, sm);
  if (threadIdx.x < K) {
    const int q = threadIdx.x;
    const bool has = q < nc;
    const uint64_t key = has ? sm.top[q] : 0;
    out_d[i * K + q] = has ? __uint_as_float((uint32_t)(key >> 32)) : INFINITY;
    out_i[i * K + q] = has ? (int64_t)(uint32_t)key : -1;
  }
}

template <int D, int K>
void launch_kmin_stream_t(dim3 grid, const KminArgs &a, hipStream_t st) {
  hipLaunchKernelGGL((kmin_stream_kernel<D, K, kmin_stream_rows(K)>), grid, dim3(kThreads), 0, st, a);
}

}  // namespace kmi
