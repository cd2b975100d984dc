// kmin_mfma.h -- pass-1 kernel of the K-min reduction for D >= 32 on gfx950
// fp32 matrix cores (KeOps pages: "Kernel Operations on the GPU, with
// Autodiff, without Memory Overflows" §2, argKmin; KeOps README feature list,
// "K-min reductions").
//
// Prefilter on MFMA, decision on the VALU, as in the VALU K-min kernel:
//   u_ij = |y_c|^2 - 2<x_c, y_c> = |x_i - y_j|^2 - |x_c|^2      (c: work-group centre)
// is the contraction <y~_j, x~_i> with y~ = (y_c, |y_c|^2, 0...) and
// x~ = (-2x_c, 1, 0...).  One v_mfma_f32_16x16x4f32 step takes the 16-column
// j tile as its A operand (read from LDS) and a 16-row i tile as its B operand
// (kept in VGPRs), so output lane l holds four candidates j = 4*(l/16) + r of
// the single row i = l%16.  A candidate passes when u is below the row's K-th
// distance minus |x_c|^2 plus a bound on the rounding of both forms; only then
// is the exact direct-form fp32 distance sum_k (x_k - y_k)^2 formed (raw
// coordinates, from global memory) and inserted into the lane's sorted
// register list.  The four lanes that share a row see disjoint j's and share
// the least of their thresholds; their lists are merged with cross-lane
// exchanges at the end.  The result is that of a
// direct-form K-min in fp32, for any spread of the data.
#pragma once

#include "common.h"
#include "kmin_kernel.h"

namespace kmi {

typedef float floatx4 __attribute__((ext_vector_type(4)));

// 16-row tiles per wave: three where the kernel still fits in 256 VGPRs (two
// waves per SIMD; the LDS tiles allow no more than three work-groups per CU),
// else two.  A third tile reuses each A operand once more and gives the
// matrix core a third independent accumulation chain.
constexpr int kmin_mfma_tiles(int D, int K) { return K <= (D <= 50 ? 13 : (D <= 64 ? 12 : 8)) ? 3 : 2; }

template <int D, int K>
struct KminMfmaShape {
  static constexpr int DP = (D + 1 + 3) / 4 * 4;
  static constexpr int KS = DP / 4;
  static constexpr int KSP = (KS + 3) / 4 * 4;
  static constexpr int JSTRIDE = 4 * KSP + 4;
  static constexpr int TJ = 64;                    // j rows per LDS tile
  static constexpr int TI = kmin_mfma_tiles(D, K);
  static constexpr int ROWS_WG = 4 * 16 * TI;      // rows per work-group
};

template <int D, int K>
__global__ __launch_bounds__(kThreads) void kmin_mfma_kernel(KminArgs a) {
  using S = KminMfmaShape<D, K>;
  constexpr int KS = S::KS, KSP = S::KSP, JS = S::JSTRIDE, TJ = S::TJ, TI = S::TI;
  static_assert(S::ROWS_WG <= kThreads, "one thread per row for the centre");
  __shared__ __attribute__((aligned(16))) float sMem[2 * TJ * JS];   // double-buffered y~ tiles
  __shared__ float sRed[2 * D * (kThreads / kWave) + 8];
  __shared__ float sCen[D];

  const int tid = threadIdx.x;
  const int wid = tid / kWave, lane = tid & (kWave - 1);
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int64_t M = a.M, N = a.N;
  const int64_t wg_row0 = (int64_t)blockIdx.x * S::ROWS_WG;

  // ---- work-group bounding-box centre
  {
    const int64_t i = wg_row0 + tid;
    const bool ok = tid < S::ROWS_WG && i < M;
    for (int d0 = 0; d0 < D; d0 += 4) {
      float lo[4], hi[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d = d0 + q;
        const float v = (ok && d < D) ? a.x[i * D + d] : 0.0f;
        // finite coordinates only: an infinite one would put the centre at infinity
        lo[q] = wave_min((ok && d < D && isfinite(v)) ? v : INFINITY);
        hi[q] = wave_max((ok && d < D && isfinite(v)) ? v : -INFINITY);
      }
      if (lane == 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (d0 + q < D) { sRed[(2 * (d0 + q)) * 4 + wid] = lo[q]; sRed[(2 * (d0 + q) + 1) * 4 + wid] = hi[q]; }
      }
    }
    __syncthreads();
    for (int d = tid; d < D; d += kThreads) {
      float l = sRed[(2 * d) * 4], h = sRed[(2 * d + 1) * 4];
#pragma unroll
      for (int w = 1; w < kThreads / kWave; ++w) { l = fminf(l, sRed[(2 * d) * 4 + w]); h = fmaxf(h, sRed[(2 * d + 1) * 4 + w]); }
      sCen[d] = l <= h ? 0.5f * l + 0.5f * h : 0.0f;   // 0 where no row is finite
    }
    __syncthreads();
  }

  // ---- B operands x~ (row t*16 + l%16, k = 4s + l/16), |x_c|^2 and |x_c| per row
  float xb[TI][KS];
  float nx[TI], ax[TI];
  int64_t row[TI];
#pragma unroll
  for (int t = 0; t < TI; ++t) {
    row[t] = wg_row0 + wid * (16 * TI) + t * 16 + lrow;
    const bool ok = row[t] < M;
    float n = 0.0f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int k = 4 * s + lgrp;
      float v = 0.0f;
      if (k < D) {
        const float c = ok ? a.x[row[t] * D + k] - sCen[k] : 0.0f;
        n = fmaf(c, c, n);
        v = -2.0f * c;
      } else if (k == D) {
        v = 1.0f;
      }
      xb[t][s] = v;
    }
    n += __shfl_xor(n, 16);
    n += __shfl_xor(n, 32);
    nx[t] = n;
    ax[t] = sqrtf(n);
  }
  const float mcoef = kmin_margin_coef(D);

  // Prefilter thresholds stay below kPadU, the value padded j carry, so padding
  // never passes; rows beyond M get -inf and never pass either.
  constexpr float kPadU = 1.0e30f, kThrCap = 5.0e29f;
  float bd[TI][K];
  int bi[TI][K];
  float thr[TI];
#pragma unroll
  for (int t = 0; t < TI; ++t) {
    thr[t] = row[t] < M ? kThrCap : -INFINITY;
#pragma unroll
    for (int k = 0; k < K; ++k) { bd[t][k] = INFINITY; bi[t][k] = -1; }
  }

  const int64_t jb = (int64_t)blockIdx.y * a.j_per_split;
  const int64_t je = (jb + a.j_per_split < N) ? jb + a.j_per_split : N;

  // tile staging: thread (jl = tid/4, g = tid%4) owns k-group g of column jl
  static_assert(TJ * 4 == kThreads, "one k-group per thread");
  const int sj = tid >> 2, sg = tid & 3;
  float ry[KSP];
  auto load_tile = [&](int64_t jt) {
    const int64_t j = jt + sj;
    const bool ok = j < je;
#pragma unroll
    for (int q = 0; q < KSP; ++q) {
      const int k = 4 * q + sg;
      ry[q] = (ok && k < D) ? a.y[j * D + k] : 0.0f;
    }
  };
  auto stage_tile = [&](int buf, int64_t jt) {
    const bool ok = jt + sj < je;
    float v[KSP];
    float ny = 0.0f;
#pragma unroll
    for (int q = 0; q < KSP; ++q) {
      const int k = 4 * q + sg;
      if (k < D) {
        v[q] = ry[q] - sCen[k];
        ny = fmaf(v[q], v[q], ny);
      } else {
        v[q] = 0.0f;
      }
    }
    ny += __shfl_xor(ny, 1);
    ny += __shfl_xor(ny, 2);
    if (sg == (D & 3)) v[D >> 2] = ok ? ny : kPadU;   // padded j: u ~ kPadU, never passes
    float4 *dst = reinterpret_cast<float4 *>(sMem + buf * TJ * JS + sj * JS + sg * KSP);
#pragma unroll
    for (int q = 0; q < KSP / 4; ++q) dst[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  };

  if (jb < je) {
    load_tile(jb);
    stage_tile(0, jb);
  }
  __syncthreads();
  int buf = 0;
  for (int64_t jt = jb; jt < je; jt += TJ) {
    const bool has_next = jt + TJ < je;
    if (has_next) load_tile(jt + TJ);
    const int cnt = (int)(je - jt < TJ ? je - jt : TJ);
    const float *yt = sMem + buf * TJ * JS;
    for (int j16 = 0; j16 < cnt; j16 += 16) {
      float ya[KSP];
      const float4 *src = reinterpret_cast<const float4 *>(yt + (j16 + lrow) * JS + lgrp * KSP);
#pragma unroll
      for (int v = 0; v < KSP / 4; ++v) {
        const float4 q = src[v];
        ya[4 * v] = q.x; ya[4 * v + 1] = q.y; ya[4 * v + 2] = q.z; ya[4 * v + 3] = q.w;
      }
      floatx4 u[TI];
#pragma unroll
      for (int t = 0; t < TI; ++t) u[t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int t = 0; t < TI; ++t) u[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(ya[s], xb[t][s], u[t], 0, 0, 0);
      // one wave-uniform branch for the 4 x TI candidates of every lane
      float lowest = INFINITY;
#pragma unroll
      for (int t = 0; t < TI; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) lowest = fminf(lowest, u[t][r] - thr[t]);
      if (__builtin_amdgcn_ballot_w64(lowest < 0.0f)) {
#pragma unroll
        for (int t = 0; t < TI; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int64_t j = jt + j16 + 4 * lgrp + r;
            if (u[t][r] < thr[t] && j < je && row[t] < M) {
              const float *xi = a.x + row[t] * D;
              const float *yj = a.y + j * D;
              float d2 = 0.0f;
              for (int k = 0; k < D; ++k) { const float d = xi[k] - yj[k]; d2 = fmaf(d, d, d2); }
              if (d2 < bd[t][K - 1]) {
                kmin_insert<K>(bd[t], bi[t], d2, (int)j);
                const float kth = bd[t][K - 1];
                const float sm = 2.0f * ax[t] + sqrtf(kth);
                thr[t] = fminf(thr[t], fminf((kth - nx[t]) + mcoef * sm * sm, kThrCap));   // keep a tighter shared bound
              }
            }
          }
        // The four lane groups of a row see disjoint j, and each group's
        // threshold bounds its own K-th distance.  A candidate that fails the
        // least of the four trails K candidates of that group, so it cannot
        // be among the row's K smallest: the groups share the least threshold.
        // Tighter still: every group's Q-th smallest distance (Q = ceil(K/4))
        // is at most their largest, so the four lists hold 4Q >= K distances no
        // larger than it, and a candidate beyond it cannot reach the row's final
        // K smallest (the final merge of the four lists decides the result).
        // (All lanes run this: the branch above is wave-uniform.)
        constexpr int Q = (K + 3) / 4;
#pragma unroll
        for (int t = 0; t < TI; ++t) {
          thr[t] = fminf(thr[t], __shfl_xor(thr[t], 16));
          thr[t] = fminf(thr[t], __shfl_xor(thr[t], 32));
          float q = bd[t][Q - 1];
          q = fmaxf(q, __shfl_xor(q, 16));
          q = fmaxf(q, __shfl_xor(q, 32));
          if (q < INFINITY) {
            const float sm = 2.0f * ax[t] + sqrtf(q);
            thr[t] = fminf(thr[t], (q - nx[t]) + mcoef * sm * sm);
          }
        }
      }
    }
    if (has_next) stage_tile(buf ^ 1, jt + TJ);
    __syncthreads();
    buf ^= 1;
  }

  // ---- merge the four lane groups' lists of each row (lanes l, l^16, l^32, l^48):
  // exchange with the partner group and insert its entries, twice; the exchange
  // is symmetric, so after the two steps every group holds the row's full list.
  for (int step = 0; step < 2; ++step) {
    const int off = step == 0 ? 16 : 32;
#pragma unroll
    for (int t = 0; t < TI; ++t) {
      float pd[K];
      int pi[K];
#pragma unroll
      for (int q = 0; q < K; ++q) { pd[q] = __shfl_xor(bd[t][q], off); pi[q] = __shfl_xor(bi[t][q], off); }
#pragma unroll
      for (int q = 0; q < K; ++q) kmin_insert_lex<K>(bd[t], bi[t], pd[q], pi[q]);
    }
  }
  if (lgrp == 0) {
    const bool partial = a.nsplit > 1;
#pragma unroll
    for (int t = 0; t < TI; ++t) {
      if (row[t] >= M) continue;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        if (partial) {
          const int64_t base = ((int64_t)blockIdx.y * M + row[t]) * K;
          a.out_d[base + k] = bd[t][k];
          a.part_idx[base + k] = bi[t][k];
        } else {
          a.out_d[row[t] * K + k] = bd[t][k];
          a.out_idx[row[t] * K + k] = (int64_t)bi[t][k];
        }
      }
    }
  }
}

template <int D, int K>
void launch_kmin_mfma_t(dim3 grid, const KminArgs &a, hipStream_t st) {
  hipLaunchKernelGGL((kmin_mfma_kernel<D, K>), grid, dim3(kThreads), 0, st, a);
}

}  // namespace kmi
