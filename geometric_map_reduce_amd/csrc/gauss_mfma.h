// gauss_mfma.h -- pass-1 kernel of the Gaussian sum for D >= 32 on gfx950
// fp32 matrix cores (KeOps pages: "Kernel Operations on the GPU, with
// Autodiff, without Memory Overflows" §1 "Target operation"; §4 names
// tensor-core support as future work -- here the cross term <x, y> of a
// large-D distance is a real dense contraction and runs on MFMA).
//
// With x' = s(x - c), y' = s(y - c) (s = sqrt(log2 e)/sigma, c the
// work-group's bounding-box centre) the exponent of K_ij in log2 units is
//   -|x'_i - y'_j|^2 = <x~_i, y~_j> - |x'_i|^2,
//   x~_i = (2x'_i, 1, 0...),  y~_j = (y'_j, -|y'_j|^2, 0...),
// a K = D+1 contraction (padded to a multiple of 4).  One
// v_mfma_f32_16x16x4f32 step multiplies a 16-row tile of x~ (A operand, kept
// in VGPRs for the whole j loop) by a 16-column tile of y~ (B operand, read
// from LDS); its C input is a fixed register set holding -|x'_i|^2, so the
// MFMA output is the exponent itself.  The VALU then evaluates one v_exp_f32
// and E FMAs per pair.  Output layout of the 16x16 tile: lane l holds rows
// 4*(l/16) + r (r < 4) of column l%16, so each lane accumulates 4 rows over
// the columns l%16 (mod 16) and a 16-lane DPP reduction merges them at the
// end.
//
// Work-group: 256 threads = 4 waves; each wave owns 4 row tiles (64 rows),
// i.e. 256 rows per work-group; four independent MFMA chains per wave.
// j tiles of TJ = 64 rows are staged in LDS (double-buffered, one barrier per
// tile) in a permuted y~ layout that lets each lane read its k-slice with
// ds_read_b128; all 256 threads build it, four per column.
//
// Precision condition as for the VALU expanded form: max |x'_i|^2 <= kFastR2
// over the work-group.  A work-group beyond it records so in wg_flags and
// returns; the direct-form VALU kernel, launched next on the same stream with
// the same 256-row work-groups, computes exactly those work-groups.
#pragma once

#include "common.h"

namespace kmi {

typedef float floatx4 __attribute__((ext_vector_type(4)));

template <int D>
struct MfmaShape {
  static constexpr int DP = (D + 1 + 3) / 4 * 4;   // contraction length (x~, y~)
  static constexpr int KS = DP / 4;                // MFMA k-steps
  static constexpr int KSP = (KS + 3) / 4 * 4;     // k-slice per lane group, padded for b128 reads
  static constexpr int JSTRIDE = 4 * KSP + 4;      // floats per j in LDS (+4: no bank conflicts)
  static constexpr int TJ = 64;                    // j rows per LDS tile
  static constexpr int TI = 4;                     // 16-row tiles per wave
  static constexpr int ROWS_WG = 4 * 16 * TI;      // rows per work-group
};

template <int D, int E>
__global__ __launch_bounds__(kThreads) void gauss_mfma_sum_kernel(GaussArgs a) {
  using S = MfmaShape<D>;
  constexpr int KS = S::KS, KSP = S::KSP, JS = S::JSTRIDE, TJ = S::TJ, TI = S::TI;
  __shared__ __attribute__((aligned(16))) float sY[2][TJ * JS];   // permuted y~, double-buffered
  __shared__ float sB[2][E * TJ];                                // b of the tile, [e][j]
  __shared__ float sRed[2 * D * (kThreads / kWave) + 8];
  __shared__ float sCen[D];

  const int tid = threadIdx.x;
  const int wid = tid / kWave, lane = tid & (kWave - 1);
  const int64_t M = a.M, N = a.N;
  const int64_t wg_row0 = (int64_t)blockIdx.x * S::ROWS_WG;

  // ---- work-group bounding-box centre: thread t scans row wg_row0 + t in chunks
  {
    const int64_t i = wg_row0 + tid;
    const bool ok = i < M;
    for (int d0 = 0; d0 < D; d0 += 4) {
      float lo[4], hi[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d = d0 + q;
        const float v = (ok && d < D) ? a.x[i * D + d] : 0.0f;
        lo[q] = (ok && d < D) ? v : INFINITY;
        hi[q] = (ok && d < D) ? v : -INFINITY;
        lo[q] = wave_min(lo[q]);
        hi[q] = wave_max(hi[q]);
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
      sCen[d] = 0.5f * l + 0.5f * h;
    }
    __syncthreads();
  }

  // ---- A operands: lane holds x~[row t*16 + l%16][k = 4s + l/16]; partial |x'|^2 over its k
  const int lrow = lane & 15, lgrp = lane >> 4;
  float xa[TI][KS];
  float nxp[TI];
#pragma unroll
  for (int t = 0; t < TI; ++t) {
    const int64_t i = wg_row0 + wid * 64 + t * 16 + lrow;
    const bool ok = i < M;
    nxp[t] = 0.0f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int k = 4 * s + lgrp;
      float v = 0.0f;
      if (k < D) {
        const float xp = ok ? a.scale * (a.x[i * D + k] - sCen[k]) : 0.0f;
        nxp[t] = fmaf(xp, xp, nxp[t]);
        v = 2.0f * xp;
      } else if (k == D) {
        v = 1.0f;
      }
      xa[t][s] = v;
    }
  }
  // full |x'|^2 of row l%16 (sum over the four lane groups), then the work-group radius
  float nrow[TI];
  float r2 = 0.0f;
#pragma unroll
  for (int t = 0; t < TI; ++t) {
    float v = nxp[t];
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    nrow[t] = v;
    const int64_t i = wg_row0 + wid * 64 + t * 16 + lrow;
    if (i < M) r2 = fmaxf(r2, v);
  }
  r2 = block_max(r2, sRed + 2 * D * (kThreads / kWave));
  const bool fast = a.form == FORM_AUTO && r2 <= kFastR2;
  // Record the decision; a work-group beyond the expansion's bound is left to the
  // direct-form VALU kernel launched after this one (same 256 rows per work-group).
  if (tid == 0 && blockIdx.y == 0 && a.wg_flags) a.wg_flags[blockIdx.x] = fast ? 1 : 0;
  if (!fast) return;   // uniform across the work-group

  // C input of each tile: -|x'|^2 of the output rows 4*(l/16) + r
  floatx4 cin[TI];
#pragma unroll
  for (int t = 0; t < TI; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) cin[t][r] = -__shfl(nrow[t], 4 * lgrp + r);

  const int64_t jb = (int64_t)blockIdx.y * a.j_per_split;
  const int64_t je = (jb + a.j_per_split < N) ? jb + a.j_per_split : N;

  // Tile staging: thread (jl = tid/4, g = tid%4) owns k-group g of column jl, i.e.
  // k = g, g+4, g+8, ...: it loads those raw coordinates from HBM (the four threads
  // of a column cover its row contiguously), centres and scales them, and writes
  // them as one contiguous KSP-float slice; the column's |y'|^2 is the sum of the
  // four partial norms (two lane shuffles).
  static_assert(TJ * 4 == kThreads, "one k-group per thread");
  const int sj = tid >> 2, sg = tid & 3;
  float ry[KSP];
  float rb[E];
  auto load_tile = [&](int64_t jt) {
    const int64_t j = jt + sj;
    const bool ok = j < je;
#pragma unroll
    for (int q = 0; q < KSP; ++q) {
      const int k = 4 * q + sg;
      ry[q] = (ok && k < D) ? a.y[j * D + k] : 0.0f;
    }
    const int64_t jb2 = jt + tid;
#pragma unroll
    for (int e = 0; e < E; ++e) rb[e] = (tid < TJ && jb2 < je) ? a.b[jb2 * E + e] : 0.0f;
  };
  auto stage_tile = [&](int buf, int64_t jt) {
    const bool ok = jt + sj < je;
    float v[KSP];
    float ny = 0.0f;
#pragma unroll
    for (int q = 0; q < KSP; ++q) {
      const int k = 4 * q + sg;
      if (k < D) {
        v[q] = a.scale * (ry[q] - sCen[k]);
        ny = fmaf(v[q], v[q], ny);
      } else {
        v[q] = 0.0f;
      }
    }
    ny += __shfl_xor(ny, 1);
    ny += __shfl_xor(ny, 2);
    if (sg == (D & 3)) v[D >> 2] = ok ? -ny : -1.0e30f;   // padded j: exponent -> -1e30
    float4 *dst = reinterpret_cast<float4 *>(sY[buf] + sj * JS + sg * KSP);
#pragma unroll
    for (int q = 0; q < KSP / 4; ++q) dst[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    if (tid < TJ) {
#pragma unroll
      for (int e = 0; e < E; ++e) sB[buf][e * TJ + tid] = rb[e];
    }
  };

  float acc[TI][4][E];
#pragma unroll
  for (int t = 0; t < TI; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[t][r][e] = 0.0f;

  if (jb < je) {
    load_tile(jb);
    stage_tile(0, jb);
  }
  __syncthreads();
  int buf = 0;
  for (int64_t jt = jb; jt < je; jt += TJ) {
    const bool has_next = jt + TJ < je;
    if (has_next) load_tile(jt + TJ);   // HBM loads in flight while this tile is reduced
    const int cnt = (int)(je - jt < TJ ? je - jt : TJ);
    const float *yt = sY[buf];
    const float *bt = sB[buf];
    float part[TI][4][E];
#pragma unroll
    for (int t = 0; t < TI; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < E; ++e) part[t][r][e] = 0.0f;
    for (int j16 = 0; j16 < cnt; j16 += 16) {
      // B operand: k-slice of column j16 + l%16 for lane group l/16
      float yb[KSP];
      const float4 *src = reinterpret_cast<const float4 *>(yt + (j16 + lrow) * JS + lgrp * KSP);
#pragma unroll
      for (int v = 0; v < KSP / 4; ++v) {
        const float4 q = src[v];
        yb[4 * v] = q.x; yb[4 * v + 1] = q.y; yb[4 * v + 2] = q.z; yb[4 * v + 3] = q.w;
      }
      floatx4 dacc[TI];
#pragma unroll
      for (int t = 0; t < TI; ++t) dacc[t] = cin[t];
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int t = 0; t < TI; ++t)
          dacc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[t][s], yb[s], dacc[t], 0, 0, 0);
      float bj[E];
#pragma unroll
      for (int e = 0; e < E; ++e) bj[e] = bt[e * TJ + j16 + lrow];
      float ex[TI][4];
#pragma unroll
      for (int t = 0; t < TI; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) ex[t][r] = fast_exp2(dacc[t][r]);
#pragma unroll
      for (int t = 0; t < TI; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int e = 0; e < E; ++e) part[t][r][e] = fmaf(ex[t][r], bj[e], part[t][r][e]);
    }
#pragma unroll
    for (int t = 0; t < TI; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[t][r][e] += part[t][r][e];
    if (has_next) stage_tile(buf ^ 1, jt + TJ);
    __syncthreads();
    buf ^= 1;
  }

  // ---- merge the 16 column lanes of every output row and store
  const bool partial = a.nsplit > 1;
  {
#pragma unroll
    for (int t = 0; t < TI; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[t][r][e] = row16_sum(acc[t][r][e]);
    // lane l%16 == r' (r' < 4) of group g writes row 4g + r'
    if (lrow < 4) {
#pragma unroll
      for (int t = 0; t < TI; ++t) {
        const int64_t i = wg_row0 + wid * 64 + t * 16 + 4 * lgrp + lrow;
        if (i < M) {
#pragma unroll
          for (int e = 0; e < E; ++e) {
            float v = acc[t][0][e];
#pragma unroll
            for (int r = 1; r < 4; ++r) v = (lrow == r) ? acc[t][r][e] : v;
            const int64_t o = partial ? (((int64_t)blockIdx.y * M + i) * E + e) : (i * E + e);
            a.out[o] = v;
          }
        }
      }
    }
  }
}

template <int D, int E>
void launch_gauss_mfma_sum_t(dim3 grid, const GaussArgs &a, hipStream_t st) {
  hipLaunchKernelGGL((gauss_mfma_sum_kernel<D, E>), grid, dim3(kThreads), 0, st, a);
}

}  // namespace kmi
