// gauss_mfma.h -- pass-1 kernels of the Gaussian sum, LogSumExp and gradient with
// respect to x for D >= 32 on gfx950 fp32 matrix cores (KeOps pages: "Kernel
// Operations on the GPU, with Autodiff, without Memory Overflows" §1 "Target
// operation", §2 reductions (log-sum-exp) and autodiff; §4 names tensor-core
// support as future work -- here the cross term <x, y> of a large-D distance is a
// real dense contraction and runs on MFMA).
//
// With x' = s(x - c), y' = s(y - c) (s = sqrt(log2 e)/sigma, c the work-group's
// bounding-box centre) the exponent of K_ij in log2 units is
//   -|x'_i - y'_j|^2 = <x~_i, y~_j> - |x'_i|^2,
//   x~_i = (2x'_i, 1, 0...),  y~_j = (y'_j, -|y'_j|^2 + c_j, 0...),
// a K = D+1 contraction (padded to a multiple of 4); c_j is 0 except for the
// LogSumExp with one payload column, where it is b_j log2 e - m (below).  One
// v_mfma_f32_16x16x4f32 step multiplies a 16 x 4 slice of one operand by a 4 x 16
// slice of the other; the x~ slices stay in VGPRs for the whole j loop, the y~
// slices come from LDS, and the C input holds -|x'_i|^2, so the MFMA output is the
// exponent itself.
//
// Sum and LogSumExp: A = x~ (16 rows), B = y~ (16 columns j); output lane l holds
// rows 4(l/16) + r (r < 4) of column l%16, accumulates over the columns l%16 mod 16
// and a 16-lane DPP reduction merges them at the end.  The VALU evaluates one
// v_exp_f32 and E FMAs (sum) or adds (LogSumExp) per pair.  The LogSumExp takes a
// work-group shift m_e = max_j b_je log2 e over its j, so that every term
// exp2(u + b log2 e - m) is at most 1 and the sum at most nj: no running maximum.
//
// Gradient: the same contraction with the operands swapped (A = y~, B = x~) gives
// the exponent tile transposed: lane l holds row l%16 and the columns
// j = 4(l/16) + r.  Those four weights w_ij = K_ij <g_i, b_j> are exactly the A
// operand of a second product over j, O_i = sum_j w_ij y'_j, whose B operand (y'
// of the tile, coordinate-major in LDS) is read four j at a time; then
//   sum_j w_ij (x'_i - y'_j) = x'_i sum_j w_ij - O_i
// and G_i = -(2 / sigma^2) / s times that (for one payload column, g_i factors out
// and is applied at the end).
//
// Work-group: 256 threads = 4 waves; each wave owns 4 row tiles (64 rows), i.e. 256
// rows per work-group; four independent MFMA chains per wave (the gradient at D > 64:
// eight waves of two row tiles, the same 256 rows).  j tiles of TJ = 64 rows are
// staged in LDS (double-buffered, one barrier per tile) in a permuted y~ layout that
// lets each lane read its k-slice with ds_read_b128; 256 threads build it, four per
// column.
//
// Range conditions, each decided by the work-group for its (row block, j split):
//  * the expansion's precision condition of the VALU expanded form, max |x'_i|^2 <=
//    kFastR2 over the work-group, and finite payload (and LogSumExp shift);
//  * underflow: terms below 2^-126 are flushed; a row result below nj max|b| 2^-109
//    (gradient: times 32, and sum_e |g_e| for several payload columns; LogSumExp: a
//    sum below nj 2^-110), or a non-finite one, could have lost more than 2^-17 of
//    itself.
// A work-group that fails either records 0 in wg_flags[block * nsplit + split]
// (1 when its results stand); the VALU kernel, launched next on the same stream
// with the same 256-row work-groups and j splits, computes exactly the flagged
// work-groups in the direct form, with its own range checks.
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
  static constexpr int DT = (D + 15) / 16;         // 16-coordinate tiles of the gradient's y' product
  static constexpr int YTS = TJ + 4;               // floats per coordinate row of the coordinate-major y'
};

// The gradient's work-group: 256 rows like the sum's (the VALU kernel that takes over
// failed work-groups uses the same blocks), as four waves of four row tiles, or at
// D > 64 eight waves of two (four tiles' x~ slices and 16-coordinate accumulator tiles
// would not fit one wave's registers there); the first 256 threads stage the tiles.
template <int D>
struct MfmaGradShape : MfmaShape<D> {
  static constexpr int NW = D > 64 ? 8 : 4;        // waves per work-group
  static constexpr int TI = D > 64 ? 2 : 4;        // 16-row tiles per wave
  static constexpr int NT = NW * kWave;            // threads per work-group
  static constexpr int ROWS_WG = NW * 16 * TI;
  static_assert(ROWS_WG == 256, "the VALU kernel's 256-row blocks");
};

// Work-group maximum over NW waves; `red` holds NW floats.  Contains barriers.
template <int NW>
__device__ __forceinline__ float block_max_w(float v, float *red) {
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int k = 1; k < NW; ++k) r = fmaxf(r, red[k]);
  return r;
}

// Bounding-box centre of the work-group's ROWS rows (thread t < ROWS scans row
// wg_row0 + t) into sCen; NW waves, sRed holds 2 D NW floats.  Contains barriers:
// every thread of the work-group calls it.
template <int D, int NW, int ROWS>
__device__ __forceinline__ void mfma_centre(const float *x, int64_t M, int64_t wg_row0, float *sRed, float *sCen) {
  const int tid = threadIdx.x, wid = tid / kWave, lane = tid & (kWave - 1);
  const int64_t i = wg_row0 + tid;
  const bool ok = tid < ROWS && i < M;
  for (int d0 = 0; d0 < D; d0 += 4) {
    float lo[4], hi[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int d = d0 + q;
      const float v = (ok && d < D) ? x[i * D + d] : 0.0f;
      lo[q] = wave_min((ok && d < D) ? v : INFINITY);
      hi[q] = wave_max((ok && d < D) ? v : -INFINITY);
    }
    if (lane == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (d0 + q < D) { sRed[(2 * (d0 + q)) * NW + wid] = lo[q]; sRed[(2 * (d0 + q) + 1) * NW + wid] = hi[q]; }
    }
  }
  __syncthreads();
  for (int d = tid; d < D; d += NW * kWave) {
    float l = sRed[(2 * d) * NW], h = sRed[(2 * d + 1) * NW];
#pragma unroll
    for (int w = 1; w < NW; ++w) { l = fminf(l, sRed[(2 * d) * NW + w]); h = fmaxf(h, sRed[(2 * d + 1) * NW + w]); }
    sCen[d] = 0.5f * l + 0.5f * h;
  }
  __syncthreads();
}

// x~ slices of the wave's TI row tiles (wave w owns rows w*16*TI ...): lane l holds
// x~[row t*16 + l%16][k = 4s + l/16]; nrow[t] gets |x'|^2 of row t*16 + l%16 (whole, in
// all four lanes of the row).  Returns the largest |x'|^2 over the wave's rows below M.
template <int D, int TI>
__device__ __forceinline__ float mfma_rows(const GaussArgs &a, int64_t wg_row0, const float *sCen,
                                           float (&xa)[TI][MfmaShape<D>::KS], float (&nrow)[TI]) {
  using S = MfmaShape<D>;
  const int tid = threadIdx.x, wid = tid / kWave, lane = tid & (kWave - 1);
  const int lrow = lane & 15, lgrp = lane >> 4;
  float r2 = 0.0f;
#pragma unroll
  for (int t = 0; t < TI; ++t) {
    const int64_t i = wg_row0 + wid * (16 * TI) + t * 16 + lrow;
    const bool ok = i < a.M;
    float n = 0.0f;
#pragma unroll
    for (int s = 0; s < S::KS; ++s) {
      const int k = 4 * s + lgrp;
      float v = 0.0f;
      if (k < D) {
        const float xp = ok ? a.scale * (a.x[i * D + k] - sCen[k]) : 0.0f;
        n = fmaf(xp, xp, n);
        v = 2.0f * xp;
      } else if (k == D) {
        v = 1.0f;
      }
      xa[t][s] = v;
    }
    n += __shfl_xor(n, 16);
    n += __shfl_xor(n, 32);
    nrow[t] = n;
    if (ok) r2 = fmaxf(r2, n);
  }
  return r2;
}

// Tile staging shared by the kernels: thread (sj = tid/4, sg = tid%4) owns k-group sg
// of column sj, i.e. k = sg, sg+4, ...: it loads those raw coordinates (the four
// threads of a column cover its row contiguously), centres and scales them and writes
// them as one contiguous KSP-float slice; the column's |y'|^2 is the sum of the four
// partial norms (two lane shuffles).  Slot D of the slice holds -|y'|^2 + cadd
// (padded j: -1e30, so that their exponent flushes to 0).  yT (gradient only): the
// centred, scaled coordinates again, coordinate-major ([d][j], row stride YTS).
template <int D>
__device__ __forceinline__ void mfma_stage_y(float *sYb, float *yT, const float (&ry)[MfmaShape<D>::KSP],
                                             const float *sCen, float scale, bool ok, float cadd) {
  using S = MfmaShape<D>;
  const int tid = threadIdx.x, sj = tid >> 2, sg = tid & 3;
  float v[S::KSP];
  float ny = 0.0f;
#pragma unroll
  for (int q = 0; q < S::KSP; ++q) {
    const int k = 4 * q + sg;
    if (k < D) {
      v[q] = scale * (ry[q] - sCen[k]);
      ny = fmaf(v[q], v[q], ny);
      if (yT) yT[k * S::YTS + sj] = v[q];
    } else {
      v[q] = 0.0f;
    }
  }
  ny += __shfl_xor(ny, 1);
  ny += __shfl_xor(ny, 2);
  if (sg == (D & 3)) v[D >> 2] = ok ? -ny + cadd : -1.0e30f;
  float4 *dst = reinterpret_cast<float4 *>(sYb + sj * S::JSTRIDE + sg * S::KSP);
#pragma unroll
  for (int q = 0; q < S::KSP / 4; ++q) dst[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
}

// ---------------------------------------------------------------- sum and LogSumExp
template <int OP, int D, int E>
__global__ __launch_bounds__(kThreads) void gauss_mfma_kernel(GaussArgs a) {
  static_assert(OP == OP_SUM || OP == OP_LSE, "sum or LogSumExp");
  using S = MfmaShape<D>;
  constexpr int KS = S::KS, KSP = S::KSP, JS = S::JSTRIDE, TJ = S::TJ, TI = S::TI;
  constexpr bool FOLD = OP == OP_LSE && E == 1;   // b log2 e - m rides in y~'s last slot
  __shared__ __attribute__((aligned(16))) float sY[2][TJ * JS];   // permuted y~, double-buffered
  __shared__ float sB[2][E * TJ];                                // payload of the tile, [e][j]
  __shared__ float sRed[2 * D * (kThreads / kWave) + 8];
  __shared__ float sCen[D];

  const int tid = threadIdx.x;
  const int wid = tid / kWave, lane = tid & (kWave - 1);
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int64_t M = a.M, N = a.N;
  const int64_t wg_row0 = (int64_t)blockIdx.x * S::ROWS_WG;
  const int64_t flag_at = (int64_t)blockIdx.x * gridDim.y + blockIdx.y;
  float *red = sRed + 2 * D * (kThreads / kWave);

  mfma_centre<D, 4, S::ROWS_WG>(a.x, M, wg_row0, sRed, sCen);
  float xa[TI][KS];
  float nrow[TI];
  const float r2 = block_max(mfma_rows<D, TI>(a, wg_row0, sCen, xa, nrow), red);

  const int64_t jb = (int64_t)blockIdx.y * a.j_per_split;
  const int64_t je = (jb + a.j_per_split < N) ? jb + a.j_per_split : N;

  // LogSumExp: the work-group shift m_e = max_j b_je log2 e over its j (one extra
  // read of b, 1/D of the y traffic)
  float m[E];
#pragma unroll
  for (int e = 0; e < E; ++e) m[e] = 0.0f;
  bool finite_m = true;
  if (OP == OP_LSE) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float mx = -INFINITY;
      for (int64_t j = jb + tid; j < je; j += kThreads) mx = fmaxf(mx, kLog2e * a.b[j * E + e]);
      m[e] = block_max(mx, red);
      finite_m &= isfinite(m[e]);
    }
  }
  const bool fast = a.form == FORM_AUTO && r2 <= kFastR2 && finite_m;
  if (!fast) {   // uniform across the work-group: the VALU kernel takes it
    if (tid == 0 && a.wg_flags) a.wg_flags[flag_at] = 0;
    return;
  }

  // C input of each tile: -|x'|^2 of the output rows 4*(l/16) + r
  floatx4 cin[TI];
#pragma unroll
  for (int t = 0; t < TI; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) cin[t][r] = -__shfl(nrow[t], 4 * lgrp + r);

  static_assert(TJ * 4 == kThreads, "one k-group per thread");
  const int sj = tid >> 2, sg = tid & 3;
  float ry[KSP];
  float rb[E];
  float bmx = 0.0f;   // the largest |b| of the work-group's j (sum: underflow threshold)
  auto load_tile = [&](int64_t jt) {
    const int64_t j = jt + sj;
    const bool ok = j < je;
#pragma unroll
    for (int q = 0; q < KSP; ++q) {
      const int k = 4 * q + sg;
      ry[q] = (ok && k < D) ? a.y[j * D + k] : 0.0f;
    }
    // payload: thread t < TJ loads column t (FOLD: the column's own, all four threads)
    const int64_t jp = FOLD ? j : jt + tid;
    const bool okp = FOLD ? ok : (tid < TJ && jp < je);
#pragma unroll
    for (int e = 0; e < E; ++e) rb[e] = okp ? a.b[jp * E + e] : 0.0f;
  };
  auto stage_tile = [&](int buf, int64_t jt) {
    const bool ok = jt + sj < je;
    mfma_stage_y<D>(sY[buf], nullptr, ry, sCen, a.scale, ok, FOLD ? fmaf(kLog2e, rb[0], -m[0]) : 0.0f);
    if (!FOLD && tid < TJ) {
      const bool okp = jt + tid < je;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (OP == OP_SUM) {
          bmx = fmaxf(bmx, fabsf(rb[e]));
          sB[buf][e * TJ + tid] = rb[e];
        } else {
          sB[buf][e * TJ + tid] = okp ? fmaf(kLog2e, rb[e], -m[e]) : -INFINITY;
        }
      }
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
      if (FOLD) {
#pragma unroll
        for (int t = 0; t < TI; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) part[t][r][0] += fast_exp2(dacc[t][r]);
      } else {
        float bj[E];
#pragma unroll
        for (int e = 0; e < E; ++e) bj[e] = bt[e * TJ + j16 + lrow];
        if (OP == OP_SUM) {
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
        } else {
#pragma unroll
          for (int t = 0; t < TI; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
              for (int e = 0; e < E; ++e) part[t][r][e] += fast_exp2(dacc[t][r] + bj[e]);
        }
      }
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

  // ---- merge the 16 column lanes of every output row, check, store
  const int64_t nj = je - jb;
  const float log2n = nj > 1 ? ceilf(log2f((float)nj)) : 0.0f;
  float thr;
  if (OP == OP_SUM) thr = exp2f(log2n - kGuardLoss) * fmaxf(block_max(bmx, red), 1.0f);
  else thr = exp2f(log2n - kGuardLoss - 1.0f);
  const bool partial = a.nsplit > 1;
  bool low = false;
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
          if (OP == OP_SUM) {
            low |= !(fabsf(v) >= thr) || !(fabsf(v) < INFINITY);
            const int64_t o = partial ? (((int64_t)blockIdx.y * M + i) * E + e) : (i * E + e);
            a.out[o] = v;
          } else {
            low |= !(v >= thr) || !(v < INFINITY);
            if (partial) {
              float *dst = a.out + (((int64_t)blockIdx.y * M + i) * E + e) * 2;
              dst[0] = m[e];
              dst[1] = v;
            } else {
              a.out[i * E + e] = kLn2 * (m[e] + log2f(v));
            }
          }
        }
      }
    }
  }
  const bool any_low = __syncthreads_or(low);
  if (tid == 0 && a.wg_flags) a.wg_flags[flag_at] = any_low ? 0 : 1;
}

// ---------------------------------------------------------------- gradient
template <int D, int E>
__global__ __launch_bounds__(MfmaGradShape<D>::NT) void gauss_mfma_grad_kernel(GaussArgs a) {
  using S = MfmaGradShape<D>;
  constexpr int KS = S::KS, KSP = S::KSP, JS = S::JSTRIDE, TJ = S::TJ, TI = S::TI, DT = S::DT, YTS = S::YTS;
  constexpr int NW = S::NW, NT = S::NT;
  __shared__ __attribute__((aligned(16))) float sY[2][TJ * JS];         // permuted y~, double-buffered
  __shared__ __attribute__((aligned(16))) float sYT[2][16 * DT * YTS];  // y' coordinate-major [d][j]
  __shared__ __attribute__((aligned(16))) float sB[2][E * TJ];          // payload of the tile, [e][j]
  __shared__ float sRed[2 * D * NW + NW];
  __shared__ float sCen[D];

  const int tid = threadIdx.x;
  const int wid = tid / kWave, lane = tid & (kWave - 1);
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int64_t M = a.M, N = a.N;
  const int64_t wg_row0 = (int64_t)blockIdx.x * S::ROWS_WG;
  const int64_t flag_at = (int64_t)blockIdx.x * gridDim.y + blockIdx.y;
  float *red = sRed + 2 * D * NW;

  mfma_centre<D, NW, S::ROWS_WG>(a.x, M, wg_row0, sRed, sCen);
  float xa[TI][KS];
  float nrow[TI];
  const float r2 = block_max_w<NW>(mfma_rows<D, TI>(a, wg_row0, sCen, xa, nrow), red);
  // g of row t*16 + l%16 (several payload columns: it weights every pair; one: it
  // factors out and is applied at the end)
  float gi[TI][E];
  float gs = 0.0f;
#pragma unroll
  for (int t = 0; t < TI; ++t) {
    const int64_t i = wg_row0 + wid * (16 * TI) + t * 16 + lrow;
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      gi[t][e] = i < M ? a.g[i * E + e] : 0.0f;
      s += fabsf(gi[t][e]);
    }
    gs = fmaxf(gs, s);
  }
  const float gmax = block_max_w<NW>(gs, red);
  const bool fast = a.form == FORM_AUTO && r2 <= kFastR2 && isfinite(gmax);
  if (!fast) {
    if (tid == 0 && a.wg_flags) a.wg_flags[flag_at] = 0;
    return;
  }
  // the transposed product's C input: -|x'|^2 of row l%16 in all four slots
  floatx4 cin[TI];
#pragma unroll
  for (int t = 0; t < TI; ++t) cin[t] = (floatx4){-nrow[t], -nrow[t], -nrow[t], -nrow[t]};
  // coordinates D .. 16 DT - 1 of the coordinate-major tiles stay 0
  for (int f = tid; f < (16 * DT - D) * YTS; f += NT) {
    sYT[0][D * YTS + f] = 0.0f;
    sYT[1][D * YTS + f] = 0.0f;
  }

  const int64_t jb = (int64_t)blockIdx.y * a.j_per_split;
  const int64_t je = (jb + a.j_per_split < N) ? jb + a.j_per_split : N;

  static_assert(TJ * 4 <= NT, "four staging threads per j");
  const int sj = tid >> 2;
  const bool stager = tid < 4 * TJ;
  float ry[KSP];
  float rb[E];
  float bmx = 0.0f;
  auto load_tile = [&](int64_t jt) {
    const int64_t j = jt + sj;
    const bool ok = stager && j < je;
    const int sg = tid & 3;
#pragma unroll
    for (int q = 0; q < KSP; ++q) {
      const int k = 4 * q + sg;
      ry[q] = (ok && k < D) ? a.y[j * D + k] : 0.0f;
    }
    const int64_t jp = jt + tid;
#pragma unroll
    for (int e = 0; e < E; ++e) rb[e] = (tid < TJ && jp < je) ? a.b[jp * E + e] : 0.0f;
  };
  auto stage_tile = [&](int buf, int64_t jt) {
    if (stager) mfma_stage_y<D>(sY[buf], sYT[buf], ry, sCen, a.scale, jt + sj < je, 0.0f);
    if (tid < TJ) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        bmx = fmaxf(bmx, fabsf(rb[e]));
        sB[buf][e * TJ + tid] = rb[e];
      }
    }
  };

  floatx4 O[TI][DT];   // sum_j w_ij y'_j: rows 4(l/16) + r, coordinate 16 dt + l%16
  float ws[TI];        // sum_j w_ij over this lane's j, row l%16
#pragma unroll
  for (int t = 0; t < TI; ++t) {
    ws[t] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) O[t][dt] = (floatx4){0.0f, 0.0f, 0.0f, 0.0f};
  }

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
    const float *yt = sY[buf];
    const float *ytT = sYT[buf];
    const float *bt = sB[buf];
    for (int j16 = 0; j16 < cnt; j16 += 16) {
      // A operand: k-slice of column j16 + l%16 for lane group l/16
      float yb[KSP];
      const float4 *src = reinterpret_cast<const float4 *>(yt + (j16 + lrow) * JS + lgrp * KSP);
#pragma unroll
      for (int v = 0; v < KSP / 4; ++v) {
        const float4 q = src[v];
        yb[4 * v] = q.x; yb[4 * v + 1] = q.y; yb[4 * v + 2] = q.z; yb[4 * v + 3] = q.w;
      }
      floatx4 u[TI];
#pragma unroll
      for (int t = 0; t < TI; ++t) u[t] = cin[t];
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int t = 0; t < TI; ++t)
          u[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(yb[s], xa[t][s], u[t], 0, 0, 0);
      // weights of row l%16 and j = j16 + 4(l/16) + r
      float4 bq[E];
#pragma unroll
      for (int e = 0; e < E; ++e) bq[e] = *reinterpret_cast<const float4 *>(bt + e * TJ + j16 + 4 * lgrp);
      float w[TI][4];
#pragma unroll
      for (int t = 0; t < TI; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float gb;
          if (E == 1) {
            gb = lane4(bq[0], r);
          } else {
            gb = 0.0f;
#pragma unroll
            for (int e = 0; e < E; ++e) gb = fmaf(gi[t][e], lane4(bq[e], r), gb);
          }
          w[t][r] = fast_exp2(u[t][r]) * gb;
          ws[t] += w[t][r];
        }
      // O += w y': step r contracts over j = j16 + 4(l/16) + r
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const float4 yv = *reinterpret_cast<const float4 *>(ytT + (16 * dt + lrow) * YTS + j16 + 4 * lgrp);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int t = 0; t < TI; ++t)
            O[t][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(w[t][r], lane4(yv, r), O[t][dt], 0, 0, 0);
      }
    }
    if (has_next) stage_tile(buf ^ 1, jt + TJ);
    __syncthreads();
    buf ^= 1;
  }

  // ---- sum_j w_ij (x'_i - y'_j) = x'_i W_i - O_i, checked and stored
  const int64_t nj = je - jb;
  const float log2n = nj > 1 ? ceilf(log2f((float)nj)) : 0.0f;
  const float thr = exp2f(log2n - kGuardLoss) * fmaxf(block_max_w<NW>(bmx, red), 1.0f) * 32.0f * (E == 1 ? 1.0f : gmax);
  const bool partial = a.nsplit > 1;
  bool low = false;
#pragma unroll
  for (int t = 0; t < TI; ++t) {
    ws[t] += __shfl_xor(ws[t], 16);
    ws[t] += __shfl_xor(ws[t], 32);
  }
#pragma unroll
  for (int t = 0; t < TI; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int il = t * 16 + 4 * lgrp + r;
      const int64_t i = wg_row0 + wid * (16 * TI) + il;
      const float W = __shfl(ws[t], 4 * lgrp + r);
      if (i < M) {
        const float gf = a.grad_coef * (E == 1 ? a.g[i * E] : 1.0f);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int d = 16 * dt + lrow;
          if (d < D) {
            const float xp = a.scale * (a.x[i * D + d] - sCen[d]);
            const float v = fmaf(xp, W, -O[t][dt][r]);
            low |= !(fabsf(v) >= thr) || !(fabsf(v) < INFINITY);
            const int64_t o = partial ? (((int64_t)blockIdx.y * M + i) * D + d) : (i * D + d);
            a.out[o] = v * gf;
          }
        }
      }
    }
  const bool any_low = __syncthreads_or(low);
  if (tid == 0 && a.wg_flags) a.wg_flags[flag_at] = any_low ? 0 : 1;
}

template <int OP, int D, int E>
void launch_gauss_mfma_t(dim3 grid, const GaussArgs &a, hipStream_t st) {
  hipLaunchKernelGGL((gauss_mfma_kernel<OP, D, E>), grid, dim3(kThreads), 0, st, a);
}

template <int D, int E>
void launch_gauss_mfma_grad_t(dim3 grid, const GaussArgs &a, hipStream_t st) {
  hipLaunchKernelGGL((gauss_mfma_grad_kernel<D, E>), grid, dim3(MfmaGradShape<D>::NT), 0, st, a);
}

}  // namespace kmi
