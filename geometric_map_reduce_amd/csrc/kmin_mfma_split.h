// kmin_mfma_split.h -- pass-1 kernel of the K-min reduction for D >= 32 whose
// prefilter runs on gfx950's bf16 matrix cores (KeOps pages: "Kernel Operations
// on the GPU, with Autodiff, without Memory Overflows" §2, argKmin; KeOps
// README feature list, "K-min reductions").
//
// The prefilter value is the one of the fp32-MFMA kernel,
//   u_ij = |y_c|^2 - 2<x_c, y_c> = |x_i - y_j|^2 - |x_c|^2      (c: work-group centre),
// but the cross term is formed from a two-part bf16 split of each operand,
// v = v_hi + v_lo (v_hi = bf16(v), v_lo = bf16(v - v_hi)):
//   <y, -2x> ~ <y_hi, (-2x)_hi> + <y_hi, (-2x)_lo> + <y_lo, (-2x)_hi>
// with three v_mfma_f32_16x16x32_bf16 per 32 coordinates (products exact in
// fp32, fp32 accumulation), and |y_c|^2 entering as the instruction's C input.
// bf16 keeps 8 significant bits, so |v - v_hi| <= 2^-8 |v| and the rounding of
// the lo part is below 2^-16 |v|.  The dropped product y_lo (-2x)_lo and the two
// lo roundings are then each below about 2^-16 |y_k| |2x_k|, and the split error
// is below 3.01 * 2^-16 sum_k |y_k| |2x_k| <= 1.51 * 2^-16 (2|x_c| + sqrt(kth))^2
// (kth: the row's K-th distance, with |y_c| <= |x_c| + sqrt(kth) for every
// candidate that matters).  The pass margin adds 2^-14 of that square, 2.66
// times the bound, to the accumulation bound of the fp32 form over
// 3 * 32 * ceil(D / 32) products.  A candidate whose exact distance could be
// below the row's K-th therefore always passes; passing candidates get the exact direct-form fp32 distance
// from raw coordinates and the same register insertion, lane-group threshold
// sharing and final merge as the fp32-MFMA kernel, so the result is that of
// the direct-form K-min in fp32, bit for bit.
//
// Per 16 x 16 tile at D = 64 this is 6 bf16 MFMA (16 cycles each) against 17
// fp32 ones (32 cycles each) for the fp32 form.
#pragma once

#include "common.h"
#include "kmin_kernel.h"

namespace kmi {

typedef float floatx4s __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8s __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2s __attribute__((ext_vector_type(2)));
typedef float float2s __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4s __attribute__((ext_vector_type(4)));

// Split two floats into packed bf16 hi parts (round to nearest even, one
// v_cvt_pk_bf16_f32) and packed bf16 parts of the exact remainders.
__device__ __forceinline__ void split_bf16x2(float v0, float v1, unsigned &hi, unsigned &lo) {
  hi = __builtin_bit_cast(unsigned, __builtin_convertvector((float2s){v0, v1}, bf16x2s));
  const float h0 = __builtin_bit_cast(float, hi << 16);
  const float h1 = __builtin_bit_cast(float, hi & 0xffff0000u);
  lo = __builtin_bit_cast(unsigned, __builtin_convertvector((float2s){v0 - h0, v1 - h1}, bf16x2s));
}

// Pass margin coefficient of the split form (see the header comment): the fp32
// form's bound taken over the 3 * DP products, plus 2^-14 for the split.
__device__ __forceinline__ float kmin_split_margin_coef(int DP) { return kmin_margin_coef(3 * DP) + 6.103515625e-5f; }

// Exact direct-form squared distance sum_k (x_k - y_k)^2 in fp32, in coordinate
// order (the same arithmetic as every other K-min kernel), from raw rows staged in
// LDS (16-byte aligned, padded to whole float4).
template <int D>
__device__ __forceinline__ float exact_sq_dist_lds(const float *xi, const float *yj) {
  float d2 = 0.0f;
#pragma unroll
  for (int k = 0; k < D / 4 * 4; k += 4) {
    const float4 p = *reinterpret_cast<const float4 *>(xi + k);
    const float4 q = *reinterpret_cast<const float4 *>(yj + k);
    float d = p.x - q.x; d2 = fmaf(d, d, d2);
    d = p.y - q.y; d2 = fmaf(d, d, d2);
    d = p.z - q.z; d2 = fmaf(d, d, d2);
    d = p.w - q.w; d2 = fmaf(d, d, d2);
  }
#pragma unroll
  for (int k = D / 4 * 4; k < D; ++k) { const float d = xi[k] - yj[k]; d2 = fmaf(d, d, d2); }
  return d2;
}

// Work-group shape.  Twelve waves (768 threads, three waves per SIMD at <= 168
// VGPRs) with two 16-row tiles per wave up to K = 15 at D = 32 and K = 10 at
// D <= 64 (beyond, the K-lists spill; at D = 64 the compiler spills 2 to 8
// registers from K = 8 to 10, and that form still ran faster than eight waves:
// 558 against 624 ms at K = 10); else eight waves (two per SIMD, <= 256 VGPRs)
// with three tiles per wave where that still fits, else two, and one at K = 32
// (with two, the 128 registers of its lists were placed in scratch memory).  The
// two main forms hold 384 rows (12 x 2 x 16, 8 x 3 x 16).
constexpr bool kmin_split_wide(int D, int K) { return D <= 32 ? K <= 15 : (D <= 64 ? K <= 10 : false); }
constexpr int kmin_split_threads(int D, int K) { return kmin_split_wide(D, K) ? 768 : 512; }
constexpr int kmin_split_tiles(int D, int K) {
  return kmin_split_wide(D, K) ? 2 : (K <= (D <= 32 ? 13 : (D <= 64 ? 12 : 0)) ? 3 : (K <= 16 ? 2 : 1));
}

// One work-group per CU: every y tile staged in LDS serves 16 * TI rows per wave.
// Besides the split tiles, LDS holds the raw fp32 rows of the work-group's x and of
// the current y tile, so that the exact distance of a passing candidate is read at
// LDS latency (from HBM it took four dependent rounds of global loads, and that
// recheck was over half the kernel's time at K = 10).  The y tile is the largest
// multiple of 16 j that fits beside them (80 at D = 64, 192 at D = 32), single
// buffered for the raw rows: a double-buffered raw tile leaves room for 48 j at
// D = 64 and ran slower.  Measured at 1M x 1M, D = 64, K = 10: 797 ms with
// rechecks from HBM and 128-j tiles, 624 ms with 64-j LDS tiles in the eight-wave
// form, 558 ms in the twelve-wave form, 530 ms with 80-j tiles.

template <int D, int K>
struct KminSplitShape {
  static constexpr int DP = (D + 31) / 32 * 32;    // coordinates padded to whole MFMA steps
  static constexpr int NS = DP / 32;               // MFMA steps per product
  static constexpr int RS = DP + 4;                // u32 per LDS record: DP/2 hi, DP/2 lo, 4 pad
  static constexpr int DX = (D + 3) / 4 * 4;       // floats per raw row in LDS
  static constexpr int NT = kmin_split_threads(D, K);   // threads per work-group
  static constexpr int NW = NT / kWave;               // waves per work-group
  static constexpr int TI = kmin_split_tiles(D, K);
  static constexpr int ROWS_WG = NW * 16 * TI;        // rows per work-group
  static constexpr int FIXED_FLOATS = ROWS_WG * DX + D + 64;
  static constexpr int TJ_FIT = (40960 - FIXED_FLOATS) / (2 * RS + 2 + DX) / 16 * 16;
  static constexpr int TJ = TJ_FIT < NT / 4 ? TJ_FIT : NT / 4;   // j rows per LDS tile (four staging threads each)
  static constexpr int LDS_BYTES = 4 * (TJ * (2 * RS + 2 + DX) + FIXED_FLOATS);
  static_assert(LDS_BYTES <= 160 * 1024, "split K-min work-group exceeds the LDS of a CU");
  static_assert(4 * TJ <= NT, "at least four staging threads per j");
};

template <int D, int K>
__global__ __launch_bounds__(kmin_split_threads(D, K)) void kmin_mfma_split_kernel(KminArgs a) {
  using S = KminSplitShape<D, K>;
  constexpr int kSplitThreads = S::NT, kSplitWaves = S::NW;
  constexpr int DP = S::DP, NS = S::NS, RS = S::RS, TJ = S::TJ, TI = S::TI;
  static_assert(S::ROWS_WG <= kSplitThreads, "one thread per row for the centre");
  static_assert(TJ % 16 == 0, "whole groups of 16 j per tile");
  constexpr int DX = S::DX;
  __shared__ __attribute__((aligned(16))) unsigned sRec[2 * TJ * RS];   // double-buffered split y tiles
  __shared__ __attribute__((aligned(16))) float sNy[2 * TJ];            // |y_c|^2 per j (kPadU: padding)
  __shared__ __attribute__((aligned(16))) float sYr[TJ * DX];           // raw y of the current tile
  __shared__ __attribute__((aligned(16))) float sXr[S::ROWS_WG * DX];   // raw x of the work-group's rows
  __shared__ float sCen[D];
  // the centre's per-wave extremes go to the raw y buffer, which is free until the
  // first tile is staged
  float *sRed = sYr;
  static_assert(2 * D * kSplitWaves <= TJ * DX, "centre scratch fits the raw y buffer");

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
          if (d0 + q < D) {
            sRed[(2 * (d0 + q)) * kSplitWaves + wid] = lo[q];
            sRed[(2 * (d0 + q) + 1) * kSplitWaves + wid] = hi[q];
          }
      }
    }
    __syncthreads();
    for (int d = tid; d < D; d += kSplitThreads) {
      float l = sRed[(2 * d) * kSplitWaves], h = sRed[(2 * d + 1) * kSplitWaves];
#pragma unroll
      for (int w = 1; w < kSplitWaves; ++w) {
        l = fminf(l, sRed[(2 * d) * kSplitWaves + w]);
        h = fmaxf(h, sRed[(2 * d + 1) * kSplitWaves + w]);
      }
      sCen[d] = l <= h ? 0.5f * l + 0.5f * h : 0.0f;   // 0 where no row is finite
    }
    __syncthreads();
  }

  // ---- raw x rows of the work-group in LDS (rows beyond M hold zeros; never read)
  for (int f = tid; f < S::ROWS_WG * DX; f += kSplitThreads) {
    const int r = f / DX, k = f - r * DX;
    const int64_t i = wg_row0 + r;
    sXr[f] = (i < M && k < D) ? a.x[i * D + k] : 0.0f;
  }
  // (the first barrier of the j loop orders these writes before any read)

  // ---- B operands: split -2 x_c of row t*16 + l%16, coordinates 32s + 8(l/16) + e
  u32x4s xh[TI][NS], xl[TI][NS];
  // local row index of tile t (the loop keeps only 32-bit local rows, and |x_c| is
  // recomputed where needed, to stay within three waves per SIMD)
  const int lrows = (int)(M - wg_row0 < S::ROWS_WG ? M - wg_row0 : S::ROWS_WG);   // rows of this work-group
  auto lrow_of = [&](int t) { return wid * (16 * TI) + t * 16 + lrow; };
  float nx[TI];
#pragma unroll
  for (int t = 0; t < TI; ++t) {
    const int64_t row = wg_row0 + lrow_of(t);
    const bool ok = lrow_of(t) < lrows;
    float n = 0.0f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = 32 * s + 8 * lgrp + e;
        const float c = (ok && k < D) ? a.x[row * D + k] - sCen[k < D ? k : 0] : 0.0f;
        n = fmaf(c, c, n);
        v[e] = -2.0f * c;
      }
      unsigned h[4], l[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) split_bf16x2(v[2 * e], v[2 * e + 1], h[e], l[e]);
      xh[t][s] = (u32x4s){h[0], h[1], h[2], h[3]};
      xl[t][s] = (u32x4s){l[0], l[1], l[2], l[3]};
    }
    n += __shfl_xor(n, 16);
    n += __shfl_xor(n, 32);
    nx[t] = n;
  }
  const float mcoef = kmin_split_margin_coef(DP);

  // Prefilter thresholds stay below kPadU, the value padded j carry, so padding
  // never passes; rows beyond M get -inf and never pass either.
  constexpr float kPadU = 1.0e30f, kThrCap = 5.0e29f;
  float bd[TI][K];
  int bi[TI][K];
  float thr[TI];
#pragma unroll
  for (int t = 0; t < TI; ++t) {
    thr[t] = lrow_of(t) < lrows ? kThrCap : -INFINITY;
#pragma unroll
    for (int k = 0; k < K; ++k) { bd[t][k] = INFINITY; bi[t][k] = -1; }
  }

  const int64_t jb = (int64_t)blockIdx.y * a.j_per_split;
  const int64_t je = (jb + a.j_per_split < N) ? jb + a.j_per_split : N;

  // tile staging: SPJ threads per column j; thread (sj = tid/SPJ, sg = tid%SPJ) owns the
  // 8-coordinate chunks c = sg + SPJ m (m < CPT) of column sj, chunk c holding the
  // coordinates 32 (c/4) + 8 (c%4) + e.  Eight threads per j where the work-group has
  // them (the staging then spreads over ten of twelve waves instead of five), else four.
  constexpr int SPJ = (NS >= 2 && 8 * TJ <= kSplitThreads) ? 8 : 4;
  constexpr int CPT = 4 * NS / SPJ;
  const int sj = tid / SPJ, sg = tid % SPJ;
  const bool stager = tid < SPJ * TJ;
  float ry[CPT][8];
  auto chunk_k = [&](int m, int e) {
    const int c = sg + SPJ * m;
    return 32 * (c >> 2) + 8 * (c & 3) + e;
  };
  // A chunk's 8 coordinates are consecutive: where rows allow it (D a multiple of
  // 4 or 2 and y aligned to match, a uniform test) they are read as float4 or
  // float2, 2 or 4 loads per chunk instead of 8; the parts past D are 0.
  constexpr int VW = D % 4 == 0 ? 4 : (D % 2 == 0 ? 2 : 1);
  const bool yvec = VW > 1 && ((uintptr_t)a.y & (uintptr_t)(4 * VW - 1)) == 0;
  auto load_tile = [&](int64_t jt) {
    const int64_t j = jt + sj;
    const bool ok = stager && j < je;
    if (yvec) {
#pragma unroll
      for (int m = 0; m < CPT; ++m)
#pragma unroll
        for (int e = 0; e < 8; e += VW) {
          const int k = chunk_k(m, e);   // a multiple of VW, so k < D covers the whole group
          const bool in = ok && k < D;
          if constexpr (VW == 4) {
            const float4 v = in ? *reinterpret_cast<const float4 *>(a.y + j * D + k) : make_float4(0.f, 0.f, 0.f, 0.f);
            ry[m][e] = v.x; ry[m][e + 1] = v.y; ry[m][e + 2] = v.z; ry[m][e + 3] = v.w;
          } else if constexpr (VW == 2) {
            const float2 v = in ? *reinterpret_cast<const float2 *>(a.y + j * D + k) : make_float2(0.f, 0.f);
            ry[m][e] = v.x; ry[m][e + 1] = v.y;
          }
        }
    } else {
#pragma unroll
      for (int m = 0; m < CPT; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int k = chunk_k(m, e);
          ry[m][e] = (ok && k < D) ? a.y[j * D + k] : 0.0f;
        }
    }
  };
  auto stage_tile = [&](int buf, int64_t jt) {
    if (!stager) return;
    const bool ok = jt + sj < je;
    float ny = 0.0f;
    unsigned *rec = sRec + (buf * TJ + sj) * RS;
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = chunk_k(m, e);
        v[e] = k < D ? ry[m][e] - sCen[k < D ? k : 0] : 0.0f;
        ny = fmaf(v[e], v[e], ny);
      }
      unsigned h[4], l[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) split_bf16x2(v[2 * e], v[2 * e + 1], h[e], l[e]);
      const int c = sg + SPJ * m;
      const int off = 16 * (c >> 2) + 4 * (c & 3);
      *reinterpret_cast<u32x4s *>(rec + off) = (u32x4s){h[0], h[1], h[2], h[3]};
      *reinterpret_cast<u32x4s *>(rec + DP / 2 + off) = (u32x4s){l[0], l[1], l[2], l[3]};
    }
#pragma unroll
    for (int w = 1; w < SPJ; w *= 2) ny += __shfl_xor(ny, w);
    if (sg == 0) sNy[buf * TJ + sj] = ok ? ny : kPadU;   // padded j: u ~ kPadU, never passes
  };
  // raw coordinates of the tile (those the staging thread loaded) for the exact
  // distance, as float4 stores (a chunk is 8 consecutive coordinates, 32-byte
  // aligned; coordinates past D are 0 and land in the row's padding, or are not
  // stored where they would pass its end).  (Neither these stores, in place of
  // scalar ones, nor rows padded to start on different banks changed the LDS
  // bank-conflict count or the time at D = 64.)
  auto stage_raw = [&]() {
    if (!stager) return;
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
      const int k0 = chunk_k(m, 0);
      float *dst = sYr + sj * DX + k0;
      if (k0 + 4 <= DX) *reinterpret_cast<float4 *>(dst) = make_float4(ry[m][0], ry[m][1], ry[m][2], ry[m][3]);
      if (k0 + 8 <= DX) *reinterpret_cast<float4 *>(dst + 4) = make_float4(ry[m][4], ry[m][5], ry[m][6], ry[m][7]);
    }
  };

  if (jb < je) {
    load_tile(jb);
    stage_tile(0, jb);
    stage_raw();
  }
  __syncthreads();
  int buf = 0;
  for (int64_t jt = jb; jt < je; jt += TJ) {
    const bool has_next = jt + TJ < je;
    if (has_next) load_tile(jt + TJ);
    const int cnt = (int)(je - jt < TJ ? je - jt : TJ);
    const unsigned *yt = sRec + buf * TJ * RS;
    for (int j16 = 0; j16 < cnt; j16 += 16) {
      // A operands: split y_c of column j16 + l%16, the same coordinates as the B operands
      u32x4s yh[NS], yl[NS];
      const unsigned *src = yt + (j16 + lrow) * RS + 4 * lgrp;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        yh[s] = *reinterpret_cast<const u32x4s *>(src + 16 * s);
        yl[s] = *reinterpret_cast<const u32x4s *>(src + DP / 2 + 16 * s);
      }
      // output lane l holds j = j16 + 4(l/16) + r of row l%16: C starts at |y_c|^2 of those j
      const floatx4s c0 = *reinterpret_cast<const floatx4s *>(sNy + buf * TJ + j16 + 4 * lgrp);
      floatx4s u[TI];
#pragma unroll
      for (int t = 0; t < TI; ++t) u[t] = c0;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
#pragma unroll
        for (int t = 0; t < TI; ++t)
          u[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8s, yl[s]),
                                                         __builtin_bit_cast(bf16x8s, xh[t][s]), u[t], 0, 0, 0);
#pragma unroll
        for (int t = 0; t < TI; ++t)
          u[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8s, yh[s]),
                                                         __builtin_bit_cast(bf16x8s, xl[t][s]), u[t], 0, 0, 0);
#pragma unroll
        for (int t = 0; t < TI; ++t)
          u[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8s, yh[s]),
                                                         __builtin_bit_cast(bf16x8s, xh[t][s]), u[t], 0, 0, 0);
      }
      // one wave-uniform branch for the 4 x TI candidates of every lane
      bool any = false;
#pragma unroll
      for (int t = 0; t < TI; ++t) any |= fminf(fminf(u[t][0], u[t][1]), fminf(u[t][2], u[t][3])) < thr[t];
      if (__builtin_amdgcn_ballot_w64(any)) {
#pragma unroll
        for (int t = 0; t < TI; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int64_t j = jt + j16 + 4 * lgrp + r;
            if (u[t][r] < thr[t] && j < je && lrow_of(t) < lrows) {
              const float d2 = exact_sq_dist_lds<D>(sXr + lrow_of(t) * DX,
                                                    sYr + (j16 + 4 * lgrp + r) * DX);
              if (d2 < bd[t][K - 1]) {
                kmin_insert<K>(bd[t], bi[t], d2, (int)j);
                const float kth = bd[t][K - 1];
                const float sm = 2.0f * sqrtf(nx[t]) + sqrtf(kth);
                thr[t] = fminf(thr[t], fminf((kth - nx[t]) + mcoef * sm * sm, kThrCap));   // keep a tighter shared bound
              }
            }
          }
        // The four lane groups of a row see disjoint j and keep a list each.  A
        // candidate that fails the least of their thresholds trails K candidates
        // of that group; tighter still, every group's Q-th smallest distance
        // (Q = ceil(K/4)) is at most their largest, so the four lists together hold
        // 4Q >= K distances no larger than it: a candidate beyond that largest one
        // cannot reach the row's final K smallest, and only the final merge of the
        // four lists decides the result.  (All lanes run this: the branch is
        // wave-uniform.)
        constexpr int Q = (K + 3) / 4;
#pragma unroll
        for (int t = 0; t < TI; ++t) {
          thr[t] = fminf(thr[t], __shfl_xor(thr[t], 16));
          thr[t] = fminf(thr[t], __shfl_xor(thr[t], 32));
          float q = bd[t][Q - 1];
          q = fmaxf(q, __shfl_xor(q, 16));
          q = fmaxf(q, __shfl_xor(q, 32));
          if (q < INFINITY) {
            const float sm = 2.0f * sqrtf(nx[t]) + sqrtf(q);
            thr[t] = fminf(thr[t], (q - nx[t]) + mcoef * sm * sm);
          }
        }
      }
    }
    if (has_next) stage_tile(buf ^ 1, jt + TJ);
    __syncthreads();   // every wave past this tile's raw y
    if (has_next) {
      stage_raw();
      __syncthreads();
    }
    buf ^= 1;
  }

  // ---- merge the four lane groups' lists of each row (lanes l, l^16, l^32, l^48)
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
      if (lrow_of(t) >= lrows) continue;
      const int64_t row = wg_row0 + lrow_of(t);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        if (partial) {
          const int64_t base = ((int64_t)blockIdx.y * M + row) * K;
          a.out_d[base + k] = bd[t][k];
          a.part_idx[base + k] = bi[t][k];
        } else {
          a.out_d[row * K + k] = bd[t][k];
          a.out_idx[row * K + k] = (int64_t)bi[t][k];
        }
      }
    }
  }
}

template <int D, int K>
void launch_kmin_mfma_split_t(dim3 grid, const KminArgs &a, hipStream_t st) {
  hipLaunchKernelGGL((kmin_mfma_split_kernel<D, K>), grid, dim3(KminSplitShape<D, K>::NT), 0, st, a);
}

}  // namespace kmi
