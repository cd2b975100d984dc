// gauss_stream.h -- pass-1 kernel of the Gaussian sum for few rows and many j
// (KeOps pages: "Kernel Operations on the GPU, with Autodiff, without Memory
// Overflows" §1, target operation a_i = sum_j K(x_i, y_j) b_j; the Falkon issue
// "Transparent interface for billion-scale matrices": M much smaller than N).
//
// With M of a few dozen rows the row-per-lane layout would leave most lanes
// without a row, and the work is bound by streaming y and b from HBM once.
// Here the roles swap: every lane owns J j's per step (coalesced loads straight
// into registers, prefetched one step ahead), and the MR rows of one row group
// (MR = 4, or up to 16 where the accumulators allow) sit in LDS, read with
// broadcast loads.  Each lane accumulates all MR rows;
// the work-group reduces them across lanes at the end and writes one partial
// per row, which a double-precision pass 2 sums over the work-groups in order.
//
// Distance forms are those of the row-per-lane kernel, with x and y swapped:
//   expanded: exp2(<2x', y'> - |y'|^2 - G) * exp2(G - |x'|^2), centre and G from
//             the row group's bounding box, valid while max |x'|^2 <= kFastR2
//             (rows stored as 2 s x', j's as y - c, so the scale is paid per row);
//   direct:   exp2(64 - s^2 sum_d (x_d - y_d)^2) * 2^-64 from raw differences.
#pragma once

#include "common.h"
#include "launch.h"

namespace kmi {

// j per lane per step: four, or two where the rows' coordinates and payloads
// are wide (keeps the register buffers and the row records in VGPRs).
constexpr int stream_j(int D, int E) { return D + E <= 8 ? 4 : 2; }
// Rows per row group of the large variant (the small one has 4) are
// stream_rows_large(D, E) in launch.h: the row accumulators, MR x E, stay at
// 16 registers, and at 8 from D = 5 on.
constexpr int stream_mr_large(int D, int E) { return stream_rows_large(D, E); }
// Minimum waves per SIMD asked of the compiler: four where the variant fits
// 128 VGPRs without spilling (checked in the compiled code), else no bound.
constexpr int stream_waves(int D, int E, int MR) { return (D <= 3 && E == 1) || MR * (D + E) <= 32 ? 4 : 1; }

template <int D>
constexpr int stream_record_len() { return (D + 3) / 4 * 4; }   // LDS floats per row

// One step: J j's per lane against the MR rows in LDS (rows past the group's
// end hold zeros and are computed but never stored).  ty is transformed in place.
// For each j, rows go in phases of RC: RC exponents, RC exps, RC accumulations,
// so every phase holds RC independent chains.
template <int D, int E, int MR, int J, bool FAST>
__device__ __forceinline__ void stream_step(float (&ty)[J][D], const float (&tb)[J][E], const float *sRow,
                                            const float (&cen)[D], float s, float G, float (&acc)[MR][E]) {
  constexpr int DP = stream_record_len<D>();
  float cj[J];
  if (FAST) {
    // u = y - c and c_j = -s^2 |u|^2 - G, once per j for all rows; the rows
    // hold 2 s^2 (x - c), so <row, u> + c_j = 2<x', y'> - |y'|^2 - G
#pragma unroll
    for (int k = 0; k < J; ++k) {
      float n = 0.0f;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        ty[k][d] -= cen[d];
        n = fmaf(ty[k][d], ty[k][d], n);
      }
      cj[k] = fmaf(-s * s, n, -G);
    }
  }
  const float s2 = s * s;
  // Row records are re-read from LDS every step (a compiler barrier keeps them
  // out of registers); the registers go to RC independent chains per phase.
  asm volatile("" ::: "memory");
  constexpr int RC = MR < 8 ? MR : 8;
#pragma unroll
  for (int k = 0; k < J; ++k) {
#pragma unroll
    for (int h = 0; h < MR; h += RC) {
      float ex[RC];
#pragma unroll
      for (int c = 0; c < RC; ++c) {
        float r[DP];
        const float4 *src = reinterpret_cast<const float4 *>(sRow + (h + c) * DP);
#pragma unroll
        for (int q = 0; q < DP / 4; ++q) {
          const float4 v = src[q];
          r[4 * q] = v.x; r[4 * q + 1] = v.y; r[4 * q + 2] = v.z; r[4 * q + 3] = v.w;
        }
        if (FAST) {
          float e = cj[k];
#pragma unroll
          for (int d = 0; d < D; ++d) e = fmaf(r[d], ty[k][d], e);
          ex[c] = e;
        } else {
          float q = 0.0f;
#pragma unroll
          for (int d = 0; d < D; ++d) {
            const float df = r[d] - ty[k][d];
            q = fmaf(df, df, q);
          }
          ex[c] = fmaf(-s2, q, kDirectOffset);
        }
      }
#pragma unroll
      for (int c = 0; c < RC; ++c) ex[c] = fast_exp2(ex[c]);
#pragma unroll
      for (int c = 0; c < RC; ++c)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h + c][e] = fmaf(ex[c], tb[k][e], acc[h + c][e]);
    }
  }
}

// The work-group's j range [jb, jb + cnt): two register buffers, each loaded
// one step ahead of its use.  Lanes past the end read the last valid j (always
// in bounds) with b = 0, so they add nothing.
template <int D, int E, int MR, bool FAST>
__device__ __forceinline__ void stream_jloop(const StreamArgs &a, const float *sRow, const float (&cen)[D],
                                             float G, int64_t jb, int cnt, float (&acc)[MR][E], float &bmx) {
  constexpr int J = stream_j(D, E), STEP = kThreads * J;
  const int tid = threadIdx.x;
  const float s = a.scale;
  const float *__restrict__ yb = a.y + jb * D;
  const float *__restrict__ bb = a.b + jb * E;
  auto load = [&](float (&ty)[J][D], float (&tb)[J][E], int off) {
#pragma unroll
    for (int k = 0; k < J; ++k) {
      const int jl = off + k * kThreads + tid;
      const bool ok = jl < cnt;
      const int jc = ok ? jl : cnt - 1;
      const float *py = yb + (int64_t)jc * D;
      const float *pb = bb + (int64_t)jc * E;
#pragma unroll
      for (int d = 0; d < D; ++d) ty[k][d] = py[d];
#pragma unroll
      for (int e = 0; e < E; ++e) tb[k][e] = ok ? pb[e] : 0.0f;
    }
  };
  // max |b| for the underflow guard, one per j (not per pair), taken when the
  // payload is used so that the loads stay one step ahead
  auto track = [&](const float (&tb)[J][E]) {
#pragma unroll
    for (int k = 0; k < J; ++k)
#pragma unroll
      for (int e = 0; e < E; ++e) bmx = fmaxf(bmx, fabsf(tb[k][e]));
  };
  float y0[J][D], b0[J][E], y1[J][D], b1[J][E];
  load(y0, b0, 0);
  for (int off = 0; off < cnt; off += 2 * STEP) {
    load(y1, b1, off + STEP);
    stream_step<D, E, MR, J, FAST>(y0, b0, sRow, cen, s, G, acc);
    track(b0);
    if (off + STEP < cnt) {            // wave-uniform
      load(y0, b0, off + 2 * STEP);
      stream_step<D, E, MR, J, FAST>(y1, b1, sRow, cen, s, G, acc);
      track(b1);
    }
  }
}

// Work-group w of the one-dimensional grid of 8 G ceil(C / 8) work-groups (G row
// groups, C chunks of j) -> (row group rg, chunk c).  Chunk c goes to XCD c % 8 (the
// dispatcher hands out ids round-robin over the eight), and the G row groups of a
// chunk get consecutive ids among that XCD's, so they run together and all but the
// first read the chunk's y and b from the XCD's L2 (with the chunk's row groups far
// apart in the grid, each read it from HBM).  Returns false for the padding ids
// (c >= C), which exit at once.
__device__ __forceinline__ bool stream_place(int64_t w, int64_t G, int64_t C, int64_t &rg, int64_t &c) {
  const int64_t xcd = w & 7, k = w >> 3;
  rg = k % G;
  c = (k / G) * 8 + xcd;
  return c < C;
}

template <int D, int E, int MR>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(stream_waves(D, E, MR))))
void gauss_stream_kernel(StreamArgs a) {
  constexpr int DP = stream_record_len<D>();
  __shared__ __attribute__((aligned(16))) float sRow[MR * DP];
  __shared__ float sCen[D];
  __shared__ float sFac[MR];
  __shared__ float sG;
  __shared__ int sFast;
  __shared__ float sRed[kThreads / kWave][MR * E];
  __shared__ float sBm[kThreads / kWave];

  const int tid = threadIdx.x;
  int64_t rg, c;
  if (!stream_place(blockIdx.x, (a.M + MR - 1) / MR, (a.N + a.j_per_wg - 1) / a.j_per_wg, rg, c)) return;
  const int64_t r0 = rg * MR;
  const int nr = (int)((a.M - r0) < MR ? (a.M - r0) : MR);   // >= 1 by the grid

  // ---- row group set-up: one thread, at most MR x D values
  if (tid == 0) {
    const float s = a.scale;
    for (int d = 0; d < D; ++d) {
      float lo = a.x[r0 * D + d], hi = lo;
      for (int i = 1; i < nr; ++i) {
        const float v = a.x[(r0 + i) * D + d];
        lo = fminf(lo, v);
        hi = fmaxf(hi, v);
      }
      sCen[d] = 0.5f * lo + 0.5f * hi;
    }
    float r2 = 0.0f;
    for (int i = 0; i < nr; ++i) {
      float n = 0.0f;
      for (int d = 0; d < D; ++d) {
        const float c = (a.x[(r0 + i) * D + d] - sCen[d]) * s;
        n = fmaf(c, c, n);
      }
      sFac[i] = n;                        // |x'_i|^2 for now
      r2 = fmaxf(r2, n);
    }
    const bool fast = a.form == FORM_AUTO && r2 <= kFastR2;
    const float G = 0.5f * r2;
    for (int i = 0; i < MR; ++i) {
      for (int d = 0; d < DP; ++d) {
        float v = 0.0f;
        if (i < nr && d < D) {
          const float xv = a.x[(r0 + i) * D + d];
          v = fast ? (2.0f * s) * ((xv - sCen[d]) * s) : xv;
        }
        sRow[i * DP + d] = v;
      }
      sFac[i] = i < nr ? (fast ? exp2f(G - sFac[i]) : exp2f(-kDirectOffset)) : 0.0f;
    }
    sG = G;
    sFast = fast ? 1 : 0;
    if (a.row_fac && c == 0)
      for (int i = 0; i < nr; ++i) a.row_fac[r0 + i] = fast ? sFac[i] : -1.0f;
  }
  __syncthreads();

  // uniform across the work-group: held in scalar registers
  float cen[D];
#pragma unroll
  for (int d = 0; d < D; ++d) cen[d] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sCen[d])));
  const float Gs = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sG)));
  float acc[MR][E];
#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[i][e] = 0.0f;

  const int64_t jb = c * a.j_per_wg;
  const int cnt = (int)((jb + a.j_per_wg < a.N) ? a.j_per_wg : a.N - jb);   // >= 1 by the grid
  float bmx = 0.0f;
  if (sFast) stream_jloop<D, E, MR, true>(a, sRow, cen, Gs, jb, cnt, acc, bmx);
  else stream_jloop<D, E, MR, false>(a, sRow, cen, Gs, jb, cnt, acc, bmx);

  // ---- reduce every (row, e) over the work-group: DPP rows, shuffles, then LDS
  const int wid = tid / kWave, lane = tid & (kWave - 1);
#pragma unroll
  for (int i = 0; i < MR; ++i) {
    if (i < nr) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float v = row16_sum(acc[i][e]);
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (lane == 0) sRed[wid][i * E + e] = v;
      }
    }
  }
  if (a.chunk_bmax && rg == 0) {
    const float m = wave_max(bmx);
    if (lane == 0) sBm[wid] = m;
  }
  __syncthreads();
  if (a.chunk_bmax && rg == 0 && tid == 0) {
    float m = sBm[0];
#pragma unroll
    for (int w = 1; w < kThreads / kWave; ++w) m = fmaxf(m, sBm[w]);
    a.chunk_bmax[c] = m;
  }
  if (tid < nr * E) {
    const int i = tid / E, e = tid - i * E;
    float v = sRed[0][tid];
#pragma unroll
    for (int w = 1; w < kThreads / kWave; ++w) v += sRed[w][tid];
    a.part[(c * a.M + r0 + i) * E + e] = v * sFac[i];
  }
}

template <int D, int E, int MR>
void launch_gauss_stream_t(dim3 grid, const StreamArgs &a, hipStream_t st) {
  hipLaunchKernelGGL((gauss_stream_kernel<D, E, MR>), grid, dim3(kThreads), 0, st, a);
}

}  // namespace kmi
