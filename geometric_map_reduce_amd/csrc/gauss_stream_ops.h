// gauss_stream_ops.h -- pass-1 kernels of the Gaussian LogSumExp and gradient with
// respect to x for few rows and many j (KeOps pages: "Kernel Operations on the GPU,
// with Autodiff, without Memory Overflows" §2 reductions (log-sum-exp) and autodiff;
// the Falkon issue "Transparent interface for billion-scale matrices": M much
// smaller than N).
//
// The layout of the few-rows sum (gauss_stream.h): every lane owns J j's per step,
// loaded coalesced straight into registers one step ahead; the MR rows of a row
// group sit in LDS and are read with broadcast loads; each lane accumulates all MR
// rows and the work-group reduces them at the end into one partial per row.
//
// LogSumExp: each lane keeps, per (row, e), a running maximum m of its exponents
// and the sum s of exp2(v - m) over its j (an online LogSumExp: when one of a step's
// J exponents exceeds m, s is rescaled first).  The work-group merges its lanes'
// (m, s) pairs and writes (m, s) in log2 units; the split-j pass 2 merges those as
// log values.  Exponent v in log2 units, up to a per-row constant added at the end:
//   expanded (max |x'|^2 <= kFastR2 over the row group):
//       v = <2x', y'> - |y'|^2 + b log2 e,  row constant -|x'|^2;
//   direct: v = -s^2 |x - y|^2 + b log2 e.
// The running maximum leaves no range condition on b or on the distance.
// In the expanded form a first pass takes one shift per work-group and column
// instead, folded into each j's constant, so that a pair costs the sum's three
// FMAs, one exp and one add, without the running maximum:
//   M = r2 / 2 + log2 e b0   (r2 = max |x'|^2 of the group, b0 = the largest b of
// the chunk's first step).  The expanded v is at most |x'|^2 - |x' - y'|^2 + b log2 e,
// so while every b of the chunk stays below b0 + 16 a term is below 2^(64 + 23.1)
// and a sum of 2^31 of them below 2^119: no overflow.  The work-group runs the
// online pass over its chunk instead when some b exceeds b0 + 16, or when a row's
// shifted sum falls below 2^-60 (it may have lost terms below the fp32 range).
//
// Gradient: the direct form, exp2(64 - s^2 |x - y|^2) <g_i, b_j> (x - y) from raw
// differences, accumulated per (row, coordinate) with the 2^64 offset (one payload
// column: g_i factors out and is applied at the end); the partial is scaled back
// to the true value.  A non-finite sum of a row's partials (an overflow of the
// offset accumulators) is recomputed by pass 2 in double.
#pragma once

#include "common.h"
#include "gauss_stream.h"

namespace kmi {

// Loads of one step: J j's per lane; lanes past the end read the last valid j (in
// bounds) and are marked invalid.
template <int D, int E, int J>
__device__ __forceinline__ void stream_ops_load(const float *__restrict__ yb, const float *__restrict__ bb, int cnt,
                                                int off, float (&ty)[J][D], float (&tb)[J][E], bool (&ok)[J]) {
#pragma unroll
  for (int k = 0; k < J; ++k) {
    const int jl = off + k * kThreads + (int)threadIdx.x;
    ok[k] = jl < cnt;
    const int jc = ok[k] ? jl : cnt - 1;
    const float *py = yb + (int64_t)jc * D;
    const float *pb = bb + (int64_t)jc * E;
#pragma unroll
    for (int d = 0; d < D; ++d) ty[k][d] = py[d];
#pragma unroll
    for (int e = 0; e < E; ++e) tb[k][e] = pb[e];
  }
}

// Row-group set-up shared by both kernels (thread 0): centre of the group's
// bounding box into sCen and the largest |x'|^2 of its rows; returns it.
template <int D>
__device__ __forceinline__ float stream_ops_centre(const float *x, int64_t r0, int nr, float s, float *sCen,
                                                   float *sN) {
  for (int d = 0; d < D; ++d) {
    float lo = x[r0 * D + d], hi = lo;
    for (int i = 1; i < nr; ++i) {
      const float v = x[(r0 + i) * D + d];
      lo = fminf(lo, v);
      hi = fmaxf(hi, v);
    }
    sCen[d] = 0.5f * lo + 0.5f * hi;
  }
  float r2 = 0.0f;
  for (int i = 0; i < nr; ++i) {
    float n = 0.0f;
    for (int d = 0; d < D; ++d) {
      const float c = (x[(r0 + i) * D + d] - sCen[d]) * s;
      n = fmaf(c, c, n);
    }
    sN[i] = n;
    r2 = fmaxf(r2, n);
  }
  return r2;
}

// ---------------------------------------------------------------- LogSumExp
template <int D, int E, int MR>
__global__ __launch_bounds__(kThreads) void gauss_stream_lse_kernel(StreamArgs a) {
  constexpr int DP = stream_record_len<D>();
  constexpr int J = stream_j(D, E), STEP = kThreads * J;
  __shared__ __attribute__((aligned(16))) float sRow[MR * DP];
  __shared__ float sCen[D];
  __shared__ float sN[MR];
  __shared__ int sFast;
  __shared__ float sR2;
  __shared__ float sRed[kThreads / kWave][MR * E];

  const int tid = threadIdx.x;
  int64_t rg, c;
  if (!stream_place(blockIdx.x, (a.M + MR - 1) / MR, (a.N + a.j_per_wg - 1) / a.j_per_wg, rg, c)) return;
  const int64_t r0 = rg * MR;
  const int nr = (int)((a.M - r0) < MR ? (a.M - r0) : MR);   // >= 1 by the grid
  const float s = a.scale;
  if (tid == 0) {
    const float r2 = stream_ops_centre<D>(a.x, r0, nr, s, sCen, sN);
    const bool fast = a.form == FORM_AUTO && r2 <= kFastR2;
    sR2 = r2;
    for (int i = 0; i < MR; ++i)
      for (int d = 0; d < DP; ++d) {
        float v = 0.0f;
        if (i < nr && d < D) {
          const float xv = a.x[(r0 + i) * D + d];
          v = fast ? (2.0f * s) * ((xv - sCen[d]) * s) : xv;
        }
        sRow[i * DP + d] = v;
      }
    // the rows' constants in log2 units: -|x'|^2 (expanded), 0 (direct)
    for (int i = 0; i < MR; ++i) sN[i] = (fast && i < nr) ? -sN[i] : 0.0f;
    sFast = fast ? 1 : 0;
  }
  __syncthreads();
  const bool fast = __builtin_amdgcn_readfirstlane(sFast) != 0;
  float cen[D];
#pragma unroll
  for (int d = 0; d < D; ++d) cen[d] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sCen[d])));

  float m[MR][E], sm[MR][E];

  const int64_t jb = c * a.j_per_wg;
  const int cnt = (int)((jb + a.j_per_wg < a.N) ? a.j_per_wg : a.N - jb);   // >= 1 by the grid
  const float *yb = a.y + jb * D, *bb = a.b + jb * E;
  const float s2 = s * s;
  const int wid = tid / kWave, lane = tid & (kWave - 1);
  float ty[J][D], tb[J][E];
  bool ok[J];

  // ---- expanded form: one shift per work-group and column, M = r2 / 2 + log2 e b0
  if (fast) {
    __shared__ float sB0[E];
    __shared__ int sRedo;
    stream_ops_load<D, E, J>(yb, bb, cnt, 0, ty, tb, ok);
    float bm[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      bm[e] = -INFINITY;
#pragma unroll
      for (int k = 0; k < J; ++k) bm[e] = ok[k] ? fmaxf(bm[e], tb[k][e]) : bm[e];
      const float w = wave_max(bm[e]);
      if (lane == 0) sRed[wid][e] = w;
    }
    if (tid == 0) sRedo = 0;
    __syncthreads();
    if (tid < E) {
      float w = sRed[0][tid];
#pragma unroll
      for (int q = 1; q < kThreads / kWave; ++q) w = fmaxf(w, sRed[q][tid]);
      sB0[tid] = w;
    }
    __syncthreads();
    float Ms[E], bcap[E];
    bool finite = true;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float b0 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sB0[e])));
      Ms[e] = fmaf(kLog2e, b0, 0.5f * sR2);
      bcap[e] = b0 + 16.0f;
      finite = finite && isfinite(Ms[e]);   // else (all -inf, or an infinite b): the online pass
    }
    if (finite) {   // uniform
      bool over = false;   // some b of this lane above b0 + 16
#pragma unroll
      for (int i = 0; i < MR; ++i)
#pragma unroll
        for (int e = 0; e < E; ++e) sm[i][e] = 0.0f;
      for (int off = 0; off < cnt; off += STEP) {
        // per j: the centred y and its constant b log2 e - s^2 |y - c|^2 - M
        float cj[J][E];
        float u[J][D];
#pragma unroll
        for (int k = 0; k < J; ++k) {
          float n = 0.0f;
#pragma unroll
          for (int d = 0; d < D; ++d) {
            u[k][d] = ty[k][d] - cen[d];
            n = fmaf(u[k][d], u[k][d], n);
          }
#pragma unroll
          for (int e = 0; e < E; ++e) {
            cj[k][e] = ok[k] ? fmaf(kLog2e, tb[k][e], fmaf(-s2, n, -Ms[e])) : -INFINITY;
            over = over || (ok[k] && !(tb[k][e] <= bcap[e]));   // NaN b too: the online pass decides
          }
        }
        if (off + STEP < cnt) stream_ops_load<D, E, J>(yb, bb, cnt, off + STEP, ty, tb, ok);   // next step in flight
        asm volatile("" ::: "memory");   // row records from LDS each step, not held in registers
#pragma unroll
        for (int i = 0; i < MR; ++i) {
          float r[DP];
          const float4 *src = reinterpret_cast<const float4 *>(sRow + i * DP);
#pragma unroll
          for (int q = 0; q < DP / 4; ++q) {
            const float4 v = src[q];
            r[4 * q] = v.x; r[4 * q + 1] = v.y; r[4 * q + 2] = v.z; r[4 * q + 3] = v.w;
          }
#pragma unroll
          for (int k = 0; k < J; ++k) {
            if (E == 1) {
              float q = cj[k][0];
#pragma unroll
              for (int d = 0; d < D; ++d) q = fmaf(r[d], u[k][d], q);
              sm[i][0] += fast_exp2(q);
            } else {
              float q = 0.0f;
#pragma unroll
              for (int d = 0; d < D; ++d) q = fmaf(r[d], u[k][d], q);
#pragma unroll
              for (int e = 0; e < E; ++e) sm[i][e] += fast_exp2(q + cj[k][e]);
            }
          }
        }
      }
      // work-group sums; a row below 2^-60 sends the work-group to the online pass
#pragma unroll
      for (int i = 0; i < MR; ++i)
#pragma unroll
        for (int e = 0; e < E; ++e) {
          float v = row16_sum(sm[i][e]);
          v += __shfl_xor(v, 16);
          v += __shfl_xor(v, 32);
          if (lane == 0) sRed[wid][i * E + e] = v;
        }
      if (over) sRedo = 1;
      __syncthreads();
      float tot = 0.0f;
      if (tid < nr * E) {
        tot = sRed[0][tid];
#pragma unroll
        for (int q = 1; q < kThreads / kWave; ++q) tot += sRed[q][tid];
        if (!(tot >= 0x1p-60f)) sRedo = 1;
      }
      __syncthreads();
      if (!sRedo) {   // uniform
        if (tid < nr * E) {
          const int i = tid / E, e = tid - i * E;
          float *dst = a.part + ((c * a.M + r0 + i) * E + e) * 2;
          dst[0] = Ms[e] + sN[i];
          dst[1] = tot;
        }
        return;
      }
      __syncthreads();   // sRed is reused below
    }
  }

  // ---- online pass: a running maximum per (row, e) in each lane
#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int e = 0; e < E; ++e) { m[i][e] = -3.0e38f; sm[i][e] = 0.0f; }
  stream_ops_load<D, E, J>(yb, bb, cnt, 0, ty, tb, ok);
  for (int off = 0; off < cnt; off += STEP) {
    // this step's j: per-j constants (b log2 e, and -|y'|^2 for the expanded form)
    float cj[J][E];
    float u[J][D];
#pragma unroll
    for (int k = 0; k < J; ++k) {
      float n = 0.0f;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        u[k][d] = fast ? ty[k][d] - cen[d] : ty[k][d];
        n = fmaf(u[k][d], u[k][d], n);
      }
#pragma unroll
      for (int e = 0; e < E; ++e) cj[k][e] = ok[k] ? fmaf(kLog2e, tb[k][e], fast ? -s2 * n : 0.0f) : -INFINITY;
    }
    if (off + STEP < cnt) stream_ops_load<D, E, J>(yb, bb, cnt, off + STEP, ty, tb, ok);   // next step in flight
    asm volatile("" ::: "memory");   // row records from LDS each step, not held in registers
#pragma unroll
    for (int i = 0; i < MR; ++i) {
      float r[DP];
      const float4 *src = reinterpret_cast<const float4 *>(sRow + i * DP);
#pragma unroll
      for (int q = 0; q < DP / 4; ++q) {
        const float4 v = src[q];
        r[4 * q] = v.x; r[4 * q + 1] = v.y; r[4 * q + 2] = v.z; r[4 * q + 3] = v.w;
      }
      float v0[J];
#pragma unroll
      for (int k = 0; k < J; ++k) {
        float q = 0.0f;
        if (fast) {
#pragma unroll
          for (int d = 0; d < D; ++d) q = fmaf(r[d], u[k][d], q);
        } else {
#pragma unroll
          for (int d = 0; d < D; ++d) {
            const float df = r[d] - u[k][d];
            q = fmaf(df, df, q);
          }
          q *= -s2;
        }
        v0[k] = q;
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float v[J];
        float vmax = -INFINITY;
#pragma unroll
        for (int k = 0; k < J; ++k) {
          v[k] = v0[k] + cj[k][e];
          vmax = fmaxf(vmax, v[k]);
        }
        if (vmax > m[i][e]) {          // rare once the lane has seen a few j
          sm[i][e] *= fast_exp2(m[i][e] - vmax);
          m[i][e] = vmax;
        }
#pragma unroll
        for (int k = 0; k < J; ++k) sm[i][e] += fast_exp2(v[k] - m[i][e]);
      }
    }
  }

  // ---- merge the lanes' (m, s) per (row, e): maximum, then the rescaled sums
  __shared__ float sMax[MR * E];
#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float w = wave_max(m[i][e]);
      if (lane == 0) sRed[wid][i * E + e] = w;
    }
  __syncthreads();
  if (tid < MR * E) {
    float w = sRed[0][tid];
#pragma unroll
    for (int q = 1; q < kThreads / kWave; ++q) w = fmaxf(w, sRed[q][tid]);
    sMax[tid] = w;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float v = sm[i][e] * fast_exp2(m[i][e] - sMax[i * E + e]);
      v = row16_sum(v);
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (lane == 0) sRed[wid][i * E + e] = v;
    }
  __syncthreads();
  if (tid < nr * E) {
    const int i = tid / E, e = tid - i * E;
    float v = sRed[0][tid];
#pragma unroll
    for (int q = 1; q < kThreads / kWave; ++q) v += sRed[q][tid];
    float *dst = a.part + ((c * a.M + r0 + i) * E + e) * 2;
    dst[0] = sMax[tid] + sN[i];
    dst[1] = v;
  }
}

// ---------------------------------------------------------------- gradient
// j per lane per step of the gradient: 2, where the sum takes 4 up to D + E = 8 (at 16
// rows x 1e8, D = 3, pass 1 took 0.540 ms with 2, 0.550 with 4 and 0.557 with 8; at 64
// rows 1.91, 1.99 and 2.09 ms): its 12 VALU instructions per pair already hide the
// loads.  The launch plan keeps the sum's step (a multiple of this one).
constexpr int stream_grad_j(int, int) { return 2; }

template <int D, int E, int MR>
__global__ __launch_bounds__(kThreads) void gauss_stream_grad_kernel(StreamArgs a) {
  constexpr int DP = stream_record_len<D>();
  constexpr int J = stream_grad_j(D, E), STEP = kThreads * J;
  __shared__ __attribute__((aligned(16))) float sRow[MR * DP];
  __shared__ float sG[MR * E];
  __shared__ float sRed[kThreads / kWave][MR * D];

  const int tid = threadIdx.x;
  int64_t rg, c;
  if (!stream_place(blockIdx.x, (a.M + MR - 1) / MR, (a.N + a.j_per_wg - 1) / a.j_per_wg, rg, c)) return;
  const int64_t r0 = rg * MR;
  const int nr = (int)((a.M - r0) < MR ? (a.M - r0) : MR);
  for (int f = tid; f < MR * DP; f += kThreads) {
    const int i = f / DP, d = f - i * DP;
    sRow[f] = (i < nr && d < D) ? a.x[(r0 + i) * D + d] : 0.0f;
  }
  for (int f = tid; f < MR * E; f += kThreads) {
    const int i = f / E;
    sG[f] = i < nr ? a.g[(r0 + i) * E + (f - i * E)] : 0.0f;
  }
  __syncthreads();

  float acc[MR][D];
#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int d = 0; d < D; ++d) acc[i][d] = 0.0f;

  const int64_t jb = c * a.j_per_wg;
  const int cnt = (int)((jb + a.j_per_wg < a.N) ? a.j_per_wg : a.N - jb);
  const float *yb = a.y + jb * D, *bb = a.b + jb * E;
  const float s2 = a.scale * a.scale;
  float ty[J][D], tb[J][E];
  bool ok[J];
  stream_ops_load<D, E, J>(yb, bb, cnt, 0, ty, tb, ok);
  for (int off = 0; off < cnt; off += STEP) {
    float u[J][D], bj[J][E];
#pragma unroll
    for (int k = 0; k < J; ++k) {
#pragma unroll
      for (int d = 0; d < D; ++d) u[k][d] = ty[k][d];
#pragma unroll
      for (int e = 0; e < E; ++e) bj[k][e] = ok[k] ? tb[k][e] : 0.0f;
    }
    if (off + STEP < cnt) stream_ops_load<D, E, J>(yb, bb, cnt, off + STEP, ty, tb, ok);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < MR; ++i) {
      float r[DP];
      const float4 *src = reinterpret_cast<const float4 *>(sRow + i * DP);
#pragma unroll
      for (int q = 0; q < DP / 4; ++q) {
        const float4 v = src[q];
        r[4 * q] = v.x; r[4 * q + 1] = v.y; r[4 * q + 2] = v.z; r[4 * q + 3] = v.w;
      }
#pragma unroll
      for (int k = 0; k < J; ++k) {
        float df[D];
        float q = 0.0f;
#pragma unroll
        for (int d = 0; d < D; ++d) {
          df[d] = r[d] - u[k][d];
          q = fmaf(df[d], df[d], q);
        }
        float gb;
        if (E == 1) {
          gb = bj[k][0];
        } else {
          gb = 0.0f;
#pragma unroll
          for (int e = 0; e < E; ++e) gb = fmaf(sG[i * E + e], bj[k][e], gb);
        }
        const float w = fast_exp2(fmaf(-s2, q, kDirectOffset)) * gb;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[i][d] = fmaf(w, df[d], acc[i][d]);
      }
    }
  }

  // ---- reduce every (row, coordinate) over the work-group, scale back, store
  const int wid = tid / kWave, lane = tid & (kWave - 1);
#pragma unroll
  for (int i = 0; i < MR; ++i) {
    if (i < nr) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        float v = row16_sum(acc[i][d]);
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (lane == 0) sRed[wid][i * D + d] = v;
      }
    }
  }
  __syncthreads();
  if (tid < nr * D) {
    const int i = tid / D, d = tid - i * D;
    float v = sRed[0][tid];
#pragma unroll
    for (int q = 1; q < kThreads / kWave; ++q) v += sRed[q][tid];
    const float gf = a.coef * (E == 1 ? sG[i] : 1.0f);
    a.part[(c * a.M + r0 + i) * D + d] = (v * exp2f(-kDirectOffset)) * gf;
  }
}

template <int D, int E, int MR>
void launch_gauss_stream_lse_t(dim3 grid, const StreamArgs &a, hipStream_t st) {
  hipLaunchKernelGGL((gauss_stream_lse_kernel<D, E, MR>), grid, dim3(kThreads), 0, st, a);
}

template <int D, int E, int MR>
void launch_gauss_stream_grad_t(dim3 grid, const StreamArgs &a, hipStream_t st) {
  hipLaunchKernelGGL((gauss_stream_grad_kernel<D, E, MR>), grid, dim3(kThreads), 0, st, a);
}

}  // namespace kmi
