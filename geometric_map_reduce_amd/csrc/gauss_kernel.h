// gauss_kernel.h -- pass-1 kernel of the Gaussian sum, LogSumExp, grad_x and
// Max/ArgMax reductions, and of the Laplacian kernel sum, on gfx950 VALU (the
// D < 32 hot path; also the reference VALU path at large D).
//
// Operation (KeOps pages: "Kernel Operations on the GPU, with Autodiff,
// without Memory Overflows" §1 "Target operation" and §2; KeOps README
// example): for each row i, reduce over j the Gaussian coefficients
// K_ij = exp(-|x_i - y_j|^2 / sigma^2) without storing them.
//
// Layout of one work-group (256 threads = 4 wave64):
//   * rows: thread t owns rows i = row0 + r*256 + t, r < R, held in VGPRs;
//   * j-tiles: TJ rows of y (and b) are read from HBM with coalesced loads,
//     transformed once per work-group and stored in LDS as one record per j;
//     all lanes then read the same record (broadcast ds_read_b128);
//   * double-buffered LDS: the next tile's global loads are in flight while
//     the current tile is reduced; one barrier per tile;
//   * per-tile partial sums, folded into the row accumulators at the end of
//     each tile, so that a long j range does not round small terms away;
//   * split-j: blockIdx.y selects a j-range; partial results go to a
//     workspace that a second kernel combines.
//
// Two forms of the pair map, chosen once per work-group:
//   EXPANDED: coordinates centred on the work-group's bounding-box centre c
//            and scaled by s = sqrt(log2 e)/sigma (x' = s(x - c)), so that
//            K_ij = exp2(<x'_i, 2y'_j> + c_j) * exp2(G - |x'_i|^2) with
//            c_j = -|y'_j|^2 - G.  Three FMAs and one v_exp_f32 per pair at
//            D = 3; the row factor is applied once per row at the end.  Used
//            when max_i |x'_i|^2 <= kFastR2 over the work-group, which bounds
//            both the exponent range (|exponent| <= 64 + |x'-y'|^2) and the
//            rounding of the expansion (about 1e-5 relative in K_ij).
//   DIRECT  : K_ij = exp2(-s^2 sum_k (x_k - y_k)^2) from raw coordinates (the
//            difference is taken first, so far-apart or far-from-origin
//            points keep full relative precision); the fallback.  Sums and
//            gradients evaluate exp2(64 - s^2 |x - y|^2) and scale the row by
//            2^-64 at the end, which moves the flush-to-zero floor of
//            v_exp_f32 from 2^-126 to 2^-190 (a gradient multiplies tiny
//            K_ij by (2/sigma^2)|x - y| and can lift them into range).
#pragma once

#include <type_traits>

#include "common.h"

namespace kmi {

template <int OP, int D, int E>
struct GaussShape {
  static constexpr int NV = (D + 1 + 3) / 4;                              // float4 per j record
  static constexpr int PAY = E;                                           // payload floats per j (b)
  // per-row accumulators: sum E; LSE (max, sum) per column; grad D; max E (with indices;
  // 2 for the sign-split tile: best positive and best negative class)
  static constexpr int NACC = (OP == OP_GRAD) ? D : ((OP == OP_LSE || OP == OP_MAX) ? 2 * E : E);
  // per-tile partial sums: sum E; LSE E; grad D
  static constexpr int NPART = (OP == OP_GRAD) ? D : E;
  static constexpr int BYTES_PER_J = NV * 16 + PAY * 4;
  static constexpr int TJ = (2 * 256 * BYTES_PER_J <= 49152) ? 256
                          : (2 * 128 * BYTES_PER_J <= 49152) ? 128
                          : (2 * 64 * BYTES_PER_J <= 49152) ? 64
                          : (2 * 32 * BYTES_PER_J <= 49152) ? 32 : 16;
  // Sign-split tile (sum and Max with one payload column, expanded form, D <= 8):
  // the tile's j are stored with b > 0 first and the rest after (each class in j
  // order, padded to whole groups of 4); log2 |b| is folded into the j constant, so
  // the sum adds or subtracts exp2 of the exponent and Max compares exponents
  // without any exp2.
  static constexpr bool SPLIT = (OP == OP_SUM || OP == OP_MAX || OP == OP_GRAD) && E == 1 && D <= 8 && TJ == 256;
  static constexpr int TJR = SPLIT ? TJ + 8 : TJ;   // records per tile buffer
};

// Record of one j (NV float4 from LDS) into registers.
template <int NV>
__device__ __forceinline__ void load_rec(const float4 *rec, int j, float (&yv)[4 * NV]) {
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const float4 t = rec[j * NV + v];
    yv[4 * v] = t.x; yv[4 * v + 1] = t.y; yv[4 * v + 2] = t.z; yv[4 * v + 3] = t.w;
  }
}

// Exponent (log2 units) of the pair map for R rows and one j record, phase by
// phase over the rows so that the R chains are independent.
//   EXPANDED: q_r = <x'_r, 2y'> + c_j      (xs = x', record = (2y', c_j))
//   DIRECT  : q_r = off_r - s^2 |x_r - y|^2  (xs = raw x, record = raw y); the
//             differences are kept in d for the grad_x accumulation.
//   LAPLACE : q_r = off_r - s2 |x_r - y|      (direct form only; s2 = log2 e / sigma)
template <bool FAST, int R, int D, int NV4, bool LAPLACE = false>
__device__ __forceinline__ void pair_exponent(const float (&xs)[R][D], const float (&yv)[NV4], float s2,
                                              const float (&off)[R],
                                              float (&q)[R], float (&d)[FAST ? 1 : R][D]) {
  if (FAST) {
#pragma unroll
    for (int r = 0; r < R; ++r) q[r] = yv[D];
#pragma unroll
    for (int k = 0; k < D; ++k)
#pragma unroll
      for (int r = 0; r < R; ++r) q[r] = fmaf(xs[r][k], yv[k], q[r]);
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int k = 0; k < D; ++k) d[FAST ? 0 : r][k] = xs[r][k] - yv[k];
#pragma unroll
    for (int r = 0; r < R; ++r) q[r] = 0.0f;
#pragma unroll
    for (int k = 0; k < D; ++k)
#pragma unroll
      for (int r = 0; r < R; ++r) q[r] = fmaf(d[FAST ? 0 : r][k], d[FAST ? 0 : r][k], q[r]);
    if (LAPLACE) {
#pragma unroll
      for (int r = 0; r < R; ++r) q[r] = __builtin_amdgcn_sqrtf(q[r]);   // v_sqrt_f32, about 1 ulp
    }
#pragma unroll
    for (int r = 0; r < R; ++r) q[r] = fmaf(-s2, q[r], off[r]);
  }
}

// Expanded-form records [j0, j1) (a multiple of 4) visited in groups of 4,
// with the next group's records read from LDS as soon as this group's
// exponents are formed, into the same registers: the read's latency then
// hides behind this group's exp2 and accumulation.  The last group re-reads
// itself.  visit(q) receives the exponents q[R] of one record, in j order.
// The visitor must read nothing from LDS: a wait for such a read would also
// wait for the records in flight.
template <int NV, int R, int D, typename Visit>
__device__ __forceinline__ void pipelined_records(const float4 *rec, int j0, int j1, const float (&xs)[R][D],
                                                  float s2, Visit &&visit) {
  if (j0 >= j1) return;
  float yv[4][4 * NV];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    load_rec<NV>(rec, j0 + u, yv[u]);
    // opaque, so that the compiler cannot merge this read with the one in
    // the loop into a single read at the top of each iteration
#pragma unroll
    for (int k = 0; k < 4 * NV; ++k) asm volatile("" : "+v"(yv[u][k]));
  }
  const float nooff[R] = {};   // the expanded form reads no offset
  for (int jj = j0; jj < j1; jj += 4) {
    float q[4][R], dd[1][D];
#pragma unroll
    for (int u = 0; u < 4; ++u) pair_exponent<true>(xs, yv[u], s2, nooff, q[u], dd);
    const int jn = jj + 4 < j1 ? jj + 4 : jj;
#pragma unroll
    for (int u = 0; u < 4; ++u) load_rec<NV>(rec, jn + u, yv[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u) visit(q[u]);
  }
}

// The j loop of one work-group over [jb, je) for a fixed form (FAST = expanded
// distance).  Starts and ends with every wave past the LDS buffers, so calls
// can follow each other (one per j range in block-sparse launches).
// FIXED (LogSumExp, expanded form only): the exponent is taken relative to a
// shift fixed per row in advance instead of a running maximum, so a pair costs
// what it costs in the sum (exponent, exp2, add); see the kernel below.
template <int OP, int D, int E, int R, bool FAST, bool FIXED = false>
__device__ __forceinline__ void gauss_jloop(const GaussArgs &a,
                                            float4 (*sRec)[GaussShape<OP, D, E>::TJR * GaussShape<OP, D, E>::NV],
                                            float (*sPay)[GaussShape<OP, D, E>::PAY * GaussShape<OP, D, E>::TJ],
                                            int (*sIdx)[GaussShape<OP, D, E>::TJR], int (*sSeg)[4],
                                            const float (&xs)[R][D], const float (&gr)[R][E], const float (&cen)[D],
                                            float G, const float (&off)[R],
                                            float (&acc)[R][GaussShape<OP, D, E>::NACC], int (&ix)[R][2 * E],
                                            float &bmx, int64_t jb, int64_t je) {
  using S = GaussShape<OP, D, E>;
  constexpr int NV = S::NV, PAY = S::PAY, TJ = S::TJ, NP = S::NPART;
  constexpr bool SPLIT = S::SPLIT && FAST;
  const int tid = threadIdx.x;
  const float s2 = a.scale * a.scale;
  // off: each row's exponent offset in the direct form (not read by the expanded form;
  // 0 for LogSumExp, which tracks its own maximum)
  // the j range is uniform across the work-group: keep the tile loop's control scalar
  jb = uniform_i64(jb);
  je = uniform_i64(je);

  // raw tile registers (one j per thread for tid < TJ)
  float ry[D], rb[E];
  auto load_raw = [&](int64_t jt) {
    const int64_t j = jt + tid;
    const bool ok = (tid < TJ) && (j < je);
#pragma unroll
    for (int k = 0; k < D; ++k) ry[k] = ok ? a.y[j * D + k] : 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) rb[e] = ok ? a.b[j * E + e] : 0.0f;
    return ok;
  };
  // Transform the staged raw j rows into LDS records and payloads.  Padded j
  // (beyond je) get records whose contribution is exactly zero.
  // a record whose exponent slot holds c and every other value 0
  auto put_pad = [&](int buf, int slot, float c) {
    float pr[4 * NV];
#pragma unroll
    for (int q = 0; q < 4 * NV; ++q) pr[q] = 0.0f;
    pr[D] = c;
#pragma unroll
    for (int v = 0; v < NV; ++v)
      sRec[buf][slot * NV + v] = make_float4(pr[4 * v], pr[4 * v + 1], pr[4 * v + 2], pr[4 * v + 3]);
  };
  auto stage = [&](int buf, bool ok, int64_t jt_stage) {
    if (tid >= TJ) return;
    // the largest |b| this work-group sees, for its range checks (once per j; padded
    // j hold b = 0)
    if (OP != OP_LSE) {
#pragma unroll
      for (int e = 0; e < E; ++e) bmx = fmaxf(bmx, fabsf(rb[e]));
    }
    if (SPLIT) {
      // record (2y', c_j + log2 |b|) at the j's place in its wave's segment: b > 0
      // first, then the rest (b <= 0, NaN, and padded j), in j order within each class
      float rec[4 * NV];
#pragma unroll
      for (int q = 0; q < 4 * NV; ++q) rec[q] = 0.0f;
      float ny = 0.0f;
#pragma unroll
      for (int k = 0; k < D; ++k) {
        const float yp = a.scale * (ry[k] - cen[k]);
        rec[k] = 2.0f * yp;
        ny = fmaf(yp, yp, ny);
      }
      const float bv = OP == OP_MAX ? a.max_sign * rb[0] : rb[0];
      const bool pos = ok && bv > 0.0f;
      // padded j: 0 for the sum; never chosen by Max (its class looks for the least exponent)
      rec[D] = ok ? (-ny - G) + __builtin_amdgcn_logf(fabsf(bv)) : (OP == OP_MAX ? INFINITY : -INFINITY);
      // place = rank within the class over the whole tile: ballot counts per wave,
      // the waves' counts through LDS (one barrier; every thread of the work-group
      // stages, so all reach it)
      const int lane = tid & (kWave - 1), w = tid / kWave;
      const uint64_t mpos = __ballot(pos);
      const int below = __popcll(mpos & ((1ull << lane) - 1ull));
      if (lane == 0) sSeg[buf][w] = __popcll(mpos);
      __syncthreads();
      int P = 0, offp = 0;
#pragma unroll
      for (int v = 0; v < TJ / kWave; ++v) {
        const int c = sSeg[buf][v];
        P += c;
        offp += v < w ? c : 0;
      }
      const int P4 = (P + 3) & ~3, Q = TJ - P, Q4 = (Q + 3) & ~3;
      const int slot = pos ? offp + below : P4 + (w * kWave - offp) + (lane - below);
#pragma unroll
      for (int v = 0; v < NV; ++v)
        sRec[buf][slot * NV + v] = make_float4(rec[4 * v], rec[4 * v + 1], rec[4 * v + 2], rec[4 * v + 3]);
      if (OP == OP_MAX) sIdx[buf][slot] = ok ? (int)(jt_stage + tid) : -1;
      // pads to whole groups of 4: never contribute (sum) and never win (Max)
      if (tid < P4 - P) {
        put_pad(buf, P + tid, -INFINITY);
        if (OP == OP_MAX) sIdx[buf][P + tid] = -1;
      }
      if (tid < Q4 - Q) {
        put_pad(buf, P4 + Q + tid, OP == OP_MAX ? INFINITY : -INFINITY);
        if (OP == OP_MAX) sIdx[buf][P4 + Q + tid] = -1;
      }
      return;
    }
    float rec[4 * NV];
#pragma unroll
    for (int q = 0; q < 4 * NV; ++q) rec[q] = 0.0f;
    if (FAST) {
      float ny = 0.0f;
#pragma unroll
      for (int k = 0; k < D; ++k) {
        const float yp = a.scale * (ry[k] - cen[k]);
        rec[k] = 2.0f * yp;
        ny = fmaf(yp, yp, ny);
      }
      float cj = -ny - G;
      if (OP == OP_LSE && E == 1) cj += kLog2e * rb[0];
      rec[D] = ok ? cj : -INFINITY;
    } else {
#pragma unroll
      for (int k = 0; k < D; ++k) rec[k] = ry[k];
    }
#pragma unroll
    for (int v = 0; v < NV; ++v)
      sRec[buf][tid * NV + v] = make_float4(rec[4 * v], rec[4 * v + 1], rec[4 * v + 2], rec[4 * v + 3]);
    if (OP == OP_SUM) {
#pragma unroll
      for (int e = 0; e < E; ++e) sPay[buf][e * TJ + tid] = ok ? rb[e] : 0.0f;
    } else if (OP == OP_LSE) {
#pragma unroll
      for (int e = 0; e < E; ++e) sPay[buf][e * TJ + tid] = ok ? kLog2e * rb[e] : -INFINITY;
    } else if (OP == OP_MAX) {
      // signed payload; padded j carry -inf, so K * b is -inf or NaN and never wins
#pragma unroll
      for (int e = 0; e < E; ++e) sPay[buf][e * TJ + tid] = ok ? a.max_sign * rb[e] : -INFINITY;
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) sPay[buf][e * TJ + tid] = ok ? rb[e] : 0.0f;
    }
  };

  if (jb < je) {
    const bool ok = load_raw(jb);
    stage(0, ok, jb);
  }
  __syncthreads();
  int buf = 0;
  for (int64_t jt = jb; jt < je; jt += TJ) {
    const bool has_next = jt + TJ < je;
    bool ok_next = false;
    if (has_next) ok_next = load_raw(jt + TJ);
    const int cnt = (int)(((je - jt < TJ ? je - jt : TJ) + 3) & ~3);
    const float4 *rec = sRec[buf];
    const float *pay = sPay[buf];

    float part[R][NP];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int q = 0; q < NP; ++q) part[r][q] = 0.0f;

    if (SPLIT) {
      // the b > 0 class, then the rest; bounds are uniform
      const int *idx = sIdx[buf];
      int P = 0;
#pragma unroll
      for (int v = 0; v < TJ / kWave; ++v) P += sSeg[buf][v];
      P = __builtin_amdgcn_readfirstlane(P);
      const int p4 = (P + 3) & ~3, q4 = (TJ - P + 3) & ~3;
      if (OP == OP_SUM) {
        pipelined_records<NV>(rec, 0, p4, xs, s2, [&](const float (&q)[R]) {
#pragma unroll
          for (int r = 0; r < R; ++r) part[r][0] += fast_exp2(q[r]);
        });
        pipelined_records<NV>(rec, p4, p4 + q4, xs, s2, [&](const float (&q)[R]) {
#pragma unroll
          for (int r = 0; r < R; ++r) part[r][0] -= fast_exp2(q[r]);
        });
      } else {
        // grad and Max: the records are still needed after the exp2 (grad), or
        // the loop also reads the record's j from LDS (Max), so the records
        // are read group by group
        for (int jj = 0; jj < p4; jj += 4) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            float yv[4 * NV];
            load_rec<NV>(rec, jj + u, yv);
            float q[R], dd[1][D];
            pair_exponent<true>(xs, yv, s2, off, q, dd);
            if (OP == OP_GRAD) {
              // K b (x' - y'): the weight already holds |b|
#pragma unroll
              for (int r = 0; r < R; ++r) {
                const float wgt = fast_exp2(q[r]);
#pragma unroll
                for (int k = 0; k < D; ++k) part[r][k] = fmaf(wgt, fmaf(yv[k], -0.5f, xs[r][k]), part[r][k]);
              }
            } else {
              // largest exponent of a positive product; strict: ties keep the smaller j
              const int j = idx[jj + u];
#pragma unroll
              for (int r = 0; r < R; ++r) {
                const bool up = q[r] > acc[r][0];
                acc[r][0] = up ? q[r] : acc[r][0];
                ix[r][0] = up ? j : ix[r][0];
              }
            }
          }
        }
        for (int jj = p4; jj < p4 + q4; jj += 4) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            float yv[4 * NV];
            load_rec<NV>(rec, jj + u, yv);
            float q[R], dd[1][D];
            pair_exponent<true>(xs, yv, s2, off, q, dd);
            if (OP == OP_GRAD) {
#pragma unroll
              for (int r = 0; r < R; ++r) {
                const float wgt = fast_exp2(q[r]);
#pragma unroll
                for (int k = 0; k < D; ++k) part[r][k] = fmaf(-wgt, fmaf(yv[k], -0.5f, xs[r][k]), part[r][k]);
              }
            } else {
              // least exponent of a non-positive product (b = 0 gives -inf: the value 0)
              const int j = idx[jj + u];
#pragma unroll
              for (int r = 0; r < R; ++r) {
                const bool up = q[r] < acc[r][1];
                acc[r][1] = up ? q[r] : acc[r][1];
                ix[r][1] = up ? j : ix[r][1];
              }
            }
          }
        }
      }
    } else if (OP == OP_LSE && FIXED && E == 1 && D <= 64) {
      // the payload is folded into the records' constant: exp2 and accumulate (records
      // read one group ahead; at D = 100 the four records in flight spilled 476
      // registers, and the loop below reads them group by group)
      pipelined_records<NV>(rec, 0, cnt, xs, s2, [&](const float (&q)[R]) {
#pragma unroll
        for (int r = 0; r < R; ++r) part[r][0] += fast_exp2(q[r]);
      });
    } else if (OP == OP_LAPLACE && E == 1 && D <= 32) {
      // direct form with the records of the next group read ahead, as in
      // pipelined_records.  This group's b is read first, at the top, so that
      // waiting for it does not wait for the records in flight.
      float yv[4][4 * NV];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        load_rec<NV>(rec, u, yv[u]);
#pragma unroll
        for (int k = 0; k < 4 * NV; ++k) asm volatile("" : "+v"(yv[u][k]));   // see pipelined_records
      }
      for (int jj = 0; jj < cnt; jj += 4) {
        const float4 pb = *reinterpret_cast<const float4 *>(pay + jj);
        __builtin_amdgcn_sched_barrier(0);   // the b read stays ahead of the exponents
        float q[4][R], dd[R][D];
#pragma unroll
        for (int u = 0; u < 4; ++u) pair_exponent<false, R, D, 4 * NV, true>(xs, yv[u], s2, off, q[u], dd);
        const int jn = jj + 4 < cnt ? jj + 4 : jj;
#pragma unroll
        for (int u = 0; u < 4; ++u) load_rec<NV>(rec, jn + u, yv[u]);
        __builtin_amdgcn_sched_barrier(0);   // and the record reads ahead of the exp2s
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int r = 0; r < R; ++r) part[r][0] = fmaf(fast_exp2(q[u][r]), lane4(pb, u), part[r][0]);
      }
    } else
    for (int jj = 0; jj < cnt; jj += 4) {
      float4 pq[PAY];
#pragma unroll
      for (int p = 0; p < PAY; ++p) pq[p] = *reinterpret_cast<const float4 *>(pay + p * TJ + jj);

      if (OP == OP_LSE && FIXED) {
        // exponents are at most G + max_j b_j log2 e (< 128 with the sum below
        // 2^128): exp2 and accumulate, no maximum to track
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          float yv[4 * NV];
          load_rec<NV>(rec, jj + u, yv);
          float q[R], dd[1][D];
          pair_exponent<true>(xs, yv, s2, off, q, dd);
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int e = 0; e < E; ++e)
              part[r][e] += fast_exp2(E == 1 ? q[r] : q[r] + lane4(pq[e], u));
        }
      } else if (OP == OP_LSE) {
        // online LogSumExp in log2 units: four exponents per row, raise the
        // running max when one exceeds it (rescaling the sums), accumulate.
        float uu[4][R][E];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          float yv[4 * NV];
          load_rec<NV>(rec, jj + u, yv);
          float q[R], dd[FAST ? 1 : R][D];
          pair_exponent<FAST>(xs, yv, s2, off, q, dd);
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int e = 0; e < E; ++e) uu[u][r][e] = (FAST && E == 1) ? q[r] : q[r] + lane4(pq[e], u);
        }
        bool up = false;
        float mn[R][E];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int e = 0; e < E; ++e) {
            mn[r][e] = fmaxf(fmaxf(acc[r][2 * e], uu[0][r][e]), uu[1][r][e]);
            mn[r][e] = fmaxf(fmaxf(mn[r][e], uu[2][r][e]), uu[3][r][e]);
            up |= mn[r][e] > acc[r][2 * e];
          }
        if (up) {
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int e = 0; e < E; ++e) {
              const float f = fast_exp2(acc[r][2 * e] - mn[r][e]);
              acc[r][2 * e + 1] *= f;
              part[r][e] *= f;
              acc[r][2 * e] = mn[r][e];
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          float ex[R][E];
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int e = 0; e < E; ++e) ex[r][e] = uu[u][r][e] - acc[r][2 * e];
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int e = 0; e < E; ++e) ex[r][e] = fast_exp2(ex[r][e]);
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int e = 0; e < E; ++e) part[r][e] += ex[r][e];
        }
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          float yv[4 * NV];
          load_rec<NV>(rec, jj + u, yv);
          float ex[R], dd[FAST ? 1 : R][D];
          pair_exponent<FAST, R, D, 4 * NV, OP == OP_LAPLACE>(xs, yv, s2, off, ex, dd);
#pragma unroll
          for (int r = 0; r < R; ++r) ex[r] = fast_exp2(ex[r]);
#pragma unroll
          for (int r = 0; r < R; ++r) {
            if (OP == OP_SUM || OP == OP_LAPLACE) {
#pragma unroll
              for (int e = 0; e < E; ++e) part[r][e] = fmaf(ex[r], lane4(pq[e], u), part[r][e]);
            } else if (OP == OP_MAX) {
              // strict >: j increases along the lane's loop, so ties keep the smaller j
              const int j = (int)(jt + jj + u);
#pragma unroll
              for (int e = 0; e < E; ++e) {
                const float v = ex[r] * lane4(pq[e], u);
                const bool up = v > acc[r][e];
                acc[r][e] = up ? v : acc[r][e];
                ix[r][e] = up ? j : ix[r][e];
              }
            } else {
              // grad: A_k += K <g_i, b_j> (x_k - y_k), the difference taken per pair
              // (never as x * sum - sum * y, which cancels for near neighbours)
              float gb;
              if (E == 1) {
                gb = lane4(pq[0], u);
              } else {
                gb = 0.0f;
#pragma unroll
                for (int e = 0; e < E; ++e) gb = fmaf(gr[r][e], lane4(pq[e], u), gb);
              }
              const float w = ex[r] * gb;
#pragma unroll
              for (int k = 0; k < D; ++k) {
                // expanded form: x'_k - y'_k = x'_k - (2y'_k)/2, one rounding
                const float dk = FAST ? fmaf(yv[k], -0.5f, xs[r][k]) : dd[FAST ? 0 : r][k];
                part[r][k] = fmaf(w, dk, part[r][k]);
              }
            }
          }
        }
      }
    }
    // fold the tile's partial sums into the row accumulators
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (OP == OP_LSE) {
#pragma unroll
        for (int e = 0; e < E; ++e) acc[r][2 * e + 1] += part[r][e];
      } else if (OP == OP_MAX) {
        // the maximum is kept in acc directly
      } else {
#pragma unroll
        for (int q = 0; q < NP; ++q) acc[r][q] += part[r][q];
      }
    }
    if (has_next) stage(buf ^ 1, ok_next, jt + TJ);
    __syncthreads();
    buf ^= 1;
  }
}

// Forms a work-group's j loop can take (uniform across the work-group).
enum JMode : int {
  JM_DIRECT = 0,   // raw differences, exponent offset `off`
  JM_FAST = 1,     // expanded form, shift G = r2/2
  JM_FIXED = 2,    // LogSumExp, expanded form, fixed per-row shift G - |x'|^2
  JM_RUN = 3,      // LogSumExp, expanded form, running maximum (G = 0)
};

template <int OP, int D, int E, int R>
__global__ __launch_bounds__(kThreads) void gauss_valu_kernel(GaussArgs a) {
  using S = GaussShape<OP, D, E>;
  constexpr int NV = S::NV, PAY = S::PAY, TJ = S::TJ;
  __shared__ float4 sRec[2][S::TJR * NV];
  __shared__ __attribute__((aligned(16))) float sPay[2][PAY * TJ];
  __shared__ float sRed[2 * D * (kThreads / kWave) + 8];
  __shared__ int sIdx[S::SPLIT && OP == OP_MAX ? 2 : 1][S::SPLIT && OP == OP_MAX ? S::TJR : 1];   // j of each record
  __shared__ int sSeg[2][4];                                                                     // class sizes per wave

  // work-groups whose results the MFMA kernel has stored (uniform across the work-group)
  if (a.wg_flags && a.wg_flags[(int64_t)blockIdx.x * gridDim.y + blockIdx.y]) return;

  const int tid = threadIdx.x;
  const int wid = tid / kWave, lane = tid & (kWave - 1);
  const BsItem *item = a.items ? a.items + blockIdx.x : nullptr;
  const int64_t row0 = item ? item->row_lo : (int64_t)blockIdx.x * (kThreads * R);
  const int64_t row_end = item ? item->row_hi : a.M;
  const int64_t M = a.M;
  // the j of this work-group: one split of a dense launch, or the item's ranges
  const int64_t jb0 = (int64_t)blockIdx.y * a.j_per_split;
  const int64_t je0 = (jb0 + a.j_per_split < a.N) ? jb0 + a.j_per_split : a.N;
  int64_t nj = 0;
  if (!item) {
    nj = je0 - jb0;
  } else {
    for (int64_t k = item->k0; k <= item->k1; ++k) {
      const int64_t jb = k == item->k0 ? item->j0 : a.redr[2 * k];
      const int64_t je = k == item->k1 ? item->j1 : a.redr[2 * k + 1];
      nj += je > jb ? je - jb : 0;
    }
  }
  const float log2n = nj > 1 ? ceilf(log2f((float)nj)) : 0.0f;

  // ---- rows (raw), bounding-box centre of the work-group
  float xs[R][D];
  bool valid[R];
  auto load_rows = [&]() {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t i = row0 + (int64_t)r * kThreads + tid;
      valid[r] = i < row_end;
#pragma unroll
      for (int k = 0; k < D; ++k) xs[r][k] = valid[r] ? a.x[i * D + k] : 0.0f;
    }
  };
  load_rows();
  float cen[D];
  {
    float lo[D], hi[D];
#pragma unroll
    for (int k = 0; k < D; ++k) {
      lo[k] = INFINITY;
      hi[k] = -INFINITY;
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (valid[r]) { lo[k] = fminf(lo[k], xs[r][k]); hi[k] = fmaxf(hi[k], xs[r][k]); }
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
      cen[k] = 0.5f * l + 0.5f * h;
    }
  }
  // ---- |x'|^2 of every row and the work-group radius that selects the form
  float nx[R];
  float r2 = 0.0f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float n = 0.0f;
#pragma unroll
    for (int k = 0; k < D; ++k) {
      const float t = a.scale * (xs[r][k] - cen[k]);
      n = fmaf(t, t, n);
    }
    nx[r] = n;
    if (valid[r]) r2 = fmaxf(r2, n);
  }
  float *red = sRed + 2 * D * (kThreads / kWave);
  r2 = block_max(r2, red);
  // the Laplacian kernel needs |x - y| itself, which the expanded form cannot give
  // accurately for close pairs: always the direct form
  const bool fast = OP != OP_LAPLACE && a.form == FORM_AUTO && r2 <= kFastR2;
  if (fast) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int k = 0; k < D; ++k) xs[r][k] = a.scale * (xs[r][k] - cen[k]);
  }

  float gr[R][E];
  float gmax = 0.0f;   // grad_x: the largest sum_e |g_e| of the work-group's rows
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t i = row0 + (int64_t)r * kThreads + tid;
    float gs = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      gr[r][e] = (OP == OP_GRAD && valid[r]) ? a.g[i * E + e] : 0.0f;
      gs += fabsf(gr[r][e]);
    }
    gmax = fmaxf(gmax, gs);
  }
  if (OP == OP_GRAD) gmax = block_max(gmax, red);

  // the sign-split tile's index array only exists for Max (a 1 x 1 stand-in otherwise)
  int (*sIdxP)[S::TJR] = reinterpret_cast<int (*)[S::TJR]>(&sIdx[0][0]);
  constexpr int W = (OP == OP_SUM || OP == OP_LAPLACE) ? E : ((OP == OP_LSE || OP == OP_MAX) ? (2 * E) : D);
  float acc[R][S::NACC];
  int ix[R][2 * E];
  auto reset = [&]() {
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int q = 0; q < S::NACC; ++q) acc[r][q] = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        ix[r][e] = -1;
        ix[r][E + e] = -1;
        if (OP == OP_LSE) acc[r][2 * e] = -3.0e38f;   // running max (finite: keeps u - m defined)
        if (OP == OP_MAX) {
          acc[r][e] = -INFINITY;      // best value (sign-split tile: best exponent of a positive product)
          acc[r][E + e] = INFINITY;   // sign-split tile: least exponent of a non-positive product
        }
      }
    }
  };
  // The work-group's j loop in one form (FAST: expanded distance; FIXED: LogSumExp
  // with a fixed per-row shift): one split of a dense launch, or the item's ranges.
  auto jloop = [&](auto fast_c, auto fixed_c, float G, const float (&offv)[R], float &bmx) {
    constexpr bool F = decltype(fast_c)::value, X = decltype(fixed_c)::value;
    if (!item) {
      gauss_jloop<OP, D, E, R, F, X>(a, sRec, sPay, sIdxP, sSeg, xs, gr, cen, G, offv, acc, ix, bmx, jb0, je0);
    } else {
      for (int64_t k = item->k0; k <= item->k1; ++k) {
        const int64_t jb = k == item->k0 ? item->j0 : a.redr[2 * k];
        const int64_t je = k == item->k1 ? item->j1 : a.redr[2 * k + 1];
        if (jb < je) gauss_jloop<OP, D, E, R, F, X>(a, sRec, sPay, sIdxP, sSeg, xs, gr, cen, G, offv, acc, ix, bmx, jb, je);
      }
    }
    // sign-split Max: back from exponents to the value in the shifted scale -- the best
    // positive product if there is one, else the least negative (or zero) one
    if constexpr (OP == OP_MAX && S::SPLIT && F) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const bool haspos = acc[r][0] > -INFINITY;
        const bool hasneg = acc[r][1] < INFINITY;
        acc[r][0] = haspos ? fast_exp2(acc[r][0]) : (hasneg ? -fast_exp2(acc[r][1]) : -INFINITY);
        ix[r][0] = haspos ? ix[r][0] : (hasneg ? ix[r][1] : -1);
      }
    }
  };
  using T = std::integral_constant<bool, true>;
  using Fa = std::integral_constant<bool, false>;

  // The values row r stores after a pass in `mode` (G the shift of the expanded form,
  // off the row's direct-form offset): sums and gradients scaled back, LogSumExp's
  // (max, sum) pairs in log2 units, Max's (signed value, index bits) pairs.
  auto finals = [&](int r, int md, float G, float off, float (&res)[W]) {
    const bool fx = md != JM_DIRECT;
    // row factor f1, then f2 = 2^-off for the direct form's offset
    float f1 = 1.0f;
    const float f2 = fx ? 1.0f : exp2f(-off);
    if (OP == OP_SUM || OP == OP_LAPLACE || OP == OP_MAX) {
      f1 = fx ? exp2f(G - nx[r]) : 1.0f;
    } else if (OP == OP_GRAD) {
      // expanded: G_k = -(2/sigma^2) (1/s) exp2(G - |x'|^2) sum_j K' <g, b> (x'_k - y'_k)
      // direct:   G_k = -(2/sigma^2) sum_j K <g, b> (x_k - y_k)
      f1 = (fx ? exp2f(G - nx[r]) * a.grad_coef : a.grad_coef_direct) * (E == 1 ? gr[r][0] : 1.0f);
    }
    if (OP == OP_MAX) {
      // the row factor is positive, so the argmax is that of acc
#pragma unroll
      for (int e = 0; e < E; ++e) { res[2 * e] = (acc[r][e] * f1) * f2; res[2 * e + 1] = __int_as_float(ix[r][e]); }
    } else if (OP == OP_LSE) {
      // the fixed form's shift is G - |x'|^2; the running maximum is relative to |x'|^2
      const float offl = fx ? nx[r] : 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        res[2 * e] = md == JM_FIXED ? G - nx[r] : acc[r][2 * e] - offl;
        res[2 * e + 1] = acc[r][2 * e + 1];
      }
    } else {
#pragma unroll
      for (int w = 0; w < W; ++w) res[w] = (acc[r][w] * f1) * f2;
    }
  };
  const bool partial = a.nsplit > 1;
  auto put = [&](int r, const float (&res)[W]) {
    const int64_t i = row0 + (int64_t)r * kThreads + tid;
    if (partial) {
      const int64_t slot = item ? item->slot : blockIdx.y;
      float *dst = a.out + (slot * M + i) * W;
#pragma unroll
      for (int w = 0; w < W; ++w) dst[w] = res[w];
    } else if (OP == OP_LSE) {
#pragma unroll
      for (int e = 0; e < E; ++e) a.out[i * E + e] = kLn2 * (res[2 * e] + log2f(res[2 * e + 1]));
    } else if (OP == OP_MAX) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        a.out[i * E + e] = a.max_sign * res[2 * e];
        a.out_idx[i * E + e] = (int64_t)__float_as_int(res[2 * e + 1]);
      }
    } else {
#pragma unroll
      for (int w = 0; w < W; ++w) a.out[i * W + w] = res[w];
    }
  };

  // ---- first pass: the expanded form where its precision condition holds (LogSumExp
  // with a fixed per-row shift; shift G = r2/2: the largest exponent is r2 - G, the
  // smallest row factor exponent -G), else the direct form with offset 2^64
  const int mode = fast ? (OP == OP_LSE ? JM_FIXED : JM_FAST) : JM_DIRECT;
  const float G = fast ? 0.5f * r2 : 0.0f;
  float offr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) offr[r] = OP == OP_LSE ? 0.0f : kDirectOffset;
  float bmx = 0.0f;   // the largest |b| of the work-group's j (staging tracks it)
  reset();
  if (mode == JM_FIXED) jloop(T(), T(), G, offr, bmx);
  else if (mode == JM_FAST) jloop(T(), Fa(), G, offr, bmx);
  else jloop(Fa(), Fa(), 0.0f, offr, bmx);

  // ---- range checks (see GaussArgs).  Every row stores its first-pass values now; rows
  // that fail a check are computed once more (second pass) and overwrite them:
  //   over[r]: non-finite from finite inputs -> direct form, offset off_safe;
  //   low[r]:  below the expanded form's floor  -> direct form with the row's own offset:
  //            its terms are below the threshold in the shifted scale, i.e. below
  //            thr 2^(G - |x'|^2) in the true one, so 2^off times them stays below
  //            2^kOffsetRoom for off up to kOffsetRoom - log2(thr) - G + |x'|^2 (at least
  //            64, at most 127 so that exp2(off - s^2 d^2) itself is finite).  Kept only
  //            if finite: a row that is low by cancellation of large terms keeps the
  //            first pass.  LogSumExp: fixed-shift sum low or not finite -> running max.
  if (OP != OP_LSE) bmx = block_max(bmx, red);
  bool over[R], low[R];
  bool any = false;
  float off_safe = kDirectOffset;
  {
    const bool fx = mode != JM_DIRECT;
    const bool inputs_finite = isfinite(bmx) && isfinite(gmax);
    // direct-form offset that keeps this work-group's accumulators below 2^kOffsetRoom
    float lim = log2f(fmaxf(bmx, 1e-30f)) + (OP == OP_MAX ? 0.0f : log2n);
    if (OP == OP_GRAD) {
      // |x - y| K <= 0.43 sigma and the factor 2/sigma^2: both ends of sigma bounded
      const float ls = 0.5f * log2f(2.0f / fabsf(a.grad_coef_direct));   // log2 sigma
      lim += log2f(fmaxf(gmax, 1.0f)) + fabsf(ls) + 1.0f;
    }
    off_safe = fminf(kDirectOffset, floorf(kOffsetRoom - lim));
    // the underflow threshold of the expanded form (sign-split tile: log2 |b| is in the
    // exponent, so a flushed term is under 2^-126 itself; max(1, max|b|) covers both)
    const float bmg = (OP == OP_SUM || OP == OP_MAX || (OP == OP_GRAD && E == 1)) ? fmaxf(bmx, 1.0f) : bmx;
    float thr = OP == OP_MAX ? exp2f(-kGuardLoss) * bmg : exp2f(log2n - kGuardLoss) * bmg;
    if (OP == OP_GRAD) thr *= 32.0f * (E == 1 ? 1.0f : gmax);
    const float lse_thr = exp2f(log2n - kGuardLoss - 1.0f);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      over[r] = false;
      low[r] = false;
      if (!valid[r]) continue;
      float res[W];
      finals(r, mode, G, offr[r], res);
      put(r, res);
      if (!inputs_finite) continue;
      if (OP == OP_LSE) {
        if (mode == JM_FIXED) {
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const float sm = acc[r][2 * e + 1];
            low[r] |= !(sm >= lse_thr) || !(sm < INFINITY);
          }
        }
      } else {
        constexpr int WA = OP == OP_MAX ? E : W;
#pragma unroll
        for (int w = 0; w < WA; ++w) {
          const float v = res[OP == OP_MAX ? 2 * w : w];
          over[r] |= !(fabsf(v) < INFINITY);
          if (fx) low[r] |= !(fabsf(acc[r][w]) >= thr);
        }
        if (!fx) over[r] &= off_safe < kDirectOffset;   // a smaller offset would not help
        // grad_x: the direct form's differences are raw, x - y = (x' - y') / s
        const float lg = OP == OP_GRAD ? fmaxf(0.0f, -log2f(a.scale)) : 0.0f;
        const float off_low = fminf(127.0f, fmaxf(kDirectOffset, floorf(kOffsetRoom - log2f(thr) - G + nx[r] - lg)));
        offr[r] = over[r] ? off_safe : (low[r] ? off_low : kDirectOffset);
      }
      any |= over[r] || low[r];
    }
  }
  if (!__syncthreads_or(any)) return;

  // ---- second pass over the same j
  reset();
  if (OP == OP_LSE) {
    jloop(T(), Fa(), 0.0f, offr, bmx);   // running maximum, expanded form (G = 0)
  } else {
    load_rows();                         // raw coordinates for the direct form
    jloop(Fa(), Fa(), 0.0f, offr, bmx);
  }
  const int mode2 = OP == OP_LSE ? JM_RUN : JM_DIRECT;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (!valid[r] || !(over[r] || low[r])) continue;
    float res[W];
    finals(r, mode2, 0.0f, offr[r], res);
    bool fin = true;
    if (OP != OP_LSE) {
#pragma unroll
      for (int w = 0; w < W; ++w) fin &= fabsf(res[w]) < INFINITY || (OP == OP_MAX && (w & 1));
    }
    if (over[r] || fin) put(r, res);
  }
}

// Rows per lane of the "wide" variant (large M); the narrow variant holds 1.
__host__ __device__ constexpr int gauss_rows_wide(int op, int D, int E) {
  // At D <= 4 (1M x 1M, D = 3): the sum and grad_x take 2 rows per lane, the other
  // ops 4.  Sum: 129.3 ms with 2, 132.0 with 4, 134 with 3; the extra waves per SIMD
  // that fewer VGPRs allow hide more than the doubled LDS record reads cost.
  // grad_x: 111 VGPRs (four waves) against 149 (three) with 4, 3.4 % faster (3 rows:
  // 120 VGPRs, no faster than 4).  LSE ran alike with 2 and 4, Max 11 % slower with
  // 2.  Before the sign-split tile the sum ran alike with 8 and 4.
  // grad_x at D = 16 keeps one row per lane: with two its E = 3, 4 variants reached
  // 256 VGPRs and spilled
  return D <= 4 ? ((op == OP_GRAD || op == OP_SUM) ? 2 : 4)
                : (D <= 8 ? (E <= 2 ? 4 : 2) : (D <= 16 ? (op == OP_GRAD ? 1 : 2) : 1));
}

template <int OP, int D, int E, int R>
void launch_gauss_t(dim3 grid, const GaussArgs &a, hipStream_t st) {
  hipLaunchKernelGGL((gauss_valu_kernel<OP, D, E, R>), grid, dim3(kThreads), 0, st, a);
}

}  // namespace kmi
