// common.h -- internal definitions shared by the gfx950 kernels and the host
// launcher of the Gaussian map-reduce engine (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kmi {

constexpr int kThreads = 256;           // work-group: four wave64
constexpr int kWave = 64;
constexpr int kTileJ = 256;             // j rows staged in LDS per tile (one per thread)
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
// Largest |x'_i|^2 (scaled, centred, log2 units) for which the expanded form
// exp2(2<x',y'> - |y'|^2 - G) keeps both range and precision: at R^2 <= 128
// the fp32 rounding of the expansion stays near 1e-5 relative in K_ij, and the
// shifted exponent stays inside the fp32 range; beyond it a work-group takes
// the direct form from raw differences.
constexpr float kFastR2 = 128.0f;
// Exponent offset (log2 units) of the direct form's sums and gradients.
constexpr float kDirectOffset = 64.0f;

enum Op : int { OP_SUM = 0, OP_LSE = 1, OP_GRAD = 2, OP_MAX = 3, OP_LAPLACE = 4 };
enum Form : int { FORM_AUTO = 0, FORM_DIRECT = 1 };

// One work-group's share of a block-sparse launch: rows [row_lo, row_hi)
// (inside one row range, at most the kernel's rows per work-group) against
// the j ranges k0..k1 of that row range, the first starting at j0 and the
// last ending before j1; its partial sums go to split slot `slot`.
struct BsItem {
  int64_t row_lo, row_hi;
  int64_t k0, j0;
  int64_t k1, j1;
  int32_t slot;
  int32_t pad;
};

// Arguments of the sum / LSE / grad_x pass-1 kernels.
struct GaussArgs {
  const float *x, *y, *b, *g;
  int64_t M, N;
  float scale;          // sqrt(log2 e) / sigma: exp(-d^2/sigma^2) = exp2(-|scale*(x-y)|^2);
                        // OP_LAPLACE: sqrt(log2 e / sigma), so scale^2 |x - y| is the log2 exponent
  float grad_coef;      // -(2 / sigma^2) / scale  (expanded form: scaled coordinates)
  float grad_coef_direct;  // -(2 / sigma^2)        (direct form: raw coordinates)
  float *out;           // final output when nsplit == 1, else partials [nsplit][M][W]
  int64_t *out_idx;     // OP_MAX: [M][E] indices when nsplit == 1
  float max_sign;       // OP_MAX: +1 (Max / ArgMax of K b) or -1 (Min / ArgMin)
  int64_t j_per_split;  // multiple of kTileJ
  int nsplit;
  int form;             // Form
  // Per work-group decisions of the MFMA kernels, [row block][j split] (1 = results
  // stored there); when set, the VALU kernel skips those work-groups.  Null otherwise.
  int *wg_flags;
  // Block-sparse launches: work item blockIdx.x and the [nrj][2] j ranges.
  // Null for dense launches (rows from blockIdx.x, j from blockIdx.y).
  const BsItem *items;
  const int64_t *redr;
};

// Range checks of one work-group's result, made by the work-group itself once its
// j range is done (no pre-pass, no second launch):
//  * underflow: the expanded form shifts each exponent by G, so a term below
//    2^-126 in the shifted scale is flushed by v_exp_f32.  With nj terms of at
//    most max|b| each, a shifted row result at or above nj max|b| 2^-109
//    (grad_x: times 32 sum_e |g_e|; Max: max|b| 2^-109) has lost at most 2^-17 of
//    itself; a row below it sends the work-group to the direct form.  LogSumExp
//    with a fixed per-row shift: a row sum below nj 2^-110 goes back to the
//    running maximum.
//  * overflow: a non-finite result from finite inputs (the shifts scale the
//    accumulators by up to 2^64) sends the work-group to the direct form with an
//    exponent offset small enough for the sums it saw: 2^off nj max|b| (grad_x:
//    times its coefficient bound) stays below 2^120.
// Each work-group redoes its own rows at most once.
constexpr float kGuardLoss = 109.0f;     // underflow threshold per term: 2^-109, 2^17 above the flush level
constexpr float kOffsetRoom = 120.0f;    // log2 bound of a direct-form accumulator

// Arguments of the few-rows sum kernel (j per lane, rows in LDS).
struct StreamArgs {
  const float *x, *y, *b;
  int64_t M, N;
  float scale;          // sqrt(log2 e) / sigma
  int64_t j_per_wg;     // multiple of the kernel's step (kThreads * j per lane)
  float *part;          // [gridDim.x][M][E] partial sums
  int form;             // Form
  // Underflow guard: each row's factor exp2(G - |x'|^2) applied to its partials
  // (expanded form), or -1 (direct form), written by the work-groups of j chunk 0;
  // and the maximum of |b| over each j chunk (written by row group 0).  Null when off.
  float *row_fac;
  float *chunk_bmax;
  // gradient with respect to x: the cotangent [M][E] and -(2 / sigma^2)
  const float *g;
  float coef;
};

// Arguments of the K-min pass-1 kernel.
struct KminArgs {
  const float *x, *y;
  int64_t M, N;
  float *out_d;         // [M][K] when nsplit == 1, else partial distances [nsplit][M][K]
  int64_t *out_idx;     // [M][K] when nsplit == 1
  int32_t *part_idx;    // partial indices [nsplit][M][K] when nsplit > 1
  int64_t j_per_split;
  int nsplit;
};

// ---------------------------------------------------------------- wave / block reductions
// Cross-lane steps use DPP inside 16-lane rows and a swizzle/bpermute across rows.
__device__ __forceinline__ float dpp_quad_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_quad_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_row_half_mirror(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_row_mirror(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
}

// Every lane of each 16-lane row receives the row's sum.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_quad_xor1(v);
  v += dpp_quad_xor2(v);
  v += dpp_row_half_mirror(v);
  v += dpp_row_mirror(v);
  return v;
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_quad_xor1(v));
  v = fmaxf(v, dpp_quad_xor2(v));
  v = fmaxf(v, dpp_row_half_mirror(v));
  v = fmaxf(v, dpp_row_mirror(v));
  return v;
}
__device__ __forceinline__ float row16_min(float v) {
  v = fminf(v, dpp_quad_xor1(v));
  v = fminf(v, dpp_quad_xor2(v));
  v = fminf(v, dpp_row_half_mirror(v));
  v = fminf(v, dpp_row_mirror(v));
  return v;
}
// Whole-wave reductions: rows of 16 by DPP, then the four row results by xor-shuffles.
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float wave_min(float v) {
  v = row16_min(v);
  v = fminf(v, __shfl_xor(v, 16));
  v = fminf(v, __shfl_xor(v, 32));
  return v;
}

// Work-group max / min of one value per thread; `red` holds kThreads/kWave floats.
// Contains barriers: every thread of the work-group must call it.
__device__ __forceinline__ float block_max(float v, float *red) {
  v = wave_max(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int k = 1; k < kThreads / kWave; ++k) r = fmaxf(r, red[k]);
  return r;
}
__device__ __forceinline__ float block_min(float v, float *red) {
  v = wave_min(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int k = 1; k < kThreads / kWave; ++k) r = fminf(r, red[k]);
  return r;
}

__device__ __forceinline__ float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }

// Component u (0..3) of a float4, u known at compile time after unrolling.
__device__ __forceinline__ float lane4(const float4 &v, int u) {
  return u == 0 ? v.x : (u == 1 ? v.y : (u == 2 ? v.z : v.w));
}

// A value the caller knows to be the same in every lane, moved to scalar registers so
// that the compiler can keep loop control on it off the VALU.
__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
  const uint64_t u = (uint64_t)v;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

}  // namespace kmi
