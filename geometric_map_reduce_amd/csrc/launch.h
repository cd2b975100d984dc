// launch.h -- host-side entry points of the kernel translation units.
#pragma once

#include "common.h"

namespace kmi {

// Shape facts of a compiled variant, filled when `info` is non-null.
struct VariantInfo {
  int rows_per_wg;  // output rows per work-group
  int tile_j;       // j rows per LDS tile (the j-split granularity)
};

// Each dispatcher returns 0 when it owns (D, E[, K]) -- launching the kernel,
// or only describing it when `info` is non-null -- and -2 otherwise.
#define KMI_DECLARE_GAUSS(NAME) \
  int NAME(int D, int E, int wide, VariantInfo *info, dim3 grid, const GaussArgs *args, hipStream_t st);
KMI_DECLARE_GAUSS(gauss_dispatch_sum_small)
KMI_DECLARE_GAUSS(gauss_dispatch_sum_large)
KMI_DECLARE_GAUSS(gauss_dispatch_lse_small)
KMI_DECLARE_GAUSS(gauss_dispatch_lse_large)
KMI_DECLARE_GAUSS(gauss_dispatch_grad_small)
KMI_DECLARE_GAUSS(gauss_dispatch_grad_large)
KMI_DECLARE_GAUSS(gauss_dispatch_max_small)
KMI_DECLARE_GAUSS(gauss_dispatch_max_large)
KMI_DECLARE_GAUSS(laplace_dispatch_sum_small)
KMI_DECLARE_GAUSS(laplace_dispatch_sum_large)
KMI_DECLARE_GAUSS(gauss_dispatch_sum_mfma)
KMI_DECLARE_GAUSS(gauss_dispatch_lse_mfma)
KMI_DECLARE_GAUSS(gauss_dispatch_grad_mfma)
#undef KMI_DECLARE_GAUSS

// Few-rows sum with row groups of mr = 4 or stream_rows_large(D, E) rows (rows_per_wg =
// mr, tile_j = j per work-group step).
constexpr int stream_rows_large(int D, int E) {
  return D <= 4 ? (E == 1 ? 16 : (E == 2 ? 8 : 4)) : (E == 1 ? 8 : 4);
}
// Rows per row group of the large few-rows gradient variant: its accumulators, MR x D,
// stay at 48 registers (sixteen rows up to D = 3: 102 VGPRs, five waves per SIMD).
constexpr int stream_grad_mr_large(int D) { return D <= 3 ? 16 : (D <= 4 ? 8 : 4); }
int gauss_dispatch_sum_stream(int D, int E, int mr, VariantInfo *info, dim3 grid, const StreamArgs *args,
                              hipStream_t st);

#define KMI_DECLARE_KMIN(NAME) \
  int NAME(int D, int K, VariantInfo *info, dim3 grid, const KminArgs *args, hipStream_t st);
KMI_DECLARE_KMIN(kmin_dispatch_d1_4)
KMI_DECLARE_KMIN(kmin_dispatch_d5_8)
KMI_DECLARE_KMIN(kmin_dispatch_large)
KMI_DECLARE_KMIN(kmin_dispatch_mfma)
KMI_DECLARE_KMIN(kmin_dispatch_mfma_split)
// few rows (lanes own j): rows_per_wg = rows per row group, tile_j = j per step;
// the grid is one-dimensional, row groups x chunks (args->nsplit chunks)
KMI_DECLARE_KMIN(kmin_dispatch_stream)
#undef KMI_DECLARE_KMIN

void launch_sum_combine(const float *ws, int nsplit, int64_t count, float *out, hipStream_t st);
void launch_lse_combine(const float *ws, int nsplit, int64_t M, int E, float *out, hipStream_t st);
// The same with one work-group per output (few outputs, many splits; M * E < 2^32).
void launch_lse_combine_rows(const float *ws, int nsplit, int64_t M, int E, float *out, hipStream_t st);
int launch_kmin_combine(const float *pd, const int32_t *pi, int nsplit, int64_t M, int K, float *out_d,
                        int64_t *out_i, hipStream_t st);
// The same merge for few rows: one work-group per row (the partial lists of all
// splits merged by the work-group's threads together).
int launch_kmin_stream_combine(const float *pd, const int32_t *pi, int nsplit, int64_t M, int K, float *out_d,
                               int64_t *out_i, hipStream_t st);
void launch_fill(float *out, int64_t count, float v, hipStream_t st);
void launch_fill2(float *out, int64_t pairs, float v0, float v1, hipStream_t st);
void launch_fill_i64(int64_t *out, int64_t count, int64_t v, hipStream_t st);
// Max/ArgMax pass 2: partials [nsplit][M][E] of (signed value, index bits); the
// largest value wins, the smaller index on ties; out = sign * value.
void launch_max_combine(const float *ws, int nsplit, int64_t M, int E, float sign, float *out, int64_t *out_idx,
                        hipStream_t st);
// Range checks of the few-rows sum's pass 2: the rows' factors from pass 1 and the
// partial maxima of |b| (row_fac null: no underflow check, the direct form throughout),
// ceil(log2 N), and what a direct recompute of a flagged output needs.
struct StreamGuard {
  const float *row_fac;
  const float *chunk_bmax;   // [nparts] maxima of |b| per j chunk
  int nparts;
  float log2n;
  const float *x, *y, *b;
  int64_t N;
  int D, E;
  float scale;
  const float *g;   // gradient: the cotangent [M][E] and -(2 / sigma^2)
  float coef;
};
void launch_stream_combine(const float *part, int nparts, int64_t count, float *out, const StreamGuard &g,
                           hipStream_t st);
// Few-rows LogSumExp and gradient (gauss_stream_ops.h); `mr` is 4 or the large
// variant's rows (stream_rows_large(D, E) for LogSumExp, stream_grad_mr_large(D) for
// the gradient).
int gauss_dispatch_lse_stream(int D, int E, int mr, VariantInfo *info, dim3 grid, const StreamArgs *args,
                              hipStream_t st);
int gauss_dispatch_grad_stream(int D, int E, int mr, VariantInfo *info, dim3 grid, const StreamArgs *args,
                               hipStream_t st);
// Gradient pass 2: out[i][d] = sum over the nparts partials in double; a non-finite
// total (an overflow of the offset accumulators) is recomputed in double.
void launch_stream_grad_combine(const float *part, int nparts, int64_t M, float *out, const StreamGuard &g,
                                hipStream_t st);

// Conjugate-gradient vector kernels (E <= 4 columns).  Each launcher that
// reduces writes kCgBlocks x E double partials to `part` and their sums to
// `out[E]` (double).
constexpr int kCgBlocks = 512;
void launch_cg_init(const float *b, int64_t N, int E, float *a, float *r, float *p, double *part, double *out,
                    hipStream_t st);
void launch_cg_apply(const float *p, float *q, float lam, int64_t N, int E, double *part, double *out,
                     hipStream_t st);
void launch_cg_step(float *a, float *r, const float *p, const float *q, const double *rr, const double *pq,
                    int64_t N, int E, double *part, double *out, hipStream_t st);
void launch_cg_direction(float *p, const float *r, const double *rr_new, const double *rr_old, int64_t N, int E,
                         hipStream_t st);
void launch_cg_residual(const float *b, const float *q, int64_t N, int E, double *part, double *out,
                        hipStream_t st);

}  // namespace kmi
