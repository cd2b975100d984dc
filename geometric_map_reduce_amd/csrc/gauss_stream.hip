// Instantiations of the few-rows Gaussian sum (D in 1..8, E in 1..4) and its pass 2.
// `mr` is 4 or stream_mr_large(D, E); anything else is not compiled.
#include "gauss_stream.h"
#include "launch.h"

namespace kmi {

int gauss_dispatch_sum_stream(int D, int E, int mr, VariantInfo *info, dim3 grid, const StreamArgs *args,
                              hipStream_t st) {

#define KMI_STREAM_CASE(DD, EE)                                            \
  if (D == DD && E == EE) {                                                \
    if (mr != 4 && mr != stream_mr_large(DD, EE)) return -2;               \
    if (info) {                                                            \
      info->rows_per_wg = mr;                                              \
      info->tile_j = kThreads * stream_j(DD, EE);                          \
      return 0;                                                            \
    }                                                                      \
    if (mr == 4) launch_gauss_stream_t<DD, EE, 4>(grid, *args, st);        \
    else launch_gauss_stream_t<DD, EE, stream_mr_large(DD, EE)>(grid, *args, st); \
    return 0;                                                              \
  }
#define KMI_STREAM_E(DD) KMI_STREAM_CASE(DD, 1) KMI_STREAM_CASE(DD, 2) KMI_STREAM_CASE(DD, 3) KMI_STREAM_CASE(DD, 4)
  KMI_STREAM_E(1) KMI_STREAM_E(2) KMI_STREAM_E(3) KMI_STREAM_E(4)
  KMI_STREAM_E(5) KMI_STREAM_E(6) KMI_STREAM_E(7) KMI_STREAM_E(8)
#undef KMI_STREAM_E
#undef KMI_STREAM_CASE
  return -2;
}

// out[r] = sum over the nparts partials part[p][r], in order of p, in double:
// one work-group per output, each thread a strided share, then a fixed-shape
// tree over the work-group (deterministic for a given nparts).
// Range checks: an expanded-form row (g.row_fac set) whose sum is below
// N max|b| 2^-109 times its factor may have lost its terms to the floor of exp2
// (each flushed term is under 2^-126 max|b| before the factor), and a sum that is
// not finite overflowed in a shifted fp32 accumulator; the work-group then
// recomputes that output in the direct form, exp2(64 - s^2 |x - y|^2) b with the
// 2^-64 applied at the end, accumulated in double.
__device__ double stream_block_sum(double v, double *red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

__device__ double stream_block_max(double v, double *red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] = fmax(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kThreads) void stream_combine_kernel(const float *part, int nparts, int64_t count,
                                                                  float *out, StreamGuard g) {
  __shared__ double red[kThreads];
  const int64_t r = blockIdx.x;
  const int64_t i = r / g.E;
  const int e = (int)(r - i * g.E);
  double v = 0.0;
  for (int p = threadIdx.x; p < nparts; p += kThreads) v += (double)part[(int64_t)p * count + r];
  double total = stream_block_sum(v, red);
  // uniform: every thread holds the same total
  bool redo = !isfinite(total);   // a shifted partial overflowed
  if (!redo && g.row_fac) {
    const float fac = g.row_fac[i];
    if (fac >= 0.0f) {
      float bm = -INFINITY;
      for (int t = threadIdx.x; t < g.nparts; t += kThreads) bm = fmaxf(bm, g.chunk_bmax[t]);
      bm = (float)stream_block_max(bm, red);
      const double thr = exp2((double)g.log2n - (double)kGuardLoss) * (double)bm * (double)fac;
      redo = !(fabs(total) >= thr);
    }
  }
  if (redo) {
    // exp2(64 - s^2 |x - y|^2) is at most 2^64 in fp32; the products and the sum are
    // taken in double, so neither the floor nor the range of fp32 is reached
    const float s2 = g.scale * g.scale;
    double acc = 0.0;
    for (int64_t j = threadIdx.x; j < g.N; j += kThreads) {
      float d2 = 0.0f;
      for (int k = 0; k < g.D; ++k) {
        const float d = g.x[i * g.D + k] - g.y[j * g.D + k];
        d2 = fmaf(d, d, d2);
      }
      acc += (double)exp2f(fmaf(-s2, d2, kDirectOffset)) * (double)g.b[j * g.E + e];
    }
    total = stream_block_sum(acc, red) * exp2(-(double)kDirectOffset);
  }
  if (threadIdx.x == 0) out[r] = (float)total;
}

void launch_stream_combine(const float *part, int nparts, int64_t count, float *out, const StreamGuard &g,
                           hipStream_t st) {
  hipLaunchKernelGGL(stream_combine_kernel, dim3((unsigned)count), dim3(kThreads), 0, st, part, nparts, count, out, g);
}

}  // namespace kmi
