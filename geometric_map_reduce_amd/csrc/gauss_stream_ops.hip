// Instantiations of the few-rows LogSumExp and gradient (D in 1..8, E in 1..4) and
// the gradient's pass 2.
#include "gauss_stream_ops.h"
#include "launch.h"

namespace kmi {

int gauss_dispatch_lse_stream(int D, int E, int mr, VariantInfo *info, dim3 grid, const StreamArgs *args,
                              hipStream_t st) {
#define KMI_STREAM_CASE(DD, EE)                                                  \
  if (D == DD && E == EE) {                                                      \
    if (mr != 4 && mr != stream_rows_large(DD, EE)) return -2;                   \
    if (info) {                                                                  \
      info->rows_per_wg = mr;                                                    \
      info->tile_j = kThreads * stream_j(DD, EE);                                \
      return 0;                                                                  \
    }                                                                            \
    if (mr == 4) launch_gauss_stream_lse_t<DD, EE, 4>(grid, *args, st);          \
    else launch_gauss_stream_lse_t<DD, EE, stream_rows_large(DD, EE)>(grid, *args, st); \
    return 0;                                                                    \
  }
#define KMI_STREAM_E(DD) KMI_STREAM_CASE(DD, 1) KMI_STREAM_CASE(DD, 2) KMI_STREAM_CASE(DD, 3) KMI_STREAM_CASE(DD, 4)
  KMI_STREAM_E(1) KMI_STREAM_E(2) KMI_STREAM_E(3) KMI_STREAM_E(4)
  KMI_STREAM_E(5) KMI_STREAM_E(6) KMI_STREAM_E(7) KMI_STREAM_E(8)
#undef KMI_STREAM_E
#undef KMI_STREAM_CASE
  return -2;
}

int gauss_dispatch_grad_stream(int D, int E, int mr, VariantInfo *info, dim3 grid, const StreamArgs *args,
                               hipStream_t st) {
#define KMI_STREAM_CASE(DD, EE)                                                  \
  if (D == DD && E == EE) {                                                      \
    if (mr != 4 && mr != stream_grad_mr_large(DD)) return -2;                    \
    if (info) {                                                                  \
      info->rows_per_wg = mr;                                                    \
      info->tile_j = kThreads * stream_j(DD, EE);                                \
      return 0;                                                                  \
    }                                                                            \
    if (mr == 4) launch_gauss_stream_grad_t<DD, EE, 4>(grid, *args, st);         \
    else launch_gauss_stream_grad_t<DD, EE, stream_grad_mr_large(DD)>(grid, *args, st); \
    return 0;                                                                    \
  }
#define KMI_STREAM_E(DD) KMI_STREAM_CASE(DD, 1) KMI_STREAM_CASE(DD, 2) KMI_STREAM_CASE(DD, 3) KMI_STREAM_CASE(DD, 4)
  KMI_STREAM_E(1) KMI_STREAM_E(2) KMI_STREAM_E(3) KMI_STREAM_E(4)
  KMI_STREAM_E(5) KMI_STREAM_E(6) KMI_STREAM_E(7) KMI_STREAM_E(8)
#undef KMI_STREAM_E
#undef KMI_STREAM_CASE
  return -2;
}

// One work-group per output (i, d): the partials in order of p, in double, through a
// fixed-shape tree (deterministic for a given nparts).  A non-finite total is
// recomputed over every j: exp2(64 - s^2 |x - y|^2) in fp32 (at most 2^64), the
// products and the sum in double, 2^-64 applied at the end.
__device__ double stream_grad_block_sum(double v, double *red) {
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

__global__ __launch_bounds__(kThreads) void stream_grad_combine_kernel(const float *part, int nparts, int64_t M,
                                                                       float *out, StreamGuard g) {
  __shared__ double red[kThreads];
  const int64_t r = blockIdx.x;   // output i * D + d
  const int D = g.D, E = g.E;
  const int64_t i = r / D;
  const int d = (int)(r - i * D);
  double v = 0.0;
  for (int p = threadIdx.x; p < nparts; p += kThreads) v += (double)part[(int64_t)p * M * D + r];
  double total = stream_grad_block_sum(v, red);
  if (!isfinite(total)) {   // uniform: every thread holds the same total
    const float s2 = g.scale * g.scale;
    double acc = 0.0;
    for (int64_t j = threadIdx.x; j < g.N; j += kThreads) {
      float d2 = 0.0f;
      for (int k = 0; k < D; ++k) {
        const float df = g.x[i * D + k] - g.y[j * D + k];
        d2 = fmaf(df, df, d2);
      }
      double gb = 0.0;
      for (int e = 0; e < E; ++e) gb += (double)(E == 1 ? 1.0f : g.g[i * E + e]) * (double)g.b[j * E + e];
      acc += (double)exp2f(fmaf(-s2, d2, kDirectOffset)) * gb * (double)(g.x[i * D + d] - g.y[j * D + d]);
    }
    total = stream_grad_block_sum(acc, red) * exp2(-(double)kDirectOffset) * (double)g.coef *
            (E == 1 ? (double)g.g[i] : 1.0);
  }
  if (threadIdx.x == 0) out[r] = (float)total;
}

void launch_stream_grad_combine(const float *part, int nparts, int64_t M, float *out, const StreamGuard &g,
                                hipStream_t st) {
  hipLaunchKernelGGL(stream_grad_combine_kernel, dim3((unsigned)(M * g.D)), dim3(kThreads), 0, st, part, nparts, M,
                     out, g);
}

}  // namespace kmi
