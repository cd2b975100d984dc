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
__global__ __launch_bounds__(kThreads) void stream_combine_kernel(const float *part, int nparts, int64_t count,
                                                                  float *out) {
  __shared__ double red[kThreads];
  const int64_t r = blockIdx.x;
  double v = 0.0;
  for (int p = threadIdx.x; p < nparts; p += kThreads) v += (double)part[(int64_t)p * count + r];
  red[threadIdx.x] = v;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[r] = (float)red[0];
}

void launch_stream_combine(const float *part, int nparts, int64_t count, float *out, hipStream_t st) {
  hipLaunchKernelGGL(stream_combine_kernel, dim3((unsigned)count), dim3(kThreads), 0, st, part, nparts, count, out);
}

}  // namespace kmi
