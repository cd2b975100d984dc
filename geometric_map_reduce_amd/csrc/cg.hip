// cg.hip -- vector kernels of the conjugate-gradient solver of (K + lam I) a = b
// (KeOps README feature list: a conjugate gradient solver for spline
// interpolation or kriging).  The products K p come from the Gaussian sum
// kernels; everything else of an iteration runs here, on E <= 4 independent
// columns at once.  Dot products are reduced in double, in two passes over a
// fixed grid, so every iteration is bitwise reproducible.
#include "common.h"
#include "launch.h"

namespace kmi {

namespace {

// Sum of one double per thread over the work-group; every thread gets it.
__device__ double block_sum_d(double v, double *red) {
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

template <int E>
__device__ void write_partials(const double (&acc)[E], double *part) {
  __shared__ double red[kThreads];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const double s = block_sum_d(acc[e], red);
    if (threadIdx.x == 0) part[(int64_t)blockIdx.x * E + e] = s;
  }
}

// a = 0, r = p = b; partials of <b, b>
template <int E>
__global__ __launch_bounds__(kThreads) void cg_init_kernel(const float *b, int64_t N, float *a, float *r, float *p,
                                                           double *part) {
  double acc[E] = {};
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < N; i += (int64_t)gridDim.x * kThreads) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float v = b[i * E + e];
      a[i * E + e] = 0.0f;
      r[i * E + e] = v;
      p[i * E + e] = v;
      acc[e] += (double)v * (double)v;
    }
  }
  write_partials<E>(acc, part);
}

// q = K p + lam p (q holds K p on entry); partials of <p, q>
template <int E>
__global__ __launch_bounds__(kThreads) void cg_apply_kernel(const float *p, float *q, float lam, int64_t N,
                                                            double *part) {
  double acc[E] = {};
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < N; i += (int64_t)gridDim.x * kThreads) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float pv = p[i * E + e];
      const float qv = fmaf(lam, pv, q[i * E + e]);
      q[i * E + e] = qv;
      acc[e] += (double)pv * (double)qv;
    }
  }
  write_partials<E>(acc, part);
}

// alpha_e = rr_e / pq_e; a += alpha p; r -= alpha q; partials of <r, r>
template <int E>
__global__ __launch_bounds__(kThreads) void cg_step_kernel(float *a, float *r, const float *p, const float *q,
                                                           const double *rr, const double *pq, int64_t N,
                                                           double *part) {
  float alpha[E];
#pragma unroll
  for (int e = 0; e < E; ++e) alpha[e] = pq[e] > 0.0 ? (float)(rr[e] / pq[e]) : 0.0f;
  double acc[E] = {};
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < N; i += (int64_t)gridDim.x * kThreads) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      a[i * E + e] = fmaf(alpha[e], p[i * E + e], a[i * E + e]);
      const float rv = fmaf(-alpha[e], q[i * E + e], r[i * E + e]);
      r[i * E + e] = rv;
      acc[e] += (double)rv * (double)rv;
    }
  }
  write_partials<E>(acc, part);
}

// beta_e = rr_new_e / rr_old_e; p = r + beta p
template <int E>
__global__ __launch_bounds__(kThreads) void cg_direction_kernel(float *p, const float *r, const double *rr_new,
                                                                const double *rr_old, int64_t N) {
  float beta[E];
#pragma unroll
  for (int e = 0; e < E; ++e) beta[e] = rr_old[e] > 0.0 ? (float)(rr_new[e] / rr_old[e]) : 0.0f;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < N; i += (int64_t)gridDim.x * kThreads) {
#pragma unroll
    for (int e = 0; e < E; ++e) p[i * E + e] = fmaf(beta[e], p[i * E + e], r[i * E + e]);
  }
}

// r = b - q; partials of <r, r> (the true residual after K a + lam a in q)
template <int E>
__global__ __launch_bounds__(kThreads) void cg_residual_kernel(const float *b, const float *q, int64_t N,
                                                               double *part) {
  double acc[E] = {};
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < N; i += (int64_t)gridDim.x * kThreads) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const double rv = (double)b[i * E + e] - (double)q[i * E + e];
      acc[e] += rv * rv;
    }
  }
  write_partials<E>(acc, part);
}

// out[e] = sum over the nblk partials, in block order (one work-group)
__global__ __launch_bounds__(kThreads) void cg_finish_kernel(const double *part, int nblk, int E, double *out) {
  __shared__ double red[kThreads];
  for (int e = 0; e < E; ++e) {
    double v = 0.0;
    for (int k = threadIdx.x; k < nblk; k += kThreads) v += part[(int64_t)k * E + e];
    const double s = block_sum_d(v, red);
    if (threadIdx.x == 0) out[e] = s;
  }
}

unsigned cg_grid(int64_t N) {
  const int64_t want = (N + kThreads - 1) / kThreads;
  return (unsigned)(want < kCgBlocks ? (want > 0 ? want : 1) : kCgBlocks);
}

}  // namespace

#define KMI_CG_E(STMT)                 \
  switch (E) {                         \
    case 1: { constexpr int EE = 1; STMT; } break; \
    case 2: { constexpr int EE = 2; STMT; } break; \
    case 3: { constexpr int EE = 3; STMT; } break; \
    case 4: { constexpr int EE = 4; STMT; } break; \
    default: break;                    \
  }

void launch_cg_init(const float *b, int64_t N, int E, float *a, float *r, float *p, double *part, double *out,
                    hipStream_t st) {
  const unsigned g = cg_grid(N);
  KMI_CG_E(hipLaunchKernelGGL((cg_init_kernel<EE>), dim3(g), dim3(kThreads), 0, st, b, N, a, r, p, part))
  hipLaunchKernelGGL(cg_finish_kernel, dim3(1), dim3(kThreads), 0, st, part, (int)g, E, out);
}

void launch_cg_apply(const float *p, float *q, float lam, int64_t N, int E, double *part, double *out,
                     hipStream_t st) {
  const unsigned g = cg_grid(N);
  KMI_CG_E(hipLaunchKernelGGL((cg_apply_kernel<EE>), dim3(g), dim3(kThreads), 0, st, p, q, lam, N, part))
  hipLaunchKernelGGL(cg_finish_kernel, dim3(1), dim3(kThreads), 0, st, part, (int)g, E, out);
}

void launch_cg_step(float *a, float *r, const float *p, const float *q, const double *rr, const double *pq,
                    int64_t N, int E, double *part, double *out, hipStream_t st) {
  const unsigned g = cg_grid(N);
  KMI_CG_E(hipLaunchKernelGGL((cg_step_kernel<EE>), dim3(g), dim3(kThreads), 0, st, a, r, p, q, rr, pq, N, part))
  hipLaunchKernelGGL(cg_finish_kernel, dim3(1), dim3(kThreads), 0, st, part, (int)g, E, out);
}

void launch_cg_direction(float *p, const float *r, const double *rr_new, const double *rr_old, int64_t N, int E,
                         hipStream_t st) {
  const unsigned g = cg_grid(N);
  KMI_CG_E(hipLaunchKernelGGL((cg_direction_kernel<EE>), dim3(g), dim3(kThreads), 0, st, p, r, rr_new, rr_old, N))
}

void launch_cg_residual(const float *b, const float *q, int64_t N, int E, double *part, double *out,
                        hipStream_t st) {
  const unsigned g = cg_grid(N);
  KMI_CG_E(hipLaunchKernelGGL((cg_residual_kernel<EE>), dim3(g), dim3(kThreads), 0, st, b, q, N, part))
  hipLaunchKernelGGL(cg_finish_kernel, dim3(1), dim3(kThreads), 0, st, part, (int)g, E, out);
}

#undef KMI_CG_E

}  // namespace kmi
