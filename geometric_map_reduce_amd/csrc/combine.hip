// combine.hip -- pass 2 of the split-j reductions and the fills of empty results.
//
// With S splits of the j range, pass 1 leaves S partial results per row:
//   sum / grad_x : partial sums,               combined as  sum_s p_s
//   LogSumExp    : (m_s, s_s) in log2 units,   combined as  m = max_s m_s,
//                  s = sum_s s_s 2^(m_s - m),  out = ln2 (m + log2 s)
//   K-min        : sorted (d^2, j) lists,      merged by (d^2, j) order;
//   Max/ArgMax   : (value, j) pairs,           the largest value, then the smaller j.
// Splits are visited in order, so results do not depend on scheduling.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace kmi {

__global__ __launch_bounds__(kThreads) void sum_combine_kernel(const float *__restrict__ ws, int nsplit,
                                                               int64_t count, float *__restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= count) return;
  float s = 0.0f;
  for (int k = 0; k < nsplit; ++k) s += ws[(int64_t)k * count + t];
  out[t] = s;
}

__global__ __launch_bounds__(kThreads) void lse_combine_kernel(const float *__restrict__ ws, int nsplit,
                                                               int64_t M, int E, float thr, float *__restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= M * E) return;
  const int64_t i = t / E;
  const int e = (int)(t - i * E);
  const int64_t stride = M * 2 * E;
  const float *p = ws + i * 2 * E + 2 * e;
  float m = -3.0e38f;
  for (int k = 0; k < nsplit; ++k) m = fmaxf(m, p[k * stride]);
  float s = 0.0f;
  for (int k = 0; k < nsplit; ++k) s += p[k * stride + 1] * exp2f(p[k * stride] - m);
  // a sum below thr (fixed-shift partials: possibly lost to underflow) or NaN is
  // left as NaN for the fix-up launch
  out[t] = s >= thr ? kLn2 * (m + log2f(s)) : __int_as_float(0x7fc00000);
}

// Maximum of b (or of |b|) over b[0..n), NaN ignored, -inf if empty: stage 1 writes
// one partial per work-group (grid-strided), stage 2 (one work-group) reduces them.
__device__ float block_max_f(float m, float *red) {
  red[threadIdx.x] = m;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  return red[0];
}

__global__ __launch_bounds__(kThreads) void bmax_kernel(const float *__restrict__ b, int64_t n, int absval,
                                                        float *__restrict__ part) {
  __shared__ float red[kThreads];
  float m = -INFINITY;
  for (int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x; t < n; t += (int64_t)gridDim.x * kThreads)
    m = fmaxf(m, absval ? fabsf(b[t]) : b[t]);
  m = block_max_f(m, red);
  if (threadIdx.x == 0) part[blockIdx.x] = m;
}

__global__ __launch_bounds__(kThreads) void bmax_final_kernel(const float *__restrict__ part, int nparts,
                                                              float *__restrict__ out) {
  __shared__ float red[kThreads];
  float m = -INFINITY;
  for (int t = threadIdx.x; t < nparts; t += kThreads) m = fmaxf(m, part[t]);
  m = block_max_f(m, red);
  if (threadIdx.x == 0) out[0] = m;
}

// Guarded sum / grad_x split launches: out[i][w] = (sum over splits of the unscaled
// partials) times the row factor f[i]; a row with threshold t[i] >= 0 whose sum is
// below it (or NaN) is written as NaN for the fix-up launch; t[i] < 0 marks a
// direct-form row (factor, then 2^-64).
__global__ __launch_bounds__(kThreads) void rows_combine_kernel(const float *__restrict__ ws, int nsplit, int64_t M,
                                                                int W, const float *__restrict__ f,
                                                                const float *__restrict__ t, float *__restrict__ out) {
  const int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (q >= M * W) return;
  const int64_t i = q / W;
  float s = 0.0f;
  for (int k = 0; k < nsplit; ++k) s += ws[(int64_t)k * M * W + q];
  const float ti = t[i];
  if (ti >= 0.0f) out[q] = fabsf(s) >= ti ? s * f[i] : __int_as_float(0x7fc00000);
  else out[q] = (s * f[i]) * exp2f(-kDirectOffset);
}

template <int K>
__global__ __launch_bounds__(kThreads) void kmin_combine_kernel(const float *__restrict__ pd, const int32_t *__restrict__ pi,
                                                                int nsplit, int64_t M, float *__restrict__ out_d,
                                                                int64_t *__restrict__ out_i) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= M) return;
  float bd[K];
  int bi[K];
#pragma unroll
  for (int k = 0; k < K; ++k) { bd[k] = INFINITY; bi[k] = 0x7fffffff; }
  for (int s = 0; s < nsplit; ++s) {
    const int64_t base = ((int64_t)s * M + i) * K;
    for (int q = 0; q < K; ++q) {
      const float v = pd[base + q];
      const int j = pi[base + q];
      if (j < 0) break;                              // rest of this list is empty
      if (!(v < bd[K - 1] || (v == bd[K - 1] && j < bi[K - 1]))) break;   // lists are sorted
#pragma unroll
      for (int k = K - 1; k > 0; --k) {
        const bool shift = v < bd[k - 1] || (v == bd[k - 1] && j < bi[k - 1]);
        const bool here = v < bd[k] || (v == bd[k] && j < bi[k]);
        const float nd = shift ? bd[k - 1] : (here ? v : bd[k]);
        const int ni = shift ? bi[k - 1] : (here ? j : bi[k]);
        bd[k] = nd;
        bi[k] = ni;
      }
      if (v < bd[0] || (v == bd[0] && j < bi[0])) { bd[0] = v; bi[0] = j; }
    }
  }
#pragma unroll
  for (int k = 0; k < K; ++k) {
    out_d[i * K + k] = bd[k];
    out_i[i * K + k] = bi[k] == 0x7fffffff ? -1 : (int64_t)bi[k];
  }
}

__global__ __launch_bounds__(kThreads) void fill_kernel(float *__restrict__ out, int64_t count, float v) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t < count) out[t] = v;
}

// Max/ArgMax: for row i, column e, the split with the largest signed value
// (NaN never wins), the smaller index among equal values; splits in order.
// rf, rt (optional): guarded launches leave the values unscaled; as in rows_combine,
// the row factor and threshold are applied here (a flagged row: NaN, index -1)
__global__ __launch_bounds__(kThreads) void max_combine_kernel(const float *__restrict__ ws, int nsplit, int64_t M,
                                                               int E, float sign, const float *__restrict__ rf,
                                                               const float *__restrict__ rt, float *__restrict__ out,
                                                               int64_t *__restrict__ out_idx) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= M * E) return;
  const int64_t i = t / E;
  const int e = (int)(t - i * E);
  const int64_t stride = M * 2 * E;
  const float *p = ws + i * 2 * E + 2 * e;
  float best = -INFINITY;
  int bi = -1;
  for (int k = 0; k < nsplit; ++k) {
    const float v = p[k * stride];
    const int j = __float_as_int(p[k * stride + 1]);
    if (j >= 0 && (v > best || (v == best && (bi < 0 || j < bi)))) { best = v; bi = j; }
  }
  if (rt) {
    const float ti = rt[i];
    if (ti >= 0.0f && !(fabsf(best) >= ti)) {
      out[t] = __int_as_float(0x7fc00000);
      out_idx[t] = -1;
      return;
    }
    best = ti >= 0.0f ? best * rf[i] : (best * rf[i]) * exp2f(-kDirectOffset);
  }
  out[t] = sign * best;
  out_idx[t] = (int64_t)bi;
}

__global__ __launch_bounds__(kThreads) void fill_i64_kernel(int64_t *__restrict__ out, int64_t count, int64_t v) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t < count) out[t] = v;
}

// out[2t] = v0, out[2t + 1] = v1: the neutral (max, sum) pair of LogSumExp partials
__global__ __launch_bounds__(kThreads) void fill2_kernel(float *__restrict__ out, int64_t pairs, float v0, float v1) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t < pairs) { out[2 * t] = v0; out[2 * t + 1] = v1; }
}

static inline unsigned blocks_for(int64_t n) { return (unsigned)((n + kThreads - 1) / kThreads); }

void launch_sum_combine(const float *ws, int nsplit, int64_t count, float *out, hipStream_t st) {
  if (count > 0) hipLaunchKernelGGL(sum_combine_kernel, dim3(blocks_for(count)), dim3(kThreads), 0, st, ws, nsplit, count, out);
}

void launch_lse_combine(const float *ws, int nsplit, int64_t M, int E, float thr, float *out, hipStream_t st) {
  if (M * E > 0)
    hipLaunchKernelGGL(lse_combine_kernel, dim3(blocks_for(M * E)), dim3(kThreads), 0, st, ws, nsplit, M, E, thr, out);
}

void launch_bmax(const float *b, int64_t n, bool absval, float *scratch, float *out, hipStream_t st) {
  const int64_t want = (n + 16 * kThreads - 1) / (16 * kThreads);   // about 16 loads per thread
  const int g = (int)std::max<int64_t>(1, std::min<int64_t>(kBmaxParts, want));
  hipLaunchKernelGGL(bmax_kernel, dim3(g), dim3(kThreads), 0, st, b, n, absval ? 1 : 0, scratch);
  hipLaunchKernelGGL(bmax_final_kernel, dim3(1), dim3(kThreads), 0, st, scratch, g, out);
}

void launch_rows_combine(const float *ws, int nsplit, int64_t M, int W, const float *f, const float *t, float *out,
                         hipStream_t st) {
  if (M * W > 0)
    hipLaunchKernelGGL(rows_combine_kernel, dim3(blocks_for(M * W)), dim3(kThreads), 0, st, ws, nsplit, M, W, f, t, out);
}

int launch_kmin_combine(const float *pd, const int32_t *pi, int nsplit, int64_t M, int K, float *out_d,
                        int64_t *out_i, hipStream_t st) {
  if (M == 0) return 0;
  const dim3 g(blocks_for(M)), b(kThreads);
  switch (K) {
#define KC(KK) case KK: hipLaunchKernelGGL((kmin_combine_kernel<KK>), g, b, 0, st, pd, pi, nsplit, M, out_d, out_i); return 0;
    KC(1) KC(2) KC(3) KC(4) KC(5) KC(6) KC(7) KC(8) KC(9) KC(10) KC(11) KC(12) KC(13) KC(14) KC(15) KC(16) KC(32)
#undef KC
    default: return -2;
  }
}

void launch_fill(float *out, int64_t count, float v, hipStream_t st) {
  if (count > 0) hipLaunchKernelGGL(fill_kernel, dim3(blocks_for(count)), dim3(kThreads), 0, st, out, count, v);
}

void launch_max_combine(const float *ws, int nsplit, int64_t M, int E, float sign, const float *rf, const float *rt,
                        float *out, int64_t *out_idx, hipStream_t st) {
  if (M * E > 0)
    hipLaunchKernelGGL(max_combine_kernel, dim3(blocks_for(M * E)), dim3(kThreads), 0, st, ws, nsplit, M, E, sign,
                       rf, rt, out, out_idx);
}

void launch_fill_i64(int64_t *out, int64_t count, int64_t v, hipStream_t st) {
  if (count > 0) hipLaunchKernelGGL(fill_i64_kernel, dim3(blocks_for(count)), dim3(kThreads), 0, st, out, count, v);
}

void launch_fill2(float *out, int64_t pairs, float v0, float v1, hipStream_t st) {
  if (pairs > 0) hipLaunchKernelGGL(fill2_kernel, dim3(blocks_for(pairs)), dim3(kThreads), 0, st, out, pairs, v0, v1);
}

}  // namespace kmi
