// combine.hip -- pass 2 of the split-j reductions and the fills of empty results.
//
// With S splits of the j range, pass 1 leaves S partial results per row:
//   sum / grad_x : partial sums,               combined as  sum_s p_s
//   LogSumExp    : (m_s, s_s) in log2 units,   combined as  v_s = m_s + log2 s_s,
//                  m = max_s v_s, out = ln2 (m + log2 sum_s 2^(v_s - m))
//   K-min        : sorted (d^2, j) lists,      merged by (d^2, j) order;
//   Max/ArgMax   : (value, j) pairs,           the largest value, then the smaller j.
// Splits are visited in order, so results do not depend on scheduling.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace kmi {

// The partials are added in split order; they are loaded eight at a time first, so
// that a thread waits for one round of loads per eight splits rather than one per
// split (at 10k rows, 40 splits: 9.3 us with the loads one at a time).
__global__ __launch_bounds__(kThreads) void sum_combine_kernel(const float *__restrict__ ws, int nsplit,
                                                               int64_t count, float *__restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= count) return;
  constexpr int U = 8;
  float s = 0.0f;
  for (int k0 = 0; k0 < nsplit; k0 += U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = k0 + u < nsplit ? ws[(int64_t)(k0 + u) * count + t] : 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (k0 + u < nsplit) s += v[u];
  }
  out[t] = s;
}

__global__ __launch_bounds__(kThreads) void lse_combine_kernel(const float *__restrict__ ws, int nsplit,
                                                               int64_t M, int E, float *__restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= M * E) return;
  const int64_t i = t / E;
  const int e = (int)(t - i * E);
  const int64_t stride = M * 2 * E;
  const float *p = ws + i * 2 * E + 2 * e;
  // each partial as one log2 value m_s + log2 s_s (a fixed-shift partial sum may be close
  // to the top of the fp32 range, so the sums are not added in their own scale)
  float m = -INFINITY;
  for (int k = 0; k < nsplit; ++k) m = fmaxf(m, p[k * stride] + log2f(p[k * stride + 1]));
  float s = 0.0f;
  if (m > -INFINITY)
    for (int k = 0; k < nsplit; ++k) s += exp2f(p[k * stride] + log2f(p[k * stride + 1]) - m);
  out[t] = m > -INFINITY ? kLn2 * (m + log2f(s)) : -INFINITY;
}

// The same merge with one work-group per output, for few outputs over many splits
// (the few-rows layout): the threads take the splits t, t + 256, ...; the maximum
// and the sum go through fixed-shape work-group reductions (deterministic for a
// given nsplit).  One thread per output looped over 2,048 splits with a dependent
// load each, and took 1 ms at 16 rows.
__global__ __launch_bounds__(kThreads) void lse_combine_rows_kernel(const float *__restrict__ ws, int nsplit,
                                                                    int64_t M, int E, float *__restrict__ out) {
  __shared__ float red[kThreads / kWave];
  const int64_t t = blockIdx.x;
  const int64_t i = t / E;
  const int e = (int)(t - i * E);
  const int64_t stride = M * 2 * E;
  const float *p = ws + i * 2 * E + 2 * e;
  float m = -INFINITY;
  for (int k = threadIdx.x; k < nsplit; k += kThreads) m = fmaxf(m, p[k * stride] + log2f(p[k * stride + 1]));
  m = block_max(m, red);
  float s = 0.0f;
  if (m > -INFINITY)
    for (int k = threadIdx.x; k < nsplit; k += kThreads) s += exp2f(p[k * stride] + log2f(p[k * stride + 1]) - m);
  s = row16_sum(s);
  s += __shfl_xor(s, 16);
  s += __shfl_xor(s, 32);
  __syncthreads();   // every thread has read the maxima out of red
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float tot = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / kWave; ++w) tot += red[w];
    out[t] = m > -INFINITY ? kLn2 * (m + log2f(tot)) : -INFINITY;
  }
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
__global__ __launch_bounds__(kThreads) void max_combine_kernel(const float *__restrict__ ws, int nsplit, int64_t M,
                                                               int E, float sign, float *__restrict__ out,
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

void launch_lse_combine(const float *ws, int nsplit, int64_t M, int E, float *out, hipStream_t st) {
  if (M * E > 0)
    hipLaunchKernelGGL(lse_combine_kernel, dim3(blocks_for(M * E)), dim3(kThreads), 0, st, ws, nsplit, M, E, out);
}

void launch_lse_combine_rows(const float *ws, int nsplit, int64_t M, int E, float *out, hipStream_t st) {
  if (M * E > 0)
    hipLaunchKernelGGL(lse_combine_rows_kernel, dim3((unsigned)(M * E)), dim3(kThreads), 0, st, ws, nsplit, M, E, out);
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

void launch_max_combine(const float *ws, int nsplit, int64_t M, int E, float sign, float *out, int64_t *out_idx,
                        hipStream_t st) {
  if (M * E > 0)
    hipLaunchKernelGGL(max_combine_kernel, dim3(blocks_for(M * E)), dim3(kThreads), 0, st, ws, nsplit, M, E, sign,
                       out, out_idx);
}

void launch_fill_i64(int64_t *out, int64_t count, int64_t v, hipStream_t st) {
  if (count > 0) hipLaunchKernelGGL(fill_i64_kernel, dim3(blocks_for(count)), dim3(kThreads), 0, st, out, count, v);
}

void launch_fill2(float *out, int64_t pairs, float v0, float v1, hipStream_t st) {
  if (pairs > 0) hipLaunchKernelGGL(fill2_kernel, dim3(blocks_for(pairs)), dim3(kThreads), 0, st, out, pairs, v0, v1);
}

}  // namespace kmi
