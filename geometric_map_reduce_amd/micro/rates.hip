// rates.hip -- instruction-rate microbenchmarks of one MI355X (gfx950), built as
// libkeops_micro.so next to the engine library (never linked into it).
//
// Each probe is a kernel of independent dependency chains with no memory
// traffic in its timed loop, launched over every CU; the host times it with HIP
// events and, from the first wave, reads the shader clock counter (s_memtime)
// against the constant-rate wall clock (s_memrealtime) to give the engine clock
// the probe actually ran at.  The rates that the engine's design rests on:
//   fma, add, exp         fp32 VALU FMA, add and the transcendental v_exp_f32;
//   fma_exp               FMA and exp chains interleaved in one wave (co-issue?);
//   mfma_f32, mfma_bf16   v_mfma_f32_16x16x4f32 and v_mfma_f32_16x16x32_bf16;
//   mfma_fma_wave         MFMA and FMA chains interleaved in one wave;
//   mfma_exp_wave         MFMA and exp chains interleaved in one wave;
//   split_{mfma,valu,both}  eight-wave work-groups, waves 0-3 MFMA-only and waves
//                         4-7 exp + FMA only (each SIMD holds one of each): run
//                         alone and together, they show whether the matrix pipe
//                         of one wave overlaps the VALU work of another;
//   pair_valu             the Gaussian sum's VALU pair map with records from LDS:
//                         three FMAs, one exp2 and one add per pair;
//   pair_mfma             the same pairs with the exponent from one
//                         v_mfma_f32_16x16x4f32 per 16 x 16 pairs (rows in the A
//                         operand, LDS records in B), then exp2 and an FMA with b;
//   bank_{free,two,three} v_fmac_f32 chains whose three VGPR reads sit in three, two or
//                         one register bank (index mod 4).
// Work per launch is returned to the host so that rates need no duplicated
// constants: keops_micro_run fills per-wave instruction counts.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kCh = 8;      // independent chains per probe
constexpr int kUnroll = 16;

struct Clock {
  unsigned long long t0, t1, w0, w1;
};

__device__ __forceinline__ void clock_start(Clock *c, unsigned tid = 0) {
  if (blockIdx.x == 0 && threadIdx.x == tid) {
    c->t0 = clock64();
    c->w0 = wall_clock64();
  }
}
__device__ __forceinline__ void clock_stop(Clock *c, unsigned tid = 0) {
  if (blockIdx.x == 0 && threadIdx.x == tid) {
    c->t1 = clock64();
    c->w1 = wall_clock64();
  }
}

// the chains' values reach memory only when they hit a value they never take, so
// no instruction of the loop is dead to the compiler
__device__ __forceinline__ void sink(float *out, float v) {
  if (v == -1.2345e-30f) out[threadIdx.x] = v;
}

__global__ void k_fma(float *out, Clock *c, int iters) {
  clock_start(c);
  float v[kCh];
  for (int k = 0; k < kCh; ++k) v[k] = 1e-3f * threadIdx.x + k;
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int k = 0; k < kCh; ++k) v[k] = fmaf(v[k], 0.999f, 0.001f);
  float s = 0.0f;
  for (int k = 0; k < kCh; ++k) s += v[k];
  sink(out, s);
  clock_stop(c);
}

__global__ void k_add(float *out, Clock *c, int iters) {
  clock_start(c);
  float v[kCh], w[kCh];
  for (int k = 0; k < kCh; ++k) { v[k] = 1e-3f * threadIdx.x + k; w[k] = 1e-7f * (k + 1); }
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int k = 0; k < kCh; ++k) v[k] = v[k] + w[k];
  float s = 0.0f;
  for (int k = 0; k < kCh; ++k) s += v[k];
  sink(out, s);
  clock_stop(c);
}

__global__ void k_exp(float *out, Clock *c, int iters) {
  clock_start(c);
  float v[kCh];
  for (int k = 0; k < kCh; ++k) v[k] = 1e-3f * threadIdx.x + 0.1f * k;
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int k = 0; k < kCh; ++k) v[k] = __builtin_amdgcn_exp2f(-v[k]);   // stays in [0.5, 1]
  float s = 0.0f;
  for (int k = 0; k < kCh; ++k) s += v[k];
  sink(out, s);
  clock_stop(c);
}

// per unrolled step: kCh FMAs on one chain set and kCh/4 exps on another
__global__ void k_fma_exp(float *out, Clock *c, int iters) {
  clock_start(c);
  float v[kCh], e[kCh / 4];
  for (int k = 0; k < kCh; ++k) v[k] = 1e-3f * threadIdx.x + k;
  for (int k = 0; k < kCh / 4; ++k) e[k] = 1e-3f * threadIdx.x + 0.1f * k;
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
      for (int k = 0; k < kCh; ++k) v[k] = fmaf(v[k], 0.999f, 0.001f);
#pragma unroll
      for (int k = 0; k < kCh / 4; ++k) e[k] = __builtin_amdgcn_exp2f(-e[k]);
    }
  float s = 0.0f;
  for (int k = 0; k < kCh; ++k) s += v[k];
  for (int k = 0; k < kCh / 4; ++k) s += e[k];
  sink(out, s);
  clock_stop(c);
}

constexpr int kMf = 4;   // independent MFMA accumulators

__global__ void k_mfma_f32(float *out, Clock *c, int iters) {
  clock_start(c);
  floatx4 acc[kMf];
  const float a = 1e-3f * threadIdx.x, b = 0.5f;
  for (int k = 0; k < kMf; ++k) acc[k] = floatx4{0.f, 0.f, 0.f, (float)k};
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int k = 0; k < kMf; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[k], 0, 0, 0);
  float s = 0.0f;
  for (int k = 0; k < kMf; ++k) s += acc[k][0] + acc[k][3];
  sink(out, s);
  clock_stop(c);
}

__global__ void k_mfma_bf16(float *out, Clock *c, int iters) {
  clock_start(c);
  floatx4 acc[kMf];
  bf16x8 a, b;
  for (int q = 0; q < 8; ++q) { a[q] = (__bf16)(1e-3f * threadIdx.x); b[q] = (__bf16)0.5f; }
  for (int k = 0; k < kMf; ++k) acc[k] = floatx4{0.f, 0.f, 0.f, (float)k};
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int k = 0; k < kMf; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[k], 0, 0, 0);
  float s = 0.0f;
  for (int k = 0; k < kMf; ++k) s += acc[k][0] + acc[k][3];
  sink(out, s);
  clock_stop(c);
}

// per unrolled step: kMf MFMAs and kCh FMAs, independent, in one wave
__global__ void k_mfma_fma_wave(float *out, Clock *c, int iters) {
  clock_start(c);
  floatx4 acc[kMf];
  float v[kCh];
  const float a = 1e-3f * threadIdx.x, b = 0.5f;
  for (int k = 0; k < kMf; ++k) acc[k] = floatx4{0.f, 0.f, 0.f, (float)k};
  for (int k = 0; k < kCh; ++k) v[k] = 1e-3f * threadIdx.x + k;
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
      for (int k = 0; k < kMf; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[k], 0, 0, 0);
#pragma unroll
      for (int k = 0; k < kCh; ++k) v[k] = fmaf(v[k], 0.999f, 0.001f);
    }
  float s = 0.0f;
  for (int k = 0; k < kMf; ++k) s += acc[k][0] + acc[k][3];
  for (int k = 0; k < kCh; ++k) s += v[k];
  sink(out, s);
  clock_stop(c);
}

// per unrolled step: kMf MFMAs and kCh exps, independent, in one wave
__global__ void k_mfma_exp_wave(float *out, Clock *c, int iters) {
  clock_start(c);
  floatx4 acc[kMf];
  float v[kCh];
  const float a = 1e-3f * threadIdx.x, b = 0.5f;
  for (int k = 0; k < kMf; ++k) acc[k] = floatx4{0.f, 0.f, 0.f, (float)k};
  for (int k = 0; k < kCh; ++k) v[k] = 1e-3f * threadIdx.x + 0.1f * k;
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
      for (int k = 0; k < kMf; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[k], 0, 0, 0);
#pragma unroll
      for (int k = 0; k < kCh; ++k) v[k] = __builtin_amdgcn_exp2f(-v[k]);
    }
  float s = 0.0f;
  for (int k = 0; k < kMf; ++k) s += acc[k][0] + acc[k][3];
  for (int k = 0; k < kCh; ++k) s += v[k];
  sink(out, s);
  clock_stop(c);
}

// Eight-wave work-groups: waves 0-3 run MFMA chains, waves 4-7 exp + FMA chains
// (per unrolled step kCh/2 exps and kCh FMAs); roles = 1 MFMA waves only,
// 2 VALU waves only, 3 both (the idle waves return at once).
__global__ __launch_bounds__(512) void k_split(float *out, Clock *c, int iters, int roles) {
  const unsigned ct = (roles & 1) ? 0 : 256;   // the clock is read by a wave that runs
  clock_start(c, ct);
  const int wave = threadIdx.x / 64;
  float s = 0.0f;
  if (wave < 4) {
    if (!(roles & 1)) return;
    floatx4 acc[kMf];
    const float a = 1e-3f * threadIdx.x, b = 0.5f;
    for (int k = 0; k < kMf; ++k) acc[k] = floatx4{0.f, 0.f, 0.f, (float)k};
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int k = 0; k < kMf; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[k], 0, 0, 0);
    for (int k = 0; k < kMf; ++k) s += acc[k][0] + acc[k][3];
  } else {
    if (!(roles & 2)) return;
    float v[kCh], e[kCh / 2];
    for (int k = 0; k < kCh; ++k) v[k] = 1e-3f * threadIdx.x + k;
    for (int k = 0; k < kCh / 2; ++k) e[k] = 1e-3f * threadIdx.x + 0.1f * k;
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
        for (int k = 0; k < kCh; ++k) v[k] = fmaf(v[k], 0.999f, 0.001f);
#pragma unroll
        for (int k = 0; k < kCh / 2; ++k) e[k] = __builtin_amdgcn_exp2f(-e[k]);
      }
    for (int k = 0; k < kCh; ++k) s += v[k];
    for (int k = 0; k < kCh / 2; ++k) s += e[k];
  }
  sink(out, s);
  clock_stop(c, ct);
}

// Gaussian-sum pair map, VALU form: 256-thread work-groups, two rows per lane,
// 256 LDS records (2y', c) per tile read by broadcast, four j per group; per
// pair three FMAs, one exp2, one add.  One iteration = one pass over the tile.
__global__ __launch_bounds__(256) void k_pair_valu(float *out, Clock *c, int iters) {
  __shared__ float4 rec[256];
  const int t = threadIdx.x;
  rec[t] = make_float4(0.01f * (t & 15), -0.02f * (t >> 4), 0.003f * t, -1.0f - 0.01f * t);
  __syncthreads();
  clock_start(c);
  const float x0[2] = {0.1f + 1e-4f * t, -0.2f}, x1[2] = {0.3f, 0.05f + 1e-4f * t}, x2[2] = {-0.1f, 0.2f};
  float acc[2] = {0.0f, 0.0f};
  for (int i = 0; i < iters; ++i) {
    for (int j = 0; j < 256; j += 4) {
      asm volatile("" ::: "memory");   // the records are read in the loop, as in the engine
      float4 r[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) r[u] = rec[j + u];
      float q[4][2];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 2; ++w) q[u][w] = fmaf(x0[w], r[u].x, fmaf(x1[w], r[u].y, fmaf(x2[w], r[u].z, r[u].w)));
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 2; ++w) acc[w] += __builtin_amdgcn_exp2f(q[u][w]);
    }
  }
  sink(out, acc[0] + acc[1]);
  clock_stop(c);
}

// Gaussian-sum pair map, MFMA form: each wave owns 4 tiles of 16 rows; per 16 j
// one B operand (lane l: component l/16 of record l%16) and b (lane l: b of
// record l%16) from LDS, four v_mfma_f32_16x16x4f32 giving 4 x 16 x 16 exponents,
// then one exp2 and one FMA per pair.  One iteration = one pass over 256 j.
__global__ __launch_bounds__(256) void k_pair_mfma(float *out, Clock *c, int iters) {
  __shared__ float brec[256 * 4];   // [j / 16][k][j % 16]
  __shared__ float bval[256];
  const int t = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float v = k == 3 ? -1.0f - 0.01f * t : 0.01f * ((t * (k + 3)) & 31);
    brec[(t >> 4) * 64 + k * 16 + (t & 15)] = v;
  }
  bval[t] = (t & 1) ? 0.5f : -0.25f;
  __syncthreads();
  clock_start(c);
  const int lane = t & 63;
  float xa[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) xa[q] = (lane >> 4) == 3 ? 1.0f : 0.01f * (lane & 15) + 0.1f * q;
  const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
  float acc[4][4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[q][r] = 0.0f;
  for (int i = 0; i < iters; ++i) {
    for (int j16 = 0; j16 < 256; j16 += 16) {
      asm volatile("" ::: "memory");   // the operands are read in the loop, as in the engine
      const float yb = brec[j16 * 4 + lane];
      const float bj = bval[j16 + (lane & 15)];
      floatx4 d[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) d[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[q], yb, zero, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[q][r] = fmaf(__builtin_amdgcn_exp2f(d[q][r]), bj, acc[q][r]);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int r = 0; r < 4; ++r) s += acc[q][r];
  sink(out, s);
  clock_stop(c);
}

// VGPR bank probes: eight independent v_fmac_f32 chains (d = s0 * s1 + d reads three
// VGPRs) with every operand pinned to a physical register, so that the register bank
// (index mod 4) of the three reads is fixed: variant 0 puts them in three different
// banks, variant 1 two of them in one bank, variant 2 all three in one bank.  The
// rate difference is the cost of a bank conflict.  No memory access in the asm.
#define KMI_BANK_BODY(A0, A1, A2, A3, A4, A5, A6, A7, X0, X1, X2, X3, X4, X5, X6, X7, Y0, Y1, Y2, Y3, Y4, Y5, Y6, Y7) \
  asm volatile(                                                                                                  \
      "v_fmac_f32 %0, %8, %16\n\tv_fmac_f32 %1, %9, %17\n\tv_fmac_f32 %2, %10, %18\n\t"                            \
      "v_fmac_f32 %3, %11, %19\n\tv_fmac_f32 %4, %12, %20\n\tv_fmac_f32 %5, %13, %21\n\t"                          \
      "v_fmac_f32 %6, %14, %22\n\tv_fmac_f32 %7, %15, %23"                                                        \
      : "+{" A0 "}"(a[0]), "+{" A1 "}"(a[1]), "+{" A2 "}"(a[2]), "+{" A3 "}"(a[3]), "+{" A4 "}"(a[4]),            \
        "+{" A5 "}"(a[5]), "+{" A6 "}"(a[6]), "+{" A7 "}"(a[7])                                                    \
      : "{" X0 "}"(x[0]), "{" X1 "}"(x[1]), "{" X2 "}"(x[2]), "{" X3 "}"(x[3]), "{" X4 "}"(x[4]),                 \
        "{" X5 "}"(x[5]), "{" X6 "}"(x[6]), "{" X7 "}"(x[7]), "{" Y0 "}"(y[0]), "{" Y1 "}"(y[1]),                 \
        "{" Y2 "}"(y[2]), "{" Y3 "}"(y[3]), "{" Y4 "}"(y[4]), "{" Y5 "}"(y[5]), "{" Y6 "}"(y[6]), "{" Y7 "}"(y[7]))

template <int V>
__global__ void k_bank(float *out, Clock *c, int iters) {
  clock_start(c);
  float a[8], x[8], y[8];
  // run-time operands, so that the compiler keeps them in their registers instead of
  // re-creating constants before every asm block
  for (int k = 0; k < 8; ++k) {
    a[k] = 1e-3f * threadIdx.x + k;
    x[k] = 0.999f - 1e-9f * (threadIdx.x + 7 * k);
    y[k] = 1e-4f * (k + 1) + 1e-9f * threadIdx.x;
  }
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (V == 0)   // acc bank b, s0 bank b+1, s1 bank b+2
        KMI_BANK_BODY("v8", "v9", "v10", "v11", "v12", "v13", "v14", "v15",
                      "v17", "v18", "v19", "v16", "v21", "v22", "v23", "v20",
                      "v26", "v27", "v24", "v25", "v30", "v31", "v28", "v29");
      else if (V == 1)   // acc and s0 in one bank, s1 in the next
        KMI_BANK_BODY("v8", "v9", "v10", "v11", "v12", "v13", "v14", "v15",
                      "v16", "v17", "v18", "v19", "v20", "v21", "v22", "v23",
                      "v25", "v26", "v27", "v24", "v29", "v30", "v31", "v28");
      else   // all three in one bank
        KMI_BANK_BODY("v8", "v9", "v10", "v11", "v12", "v13", "v14", "v15",
                      "v16", "v17", "v18", "v19", "v20", "v21", "v22", "v23",
                      "v24", "v25", "v26", "v27", "v28", "v29", "v30", "v31");
    }
  float s = 0.0f;
  for (int k = 0; k < 8; ++k) s += a[k];
  sink(out, s);
  clock_stop(c);
}
#undef KMI_BANK_BODY


// HBM read probe: float4 loads, four in flight per thread, summed into registers;
// one float written per thread.  mode 0: grid-stride over the whole buffer; mode 1:
// work-group w reads its own contiguous chunk, threads striding by the work-group
// (the access pattern of the few-rows kernels, which stream y and b that way).
__global__ __launch_bounds__(256) void k_hbm_read(const float4 *__restrict__ buf, int64_t n4, int64_t chunk4,
                                                  int mode, float *sink) {
  int64_t i, end, stride;
  if (mode == 0) {
    i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    end = n4;
    stride = (int64_t)gridDim.x * blockDim.x;
  } else {
    i = (int64_t)blockIdx.x * chunk4 + threadIdx.x;
    end = (int64_t)(blockIdx.x + 1) * chunk4 < n4 ? (int64_t)(blockIdx.x + 1) * chunk4 : n4;
    stride = blockDim.x;
  }
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (; i + 3 * stride < end; i += 4 * stride) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = buf[i + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u) { acc.x += v[u].x; acc.y += v[u].y; acc.z += v[u].z; acc.w += v[u].w; }
  }
  for (; i < end; i += stride) {
    const float4 v = buf[i];
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc.x + acc.y + acc.z + acc.w;
}

}  // namespace

extern "C" {

// Reads the device buffer `buf` of n floats (n a multiple of 4, 16-byte aligned)
// once with `blocks` work-groups of 256 threads in `mode` (see k_hbm_read); `sink`
// holds blocks * 256 floats.  *ms = kernel time (HIP events).  Returns 0, -1 for
// invalid arguments, -4 on a HIP error.
int keops_micro_hbm(const float *buf, int64_t n, float *sink, int blocks, int mode, float *ms) {
  if (!buf || !sink || !ms || n < 4 || (n & 3) || ((uintptr_t)buf & 15) || blocks < 1 || mode < 0 || mode > 1)
    return -1;
  const int64_t n4 = n / 4;
  const int64_t chunk4 = (n4 + blocks - 1) / blocks;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = 0;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    rc = -4;
  } else {
    (void)hipEventRecord(e0, nullptr);
    hipLaunchKernelGGL(k_hbm_read, dim3((unsigned)blocks), dim3(256), 0, nullptr,
                       reinterpret_cast<const float4 *>(buf), n4, chunk4, mode, sink);
    (void)hipEventRecord(e1, nullptr);
    if (hipGetLastError() != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
        hipEventElapsedTime(ms, e0, e1) != hipSuccess)
      rc = -4;
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  return rc;
}

// Probe ids, in the order listed at the top of this file.
enum {
  P_FMA = 0, P_ADD, P_EXP, P_FMA_EXP, P_MFMA_F32, P_MFMA_BF16, P_MFMA_FMA_WAVE, P_MFMA_EXP_WAVE,
  P_SPLIT_MFMA, P_SPLIT_VALU, P_SPLIT_BOTH, P_PAIR_VALU, P_PAIR_MFMA, P_BANK_FREE, P_BANK_TWO, P_BANK_THREE, P_COUNT
};

int keops_micro_count(void) { return P_COUNT; }

// Runs probe `probe` over `blocks` work-groups for `iters` loop iterations:
// *ms = kernel time (HIP events), *clk_mhz = the engine clock of the first wave's
// run, and counts[0..4] = per-wave instructions of the timed loop:
//   [0] VALU FMA, [1] VALU add, [2] v_exp_f32, [3] fp32 MFMA 16x16x4, [4] bf16 MFMA 16x16x32;
// counts[5] = waves (or, for split_both, MFMA + VALU wave pairs) that run them, counts[6] = Gaussian pairs evaluated per launch
// (pair probes), counts[7] = threads per work-group.  Returns 0, -1 for an unknown
// probe, -4 on a HIP error.
int keops_micro_run(int probe, int blocks, int iters, float *ms, double *clk_mhz, double *counts) {
  if (probe < 0 || probe >= P_COUNT || blocks < 1 || iters < 1 || !ms || !clk_mhz || !counts) return -1;
  for (int k = 0; k < 8; ++k) counts[k] = 0.0;
  const double n = (double)iters * kUnroll;
  int threads = 256;
  double waves = (double)blocks * 4;
  switch (probe) {
    case P_FMA: counts[0] = n * kCh; break;
    case P_ADD: counts[1] = n * kCh; break;
    case P_EXP: counts[2] = n * kCh; break;
    case P_FMA_EXP: counts[0] = n * kCh; counts[2] = n * kCh / 4; break;
    case P_MFMA_F32: counts[3] = n * kMf; break;
    case P_MFMA_BF16: counts[4] = n * kMf; break;
    case P_MFMA_FMA_WAVE: counts[3] = n * kMf; counts[0] = n * kCh; break;
    case P_MFMA_EXP_WAVE: counts[3] = n * kMf; counts[2] = n * kCh; break;
    case P_SPLIT_MFMA: threads = 512; counts[3] = n * kMf; break;
    case P_SPLIT_VALU: threads = 512; counts[0] = n * kCh; counts[2] = n * kCh / 2; break;
    case P_SPLIT_BOTH: threads = 512; counts[3] = n * kMf; counts[0] = n * kCh; counts[2] = n * kCh / 2; break;
    case P_PAIR_VALU: counts[6] = (double)blocks * 256 * 2 * 256 * iters; break;
    case P_PAIR_MFMA: counts[6] = (double)blocks * 4 * 64 * 256 * iters; break;
    case P_BANK_FREE: case P_BANK_TWO: case P_BANK_THREE: counts[0] = n * 8; break;
  }
  // split probes: four waves of each role per work-group; the counts of split_both are
  // those of one MFMA wave plus one VALU wave
  counts[5] = waves;
  counts[7] = threads;
  float *out = nullptr;
  Clock *clk = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = 0;
  if (hipMalloc((void **)&out, 512 * sizeof(float)) != hipSuccess ||
      hipMalloc((void **)&clk, sizeof(Clock)) != hipSuccess || hipEventCreate(&e0) != hipSuccess ||
      hipEventCreate(&e1) != hipSuccess) {
    rc = -4;
  } else {
    const dim3 g((unsigned)blocks), b((unsigned)threads);
    (void)hipEventRecord(e0, nullptr);
    switch (probe) {
      case P_FMA: hipLaunchKernelGGL(k_fma, g, b, 0, nullptr, out, clk, iters); break;
      case P_ADD: hipLaunchKernelGGL(k_add, g, b, 0, nullptr, out, clk, iters); break;
      case P_EXP: hipLaunchKernelGGL(k_exp, g, b, 0, nullptr, out, clk, iters); break;
      case P_FMA_EXP: hipLaunchKernelGGL(k_fma_exp, g, b, 0, nullptr, out, clk, iters); break;
      case P_MFMA_F32: hipLaunchKernelGGL(k_mfma_f32, g, b, 0, nullptr, out, clk, iters); break;
      case P_MFMA_BF16: hipLaunchKernelGGL(k_mfma_bf16, g, b, 0, nullptr, out, clk, iters); break;
      case P_MFMA_FMA_WAVE: hipLaunchKernelGGL(k_mfma_fma_wave, g, b, 0, nullptr, out, clk, iters); break;
      case P_MFMA_EXP_WAVE: hipLaunchKernelGGL(k_mfma_exp_wave, g, b, 0, nullptr, out, clk, iters); break;
      case P_SPLIT_MFMA: hipLaunchKernelGGL(k_split, g, b, 0, nullptr, out, clk, iters, 1); break;
      case P_SPLIT_VALU: hipLaunchKernelGGL(k_split, g, b, 0, nullptr, out, clk, iters, 2); break;
      case P_SPLIT_BOTH: hipLaunchKernelGGL(k_split, g, b, 0, nullptr, out, clk, iters, 3); break;
      case P_PAIR_VALU: hipLaunchKernelGGL(k_pair_valu, g, b, 0, nullptr, out, clk, iters); break;
      case P_PAIR_MFMA: hipLaunchKernelGGL(k_pair_mfma, g, b, 0, nullptr, out, clk, iters); break;
      case P_BANK_FREE: hipLaunchKernelGGL(k_bank<0>, g, b, 0, nullptr, out, clk, iters); break;
      case P_BANK_TWO: hipLaunchKernelGGL(k_bank<1>, g, b, 0, nullptr, out, clk, iters); break;
      case P_BANK_THREE: hipLaunchKernelGGL(k_bank<2>, g, b, 0, nullptr, out, clk, iters); break;
    }
    (void)hipEventRecord(e1, nullptr);
    Clock h{};
    if (hipGetLastError() != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
        hipEventElapsedTime(ms, e0, e1) != hipSuccess ||
        hipMemcpy(&h, clk, sizeof(Clock), hipMemcpyDeviceToHost) != hipSuccess) {
      rc = -4;
    } else {
      int khz = 0;
      int dev = 0;
      (void)hipGetDevice(&dev);
      if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0) khz = 100000;
      const double wall_s = (double)(h.w1 - h.w0) / (khz * 1e3);
      *clk_mhz = wall_s > 0 ? (double)(h.t1 - h.t0) / wall_s / 1e6 : 0.0;
    }
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (out) (void)hipFree(out);
  if (clk) (void)hipFree(clk);
  return rc;
}

}  // extern "C"
