// Instantiations of the few-rows K-min (lanes own j; D in 1..8, K in 1..16 and 32).
#include "kmin_stream.h"
#include "launch.h"

namespace kmi {

int kmin_dispatch_stream(int D, int K, VariantInfo *info, dim3 grid, const KminArgs *args, hipStream_t st) {
#define KMI_KST_CASE(DD, KK)                                          \
  if (D == DD && K == KK) {                                           \
    if (info) {                                                       \
      info->rows_per_wg = kmin_stream_rows(KK);                       \
      info->tile_j = kThreads * kmin_stream_j(DD);                    \
      return 0;                                                       \
    }                                                                 \
    launch_kmin_stream_t<DD, KK>(grid, *args, st);                    \
    return 0;                                                         \
  }
#define KMI_KST_K(DD)                                                                        \
  KMI_KST_CASE(DD, 1) KMI_KST_CASE(DD, 2) KMI_KST_CASE(DD, 3) KMI_KST_CASE(DD, 4)           \
  KMI_KST_CASE(DD, 5) KMI_KST_CASE(DD, 6) KMI_KST_CASE(DD, 7) KMI_KST_CASE(DD, 8)           \
  KMI_KST_CASE(DD, 9) KMI_KST_CASE(DD, 10) KMI_KST_CASE(DD, 11) KMI_KST_CASE(DD, 12)        \
  KMI_KST_CASE(DD, 13) KMI_KST_CASE(DD, 14) KMI_KST_CASE(DD, 15) KMI_KST_CASE(DD, 16)       \
  KMI_KST_CASE(DD, 32)
  KMI_KST_K(1) KMI_KST_K(2) KMI_KST_K(3) KMI_KST_K(4) KMI_KST_K(5) KMI_KST_K(6) KMI_KST_K(7) KMI_KST_K(8)
#undef KMI_KST_K
#undef KMI_KST_CASE
  return -2;
}

int launch_kmin_stream_combine(const float *pd, const int32_t *pi, int nsplit, int64_t M, int K, float *out_d,
                               int64_t *out_i, hipStream_t st) {
  if (M == 0) return 0;
  if (M > 0x7fffffff) return -2;
  const dim3 g((unsigned)M), b(kThreads);
  switch (K) {
#define KC(KK) case KK: hipLaunchKernelGGL((kmin_stream_combine_kernel<KK>), g, b, 0, st, pd, pi, nsplit, M, out_d, out_i); return 0;
    KC(1) KC(2) KC(3) KC(4) KC(5) KC(6) KC(7) KC(8) KC(9) KC(10) KC(11) KC(12) KC(13) KC(14) KC(15) KC(16) KC(32)
#undef KC
    default: return -2;
  }
}

}  // namespace kmi
