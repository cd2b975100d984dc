// Instantiations of the K-min with the split-bf16 MFMA prefilter for D in
// {32, 50, 64, 100} and K in 1..16 and 32.
#include "kmin_mfma_split.h"
#include "launch.h"

namespace kmi {

int kmin_dispatch_mfma_split(int D, int K, VariantInfo *info, dim3 grid, const KminArgs *args, hipStream_t st) {
#define KMI_KMS_CASE(DD, KK)                                          \
  if (D == DD && K == KK) {                                           \
    if (info) {                                                       \
      info->rows_per_wg = KminSplitShape<DD, KK>::ROWS_WG;            \
      info->tile_j = KminSplitShape<DD, KK>::TJ;                      \
      return 0;                                                       \
    }                                                                 \
    launch_kmin_mfma_split_t<DD, KK>(grid, *args, st);                \
    return 0;                                                         \
  }
#define KMI_KMS_K(DD)                                                                        \
  KMI_KMS_CASE(DD, 1) KMI_KMS_CASE(DD, 2) KMI_KMS_CASE(DD, 3) KMI_KMS_CASE(DD, 4)           \
  KMI_KMS_CASE(DD, 5) KMI_KMS_CASE(DD, 6) KMI_KMS_CASE(DD, 7) KMI_KMS_CASE(DD, 8)           \
  KMI_KMS_CASE(DD, 9) KMI_KMS_CASE(DD, 10) KMI_KMS_CASE(DD, 11) KMI_KMS_CASE(DD, 12)        \
  KMI_KMS_CASE(DD, 13) KMI_KMS_CASE(DD, 14) KMI_KMS_CASE(DD, 15) KMI_KMS_CASE(DD, 16)           \
  KMI_KMS_CASE(DD, 32)
  KMI_KMS_K(32) KMI_KMS_K(50) KMI_KMS_K(64) KMI_KMS_K(100)
#undef KMI_KMS_K
#undef KMI_KMS_CASE
  return -2;
}

}  // namespace kmi
