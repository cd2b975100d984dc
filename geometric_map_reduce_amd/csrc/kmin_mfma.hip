// Instantiations of the fp32-MFMA K-min for D in {32, 50, 64, 100} and K <= 16
// (K = 32 at these D runs on the VALU K-min kernel).
#include "kmin_mfma.h"
#include "launch.h"

namespace kmi {

int kmin_dispatch_mfma(int D, int K, VariantInfo *info, dim3 grid, const KminArgs *args, hipStream_t st) {
#define KMI_KMM_CASE(DD, KK)                                          \
  if (D == DD && K == KK) {                                           \
    if (info) {                                                       \
      info->rows_per_wg = KminMfmaShape<DD, KK>::ROWS_WG;             \
      info->tile_j = KminMfmaShape<DD, KK>::TJ;                       \
      return 0;                                                       \
    }                                                                 \
    launch_kmin_mfma_t<DD, KK>(grid, *args, st);                      \
    return 0;                                                         \
  }
#define KMI_KMM_K(DD)                                                                        \
  KMI_KMM_CASE(DD, 1) KMI_KMM_CASE(DD, 2) KMI_KMM_CASE(DD, 3) KMI_KMM_CASE(DD, 4)           \
  KMI_KMM_CASE(DD, 5) KMI_KMM_CASE(DD, 6) KMI_KMM_CASE(DD, 7) KMI_KMM_CASE(DD, 8)           \
  KMI_KMM_CASE(DD, 9) KMI_KMM_CASE(DD, 10) KMI_KMM_CASE(DD, 11) KMI_KMM_CASE(DD, 12)        \
  KMI_KMM_CASE(DD, 13) KMI_KMM_CASE(DD, 14) KMI_KMM_CASE(DD, 15) KMI_KMM_CASE(DD, 16)
  KMI_KMM_K(32) KMI_KMM_K(50) KMI_KMM_K(64) KMI_KMM_K(100)
#undef KMI_KMM_K
#undef KMI_KMM_CASE
  return -2;
}

}  // namespace kmi
