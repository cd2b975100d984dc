// dispatch_kmin.h -- instantiation helper for the K-min dispatch units.
#pragma once

#include "kmin_kernel.h"
#include "launch.h"

#define KMI_KMIN_CASE(DD, KK)                                                            \
  if (D == DD && K == KK) {                                                              \
    if (info) {                                                                          \
      info->rows_per_wg = ::kmi::kThreads * ::kmi::KminShape<DD, KK>::R;                 \
      info->tile_j = ::kmi::KminShape<DD, KK>::TJ;                                       \
      return 0;                                                                          \
    }                                                                                    \
    ::kmi::launch_kmin_t<DD, KK>(grid, *args, st);                                       \
    return 0;                                                                            \
  }
#define KMI_KMIN_K(DD)                                                                   \
  KMI_KMIN_CASE(DD, 1) KMI_KMIN_CASE(DD, 2) KMI_KMIN_CASE(DD, 3) KMI_KMIN_CASE(DD, 4)    \
  KMI_KMIN_CASE(DD, 5) KMI_KMIN_CASE(DD, 6) KMI_KMIN_CASE(DD, 7) KMI_KMIN_CASE(DD, 8)    \
  KMI_KMIN_CASE(DD, 9) KMI_KMIN_CASE(DD, 10) KMI_KMIN_CASE(DD, 11) KMI_KMIN_CASE(DD, 12) \
  KMI_KMIN_CASE(DD, 13) KMI_KMIN_CASE(DD, 14) KMI_KMIN_CASE(DD, 15) KMI_KMIN_CASE(DD, 16) \
  KMI_KMIN_CASE(DD, 32)
#define KMI_KMIN_UNIT(NAME, BODY)                                                        \
  namespace kmi {                                                                        \
  int NAME(int D, int K, VariantInfo *info, dim3 grid, const KminArgs *args, hipStream_t st) { \
    BODY                                                                                 \
    return -2;                                                                           \
  }                                                                                      \
  }
