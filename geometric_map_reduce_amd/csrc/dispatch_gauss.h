// dispatch_gauss.h -- instantiation helper for the gauss dispatch units.
#pragma once

#include "gauss_kernel.h"
#include "launch.h"

#define KMI_GAUSS_CASE(OP, DD, EE)                                                       \
  if (D == DD && E == EE) {                                                              \
    constexpr int RW = ::kmi::gauss_rows_wide(OP, DD, EE);                               \
    if (info) {                                                                          \
      info->rows_per_wg = ::kmi::kThreads * (wide ? RW : 1);                             \
      info->tile_j = ::kmi::GaussShape<OP, DD, EE>::TJ;                                  \
      return 0;                                                                          \
    }                                                                                    \
    if (wide) ::kmi::launch_gauss_t<OP, DD, EE, RW>(grid, *args, st);                    \
    else ::kmi::launch_gauss_t<OP, DD, EE, 1>(grid, *args, st);                          \
    return 0;                                                                            \
  }
#define KMI_GAUSS_E(OP, DD) KMI_GAUSS_CASE(OP, DD, 1) KMI_GAUSS_CASE(OP, DD, 2) \
                            KMI_GAUSS_CASE(OP, DD, 3) KMI_GAUSS_CASE(OP, DD, 4)

#define KMI_GAUSS_UNIT(NAME, OP, BODY)                                                   \
  namespace kmi {                                                                        \
  int NAME(int D, int E, int wide, VariantInfo *info, dim3 grid, const GaussArgs *args,  \
           hipStream_t st) {                                                             \
    BODY                                                                                 \
    return -2;                                                                           \
  }                                                                                      \
  }
