// Instantiations of the fp32-MFMA Gaussian gradient with respect to x for D in
// {32, 50, 64, 100} (at D = 100 in eight-wave work-groups of two row tiles per wave).
#include "gauss_mfma.h"
#include "launch.h"

namespace kmi {

int gauss_dispatch_grad_mfma(int D, int E, int wide, VariantInfo *info, dim3 grid, const GaussArgs *args,
                             hipStream_t st) {
  (void)wide;
#define KMI_MFMA_CASE(DD, EE)                                          \
  if (D == DD && E == EE) {                                            \
    if (info) {                                                        \
      info->rows_per_wg = MfmaGradShape<DD>::ROWS_WG;                  \
      info->tile_j = MfmaShape<DD>::TJ;                                \
      return 0;                                                        \
    }                                                                  \
    launch_gauss_mfma_grad_t<DD, EE>(grid, *args, st);                 \
    return 0;                                                          \
  }
#define KMI_MFMA_E(DD) KMI_MFMA_CASE(DD, 1) KMI_MFMA_CASE(DD, 2) KMI_MFMA_CASE(DD, 3) KMI_MFMA_CASE(DD, 4)
  KMI_MFMA_E(32) KMI_MFMA_E(50) KMI_MFMA_E(64) KMI_MFMA_E(100)
#undef KMI_MFMA_E
#undef KMI_MFMA_CASE
  return -2;
}

}  // namespace kmi
