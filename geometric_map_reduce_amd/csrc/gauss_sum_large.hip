// Instantiations of the sum pass-1 kernel (VALU path) for D in {32, 50, 64, 100}.
#include "dispatch_gauss.h"
KMI_GAUSS_UNIT(gauss_dispatch_sum_large, OP_SUM,
  KMI_GAUSS_E(OP_SUM, 32) KMI_GAUSS_E(OP_SUM, 50) KMI_GAUSS_E(OP_SUM, 64) KMI_GAUSS_E(OP_SUM, 100))
