// Instantiations of the sum pass-1 kernel for D in 1..8 and 16.
#include "dispatch_gauss.h"
KMI_GAUSS_UNIT(gauss_dispatch_sum_small, OP_SUM,
  KMI_GAUSS_E(OP_SUM, 1) KMI_GAUSS_E(OP_SUM, 2) KMI_GAUSS_E(OP_SUM, 3) KMI_GAUSS_E(OP_SUM, 4)
  KMI_GAUSS_E(OP_SUM, 5) KMI_GAUSS_E(OP_SUM, 6) KMI_GAUSS_E(OP_SUM, 7) KMI_GAUSS_E(OP_SUM, 8)
  KMI_GAUSS_E(OP_SUM, 16))
