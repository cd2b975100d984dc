// Instantiations of the lse pass-1 kernel for D in 1..8 and 16.
#include "dispatch_gauss.h"
KMI_GAUSS_UNIT(gauss_dispatch_lse_small, OP_LSE,
  KMI_GAUSS_E(OP_LSE, 1) KMI_GAUSS_E(OP_LSE, 2) KMI_GAUSS_E(OP_LSE, 3) KMI_GAUSS_E(OP_LSE, 4)
  KMI_GAUSS_E(OP_LSE, 5) KMI_GAUSS_E(OP_LSE, 6) KMI_GAUSS_E(OP_LSE, 7) KMI_GAUSS_E(OP_LSE, 8)
  KMI_GAUSS_E(OP_LSE, 16))
