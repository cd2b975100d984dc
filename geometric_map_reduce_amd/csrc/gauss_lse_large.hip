// Instantiations of the lse pass-1 kernel (VALU path) for D in {32, 50, 64, 100}.
#include "dispatch_gauss.h"
KMI_GAUSS_UNIT(gauss_dispatch_lse_large, OP_LSE,
  KMI_GAUSS_E(OP_LSE, 32) KMI_GAUSS_E(OP_LSE, 50) KMI_GAUSS_E(OP_LSE, 64) KMI_GAUSS_E(OP_LSE, 100))
