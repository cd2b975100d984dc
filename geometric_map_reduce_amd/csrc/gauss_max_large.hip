// Instantiations of the Max/ArgMax pass-1 kernel (VALU path) for D in {32, 50, 64, 100}.
#include "dispatch_gauss.h"
KMI_GAUSS_UNIT(gauss_dispatch_max_large, OP_MAX,
  KMI_GAUSS_E(OP_MAX, 32) KMI_GAUSS_E(OP_MAX, 50) KMI_GAUSS_E(OP_MAX, 64) KMI_GAUSS_E(OP_MAX, 100))
