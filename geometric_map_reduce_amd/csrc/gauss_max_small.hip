// Instantiations of the Max/ArgMax pass-1 kernel for D in 1..8 and 16.
#include "dispatch_gauss.h"
KMI_GAUSS_UNIT(gauss_dispatch_max_small, OP_MAX,
  KMI_GAUSS_E(OP_MAX, 1) KMI_GAUSS_E(OP_MAX, 2) KMI_GAUSS_E(OP_MAX, 3) KMI_GAUSS_E(OP_MAX, 4)
  KMI_GAUSS_E(OP_MAX, 5) KMI_GAUSS_E(OP_MAX, 6) KMI_GAUSS_E(OP_MAX, 7) KMI_GAUSS_E(OP_MAX, 8)
  KMI_GAUSS_E(OP_MAX, 16))
