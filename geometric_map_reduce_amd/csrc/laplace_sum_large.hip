// Instantiations of the Laplacian kernel sum for D in {32, 50, 64, 100}.
#include "dispatch_gauss.h"
KMI_GAUSS_UNIT(laplace_dispatch_sum_large, OP_LAPLACE,
  KMI_GAUSS_E(OP_LAPLACE, 32) KMI_GAUSS_E(OP_LAPLACE, 50) KMI_GAUSS_E(OP_LAPLACE, 64) KMI_GAUSS_E(OP_LAPLACE, 100))
