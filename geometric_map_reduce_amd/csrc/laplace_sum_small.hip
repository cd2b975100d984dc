// Instantiations of the Laplacian kernel sum for D in 1..8 and 16.
#include "dispatch_gauss.h"
KMI_GAUSS_UNIT(laplace_dispatch_sum_small, OP_LAPLACE,
  KMI_GAUSS_E(OP_LAPLACE, 1) KMI_GAUSS_E(OP_LAPLACE, 2) KMI_GAUSS_E(OP_LAPLACE, 3) KMI_GAUSS_E(OP_LAPLACE, 4)
  KMI_GAUSS_E(OP_LAPLACE, 5) KMI_GAUSS_E(OP_LAPLACE, 6) KMI_GAUSS_E(OP_LAPLACE, 7) KMI_GAUSS_E(OP_LAPLACE, 8)
  KMI_GAUSS_E(OP_LAPLACE, 16))
