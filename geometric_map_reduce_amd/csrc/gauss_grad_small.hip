// Instantiations of the grad pass-1 kernel for D in 1..8 and 16.
#include "dispatch_gauss.h"
KMI_GAUSS_UNIT(gauss_dispatch_grad_small, OP_GRAD,
  KMI_GAUSS_E(OP_GRAD, 1) KMI_GAUSS_E(OP_GRAD, 2) KMI_GAUSS_E(OP_GRAD, 3) KMI_GAUSS_E(OP_GRAD, 4)
  KMI_GAUSS_E(OP_GRAD, 5) KMI_GAUSS_E(OP_GRAD, 6) KMI_GAUSS_E(OP_GRAD, 7) KMI_GAUSS_E(OP_GRAD, 8)
  KMI_GAUSS_E(OP_GRAD, 16))
