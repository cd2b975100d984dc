// Instantiations of the grad pass-1 kernel (VALU path) for D in {32, 50, 64, 100}.
#include "dispatch_gauss.h"
KMI_GAUSS_UNIT(gauss_dispatch_grad_large, OP_GRAD,
  KMI_GAUSS_E(OP_GRAD, 32) KMI_GAUSS_E(OP_GRAD, 50) KMI_GAUSS_E(OP_GRAD, 64) KMI_GAUSS_E(OP_GRAD, 100))
