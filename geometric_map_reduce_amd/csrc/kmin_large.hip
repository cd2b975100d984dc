// Instantiations of the K-min pass-1 kernel (VALU path) for D in {16, 32, 50, 64, 100}.
#include "dispatch_kmin.h"
KMI_KMIN_UNIT(kmin_dispatch_large, KMI_KMIN_K(16) KMI_KMIN_K(32) KMI_KMIN_K(50) KMI_KMIN_K(64) KMI_KMIN_K(100))
