// Instantiations of the K-min pass-1 kernel for D in 5..8.
#include "dispatch_kmin.h"
KMI_KMIN_UNIT(kmin_dispatch_d5_8, KMI_KMIN_K(5) KMI_KMIN_K(6) KMI_KMIN_K(7) KMI_KMIN_K(8))
