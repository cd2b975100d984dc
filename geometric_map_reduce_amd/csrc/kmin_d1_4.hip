// Instantiations of the K-min pass-1 kernel for D in 1..4.
#include "dispatch_kmin.h"
KMI_KMIN_UNIT(kmin_dispatch_d1_4, KMI_KMIN_K(1) KMI_KMIN_K(2) KMI_KMIN_K(3) KMI_KMIN_K(4))
