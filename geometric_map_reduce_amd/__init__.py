"""MI355X (gfx950) engine for KeOps-style Gaussian map-reductions.

Reductions over the symbolic matrix K_ij = exp(-|x_i - y_j|^2 / sigma^2),
never stored, run as hand-written gfx950 HIP kernels behind the C ABI of
``include/keops_mi355x.h`` (library ``libkeops_mi355x.so``, built by
``geometric_map_reduce_amd.build``):

* ``keops_gauss_sum``    -- a_i = sum_j K_ij b_j
* ``keops_gauss_sum_noalloc`` -- the same with its workspace in a fixed device
  scratch of the library (no allocation during the call)
* ``keops_gauss_lse``    -- log sum_j exp(-|x_i - y_j|^2/sigma^2 + b_j)
* ``keops_gauss_grad_x`` -- gradient of the sum with respect to x
* ``keops_gauss_grad_y``, ``keops_gauss_grad_b`` -- gradients with respect to y
  and b (reductions over i, one output per point y_j)
* ``keops_gauss_*_ranges`` -- block-sparse sum, LSE and grad_x over kept pairs
  given as row and j ranges
* ``keops_gauss_cg``     -- conjugate-gradient solve of (K + lambda I) a = b
* ``keops_gauss_max``, ``keops_gauss_min`` -- Max/ArgMax and Min/ArgMin of K b
* ``keops_laplace_sum``  -- the Laplacian kernel sum, exp(-|x - y| / sigma)
* ``keops_kmin``         -- K nearest neighbours with indices

PyTorch supplies device memory and streams only.
"""
from .binding import (KEOPS_OPT_FAIL_ALLOC, KEOPS_OPT_FORM, KEOPS_OPT_MFMA, KEOPS_OPT_PROFILE,  # noqa: F401
                      KEOPS_OPT_ROWS, KEOPS_OPT_SPLIT_J, KEOPS_OPT_WG_TARGET, KEOPS_OPT_WS_CACHE, KeopsError,
                      keops_gauss_cg, keops_gauss_grad_b, keops_gauss_grad_x, keops_gauss_grad_x_ranges,
                      keops_gauss_grad_y, keops_gauss_lse, keops_gauss_lse_ranges, keops_gauss_max, keops_gauss_min,
                      keops_laplace_sum, keops_gauss_sum, keops_gauss_sum_noalloc, keops_gauss_sum_ranges,
                      keops_kmin, keops_profile_read, keops_set_option, keops_version, lib, status_string)
