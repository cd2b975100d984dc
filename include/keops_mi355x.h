/*
 * keops_mi355x.h -- C ABI of the MI355X (gfx950) Gaussian map-reduce engine.
 *
 * The engine evaluates reductions over a symbolic matrix M_ij = F(x_i, y_j)
 * that is never stored: coefficients are computed on the fly, tile by tile,
 * with memory linear in M + N.  Sources (web pages about the KeOps library):
 *
 *  [KO-GPU]  "Kernel Operations on the GPU, with Autodiff, without Memory
 *            Overflows" (paper summary page): §1 "Target operation" (the
 *            Gaussian kernel product a_i = sum_j k(x_i, y_j) b_j, x_i, y_j in
 *            R^D, Gaussian k of deviation sigma > 0, M and N up to a billion);
 *            §2 "Generic reduction framework" (sum, max, argmin, log-sum-exp
 *            reductions of formulas over i- and j-variables), "Performance and
 *            differentiation" (argKmin; autodiff); §4 (D <= 100).
 *  [README]  KeOps README: "symbolic matrices" paragraph (c) (formula
 *            evaluated on the fly on data arrays x_i, y_j); PyTorch example
 *            (D_ij = sum of squared differences, K_ij = exp(-D_ij), .sum(),
 *            .logsumexp(), .argmin(), grad of (a**2).sum()).
 *  [ISSUE]   GitHub issue "Transparent interface for billion-scale matrices":
 *            an output parameter so that the user allocates the result
 *            tensor, and calls made without holding the Python lock.
 *
 * Common conventions for every entry point
 * ----------------------------------------
 *  Memory:    every array pointer is a DEVICE pointer on the HIP device that is
 *             current on the calling thread.  Arrays are dense, row-major,
 *             fp32 (indices int64), at least 4-byte aligned.
 *  Ownership: the caller allocates every input and output ([ISSUE], item 1).
 *             The library keeps no reference after returning, except through
 *             work queued on `stream`; the caller keeps the buffers alive
 *             until the stream has passed that work.  Outputs must not overlap
 *             inputs.  Split-j workspace belongs to the library: one device
 *             buffer per (device, stream), allocated on first need, grown
 *             when a call needs more, and reused in stream order by later
 *             calls on that stream, so that a call allocates nothing once
 *             its stream has seen a call of its size.  A buffer is freed
 *             (with hipFree) when it grows, when more than 32 are held, or
 *             when KEOPS_OPT_WS_CACHE is set to 2.  Destroy a stream only
 *             after its calls' work has completed: a stream created later
 *             may reuse the handle, and with it the buffer.
 *  Stream:    `stream` is a hipStream_t passed as void* (NULL = the default
 *             stream).  Calls only enqueue work and never synchronise; kernel
 *             faults surface at the caller's next synchronisation.
 *  Threads:   reentrant; may be called concurrently from several host
 *             threads on different streams.  Calls running concurrently on
 *             one GPU do not share memory.
 *  Errors:    0 = KEOPS_OK, negative = error (see below); no exception ever
 *             crosses the ABI, and on an error nothing has been enqueued.
 *  Sizes:     M = 0 is a no-op.  N = 0: sums and gradients are 0, LogSumExp
 *             is -inf; K-min needs 1 <= K <= N.
 *  Supported: D in 1..8, 16, 32, 50, 64, 100; E in 1..4; K in 1..16 or 32.
 *             Other values return KEOPS_ERR_UNSUPPORTED.
 *  Kernel:    k(x, y) = exp(-|x - y|^2 / sigma^2)   (sigma finite, > 0)
 *             (sigma = 1 is the README's exp(-D_ij)).
 */
#ifndef KEOPS_MI355X_H
#define KEOPS_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KEOPS_OK 0
#define KEOPS_ERR_INVALID_ARG (-1)  /* null pointer with non-zero size, negative size,
                                       sigma not finite or <= 0, K > N, overlap  */
#define KEOPS_ERR_UNSUPPORTED (-2)  /* D, E or K outside the compiled set; N >= 2^31 for K-min */
#define KEOPS_ERR_ALLOC (-3)        /* workspace allocation failed                 */
#define KEOPS_ERR_HIP (-4)          /* a HIP call or kernel launch failed          */
#define KEOPS_ERR_SCRATCH (-5)      /* keops_gauss_sum_noalloc: the call needs more device
                                       scratch than the library holds                 */

/*
 * Gaussian kernel sum ([KO-GPU] §1 "Target operation"; [README] K_ij.sum(dim=1)):
 *   out[i, e] = sum_j exp(-|x_i - y_j|^2 / sigma^2) * b[j, e]
 * x: [M, D], y: [N, D], b: [N, E], out: [M, E].
 */
int keops_gauss_sum(const float *x, const float *y, const float *b,
                    int64_t M, int64_t N, int32_t D, int32_t E, float sigma,
                    float *out, void *stream);

/*
 * keops_gauss_sum without any allocation, for callers that cannot allocate device
 * memory during the call: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.  Arguments, layouts, results and errors are those
 * of keops_gauss_sum (the same kernels run); the difference is the workspace.  Instead
 * of stream-ordered allocations, the split-j partial results (and, at D >= 32, one
 * form flag per 256 rows) go to a fixed 64 MiB device array inside the library, one
 * copy per GPU, allocated when the library's code is first loaded on that GPU and
 * held until the process ends.  When the partials of the usual launch plan do not
 * fit, the call uses fewer j-splits (at the fewest, none: then no scratch is used),
 * which changes only the fp32 rounding order.  KEOPS_ERR_SCRATCH: the form flags
 * alone exceed the array (D >= 32 with M above about 4e9 rows); nothing is enqueued.
 * Every call on one GPU uses that GPU's same array, which keeps the last call's
 * contents: calls that overlap in time on one GPU (different streams or threads,
 * not ordered by the caller) race on it and give undefined results.  Nothing in the
 * array needs to start at zero.
 */
int keops_gauss_sum_noalloc(const float *x, const float *y, const float *b,
                            int64_t M, int64_t N, int32_t D, int32_t E, float sigma,
                            float *out, void *stream);

/*
 * LogSumExp reduction ([KO-GPU] §2 reductions list; [README] .logsumexp()):
 *   out[i, e] = log sum_j exp(-|x_i - y_j|^2 / sigma^2 + b[j, e])
 * b enters additively in the exponent.  Shapes as keops_gauss_sum.
 */
int keops_gauss_lse(const float *x, const float *y, const float *b,
                    int64_t M, int64_t N, int32_t D, int32_t E, float sigma,
                    float *out, void *stream);

/*
 * Max / ArgMax and Min / ArgMin reductions of the kernel product ([KO-GPU] §2
 * reductions list; [README] feature list "Sum, LogSumExp, Min, Max but also
 * ArgMin, ArgMax"):
 *   keops_gauss_max: out[i, e] = max_j K_ij b[j, e],  out_idx[i, e] = its j
 *   keops_gauss_min: out[i, e] = min_j K_ij b[j, e],  out_idx[i, e] = its j
 * with K_ij = exp(-|x_i - y_j|^2/sigma^2); among equal values the smaller j is
 * returned.  out: [M, E] fp32; out_idx: [M, E] int64, 8-byte aligned.  The
 * values are compared in fp32 as computed (K to about 1e-6 relative), so two
 * j whose products differ by less than that may be returned either way.
 * N = 0 gives -inf (max) or +inf (min) and index -1; NaN products never win.
 * Requires N < 2^31.
 */
int keops_gauss_max(const float *x, const float *y, const float *b, int64_t M, int64_t N, int32_t D, int32_t E,
                    float sigma, float *out, int64_t *out_idx, void *stream);
int keops_gauss_min(const float *x, const float *y, const float *b, int64_t M, int64_t N, int32_t D, int32_t E,
                    float sigma, float *out, int64_t *out_idx, void *stream);

/*
 * Laplacian kernel sum ([README] feature list: a wide range of formulas,
 * beyond the Gaussian kernel):
 *   out[i, e] = sum_j exp(-|x_i - y_j| / sigma) b[j, e],  |.| the Euclidean norm.
 * Shapes, conventions and errors as keops_gauss_sum.  Computed from raw
 * differences (never the expanded distance, whose rounding near x = y would
 * reach the square root).
 */
int keops_laplace_sum(const float *x, const float *y, const float *b, int64_t M, int64_t N, int32_t D, int32_t E,
                      float sigma, float *out, void *stream);

/*
 * Gradient of the kernel sum with respect to x ([KO-GPU] §2 "Performance and
 * differentiation"; [README] torch.autograd.grad((a_i ** 2).sum(), [x])), as
 * the vector-Jacobian product with the cotangent g = dL/da:
 *   out[i, d] = sum_j (-2/sigma^2) exp(-|x_i-y_j|^2/sigma^2) <g_i, b_j> (x[i,d] - y[j,d])
 * g: [M, E]; out: [M, D].  For L = sum_i |a_i|^2 pass g = 2a.
 */
int keops_gauss_grad_x(const float *x, const float *y, const float *b, const float *g,
                       int64_t M, int64_t N, int32_t D, int32_t E, float sigma,
                       float *out, void *stream);

/*
 * Gradients of L = sum_ie g_ie a_ie with respect to the other two inputs of
 * the kernel sum ([KO-GPU] §2 "Performance and differentiation": every input
 * of a reduction is differentiable).  Both are reductions over the rows i,
 * one output per point y_j (the transposed map-reduce):
 *   keops_gauss_grad_y:  out[j, d] = sum_i (2/sigma^2) K_ij <g_i, b_j> (x[i,d] - y[j,d])   out: [N, D]
 *   keops_gauss_grad_b:  out[j, e] = sum_i K_ij g[i, e]                                    out: [N, E]
 * with K_ij = exp(-|x_i - y_j|^2/sigma^2), x: [M, D], y: [N, D], b: [N, E],
 * g: [M, E] (dL/da).  Sizes: N = 0 is a no-op; M = 0 writes zeros.  The rest
 * of the conventions (pointers, ownership, stream, errors) are those above;
 * out must not overlap any input.
 */
int keops_gauss_grad_y(const float *x, const float *y, const float *b, const float *g,
                       int64_t M, int64_t N, int32_t D, int32_t E, float sigma,
                       float *out, void *stream);
int keops_gauss_grad_b(const float *x, const float *y, const float *g,
                       int64_t M, int64_t N, int32_t D, int32_t E, float sigma,
                       float *out, void *stream);

/*
 * Block-sparse reductions ([KO-GPU] §3 "Applications": cluster-wise
 * block-sparsity for large kernel linear systems, §4: the block-sparse
 * truncation rule; [README] feature list: an interface for block-sparse
 * strategies).  Only the kept pairs (i, j) enter the reduction; they are given
 * as ranges over rows and points, typically of points sorted by cluster:
 *   ranges_i    [nri][2]  row range c = [ranges_i[c][0], ranges_i[c][1]); row
 *                         ranges must not overlap;
 *   slices_i    [nri]     end (exclusive) in redranges_j of row range c's j
 *                         ranges, non-decreasing; they start at slices_i[c-1]
 *                         (0 for c = 0);
 *   redranges_j [nrj][2]  j range k = [redranges_j[k][0], redranges_j[k][1])
 *                         inside [0, N).
 * Row i in row range c reduces over the j of its ranges, in the listed order
 * (a j listed twice counts twice); rows in no row range get the empty
 * reduction (0, or -inf for LogSumExp).  The three arrays are HOST arrays of
 * int64 (the library validates them and plans the launch on the host, then
 * copies what the kernels need); x, y, b, g, out are device arrays as above.
 * These calls synchronise `stream` once, after that copy.  Any invalid range
 * (out of bounds, overlapping row ranges, decreasing slices) returns
 * KEOPS_ERR_INVALID_ARG before any device work.
 *   keops_gauss_sum_ranges:    out [M, E] as keops_gauss_sum over the kept pairs
 *   keops_gauss_lse_ranges:    out [M, E] as keops_gauss_lse over the kept pairs
 *   keops_gauss_grad_x_ranges: out [M, D] as keops_gauss_grad_x over the kept pairs
 */
int keops_gauss_sum_ranges(const float *x, const float *y, const float *b, int64_t M, int64_t N, int32_t D,
                           int32_t E, float sigma, const int64_t *ranges_i, int64_t nri, const int64_t *slices_i,
                           const int64_t *redranges_j, int64_t nrj, float *out, void *stream);
int keops_gauss_lse_ranges(const float *x, const float *y, const float *b, int64_t M, int64_t N, int32_t D,
                           int32_t E, float sigma, const int64_t *ranges_i, int64_t nri, const int64_t *slices_i,
                           const int64_t *redranges_j, int64_t nrj, float *out, void *stream);
int keops_gauss_grad_x_ranges(const float *x, const float *y, const float *b, const float *g, int64_t M, int64_t N,
                              int32_t D, int32_t E, float sigma, const int64_t *ranges_i, int64_t nri,
                              const int64_t *slices_i, const int64_t *redranges_j, int64_t nrj, float *out,
                              void *stream);

/*
 * Conjugate-gradient solve of (K + lambda I) a = b with the Gaussian kernel
 * matrix of one point set, K_ij = exp(-|x_i - x_j|^2/sigma^2) ([README] feature
 * list: a conjugate gradient solver for spline interpolation, kriging or
 * Gaussian process regression).  Each of the E <= 4 columns of b is solved
 * independently, starting from a = 0, until |r_e| <= rtol |b_e| for every
 * column (r the recursively updated residual) or after max_iter iterations.
 * Every product K p is one keops_gauss_sum.
 *   x: [N, D]; b, out (= a): [N, E]; sigma > 0; lambda >= 0; rtol >= 0.
 *   iters (host, may be NULL): iterations run.
 *   rel_residual (host [E], may be NULL): the true |b - (K + lambda I) a| / |b|
 *     of the returned a, from one more product (0 for a zero column of b).
 * Unlike the reductions above this call synchronises `stream`: it reads the
 * residual norms on the host after every iteration.  Returns KEOPS_OK also when
 * max_iter is reached first (see iters and rel_residual); N = 0 is a no-op.
 */
int keops_gauss_cg(const float *x, const float *b, int64_t N, int32_t D, int32_t E, float sigma, float lambda,
                   float rtol, int32_t max_iter, float *out, int32_t *iters, float *rel_residual, void *stream);

/*
 * K-min reduction with indices ([KO-GPU] §2 argmin / argKmin; [README] ArgMin,
 * K-min reductions): for each row i, the K smallest squared distances
 * |x_i - y_j|^2, ascending, and their indices j; equal distances are ordered
 * by smaller j first.  K = 1 is ArgMin.
 * The argument list follows the other reductions, (x, y, b, ..., sigma, out,
 * stream): b and sigma do not enter a nearest-neighbour search, are never read
 * and are not validated (b may be NULL, sigma any value).
 * out_d: [M, K] fp32; out_idx: [M, K] int64, 8-byte aligned.
 * Requires 1 <= K <= N < 2^31.
 */
int keops_kmin(const float *x, const float *y, const float *b,
               int64_t M, int64_t N, int32_t D, int32_t K, float sigma,
               float *out_d, int64_t *out_idx, void *stream);

/* Human-readable name of a status code (static storage). */
const char *keops_status_string(int status);

/*
 * Process-wide tuning and test switches (0 = automatic for each).  They change
 * how the work is scheduled, never what is computed beyond fp32 rounding:
 *   KEOPS_OPT_SPLIT_J   -- force this many j-splits (pass 1 partials + pass 2)
 *   KEOPS_OPT_FORM      -- 1 = use the direct distance form everywhere (the
 *                          expanded form is otherwise used wherever its range
 *                          condition holds)
 *   KEOPS_OPT_ROWS      -- 1 = one row per lane, 2 = the wide variant (several
 *                          rows per lane, for large M), 3 = the few-rows layout
 *                          of the sum, LogSumExp, gradient with respect to x
 *                          and K-min (j per lane, rows in LDS or registers;
 *                          chosen automatically for M <= 64 at D <= 8)
 *   KEOPS_OPT_WG_TARGET -- work-groups per CU the automatic j-split aims for
 *                          (1..4096; ignored when KEOPS_OPT_SPLIT_J is set)
 *   KEOPS_OPT_MFMA      -- 1 = the Gaussian sum and K-min never use the
 *                          matrix cores (the VALU expanded form runs at every
 *                          D; automatically they are used for D >= 32);
 *                          2 = the K-min prefilter at D >= 32 takes the fp32
 *                          MFMA form instead of the split-bf16 one (the same
 *                          results; the sum is unaffected)
 *   KEOPS_OPT_WS_CACHE  -- 2 = no workspace cache: every call allocates and
 *                          frees its workspace in stream order
 *                          (hipMallocAsync / hipFreeAsync); setting it also
 *                          frees the cached buffers no call holds
 *   KEOPS_OPT_FAIL_ALLOC -- test switch: 1 = every workspace allocation fails,
 *                          so that a call needing workspace returns
 *                          KEOPS_ERR_ALLOC with nothing enqueued
 * Returns KEOPS_OK, or KEOPS_ERR_INVALID_ARG for an unknown option or value.
 */
#define KEOPS_OPT_SPLIT_J 1
#define KEOPS_OPT_FORM 2
#define KEOPS_OPT_ROWS 3
#define KEOPS_OPT_PROFILE 4   /* 1 = record HIP events around each pass-1 launch */
#define KEOPS_OPT_WG_TARGET 5
#define KEOPS_OPT_MFMA 6
#define KEOPS_OPT_WS_CACHE 7
#define KEOPS_OPT_FAIL_ALLOC 8
int keops_set_option(int option, int64_t value);

/*
 * Duration of the pass-1 (pair-evaluation) kernels, for benchmarks.  While
 * KEOPS_OPT_PROFILE is 1, every call records a HIP event pair around its
 * pass-1 launch on the call's stream (at most 4096 pairs are kept).  This
 * waits for the recorded events, returns the summed duration in milliseconds
 * and the number of launches since the previous read, and forgets them.
 * total_ms and launches must be valid host pointers.
 */
int keops_profile_read(double *total_ms, int64_t *launches);

/* Library version as 10000*major + 100*minor + patch. */
int keops_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KEOPS_MI355X_H */
