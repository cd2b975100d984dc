/*
 * keops_oracle.c -- the ORACLE: a plain, slow, double-precision CPU
 * implementation of the Gaussian map-reductions and their gradients.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  The GPU library shares
 * no code, header, table or helper with it, and neither calls the other.
 *
 * Every function is the textbook definition written out, in double precision,
 * with inputs given as the same fp32 arrays the GPU receives (each element is
 * widened to double exactly).  There is no blocking, no fusion and no
 * reordering: one output row at a time, a sequential loop over j, plain
 * summation.  Rows are independent, so an OpenMP loop over rows changes no
 * row's arithmetic.
 *
 * Sources (web pages about the KeOps library):
 *  [KO-GPU]  "Kernel Operations on the GPU, with Autodiff, without Memory
 *            Overflows" (paper summary page), §1 "Target operation",
 *            §2 "Generic reduction framework", "Performance and
 *            differentiation".
 *  [README]  KeOps README (PyTorch example: squared distances D_ij, Gaussian
 *            K_ij = exp(-D_ij), reductions .sum(), .logsumexp(), .argmin(),
 *            and autograd of (a**2).sum()); feature list "Sum, LogSumExp,
 *            Min, Max but also ArgMin, ArgMax or K-min reductions".
 *
 * Conventions (readings where the pages leave the step open):
 *  - Gaussian kernel with deviation sigma:  k(x,y) = exp(-|x-y|^2 / sigma^2).
 *    sigma = 1 gives the README's exp(-D_ij).
 *  - LogSumExp of row i, column e:  log sum_j exp(-|x_i-y_j|^2/sigma^2 + b_je).
 *  - grad_x is the vector-Jacobian product of a = sum-reduction with a given
 *    cotangent g[M,E] = dL/da (the README differentiates (a**2).sum(), i.e.
 *    g = 2a).
 *  - grad_y and grad_b are the vector-Jacobian products of the same sum in y
 *    and b (reductions over i, one output per point y_j).
 *  - K-min: the K smallest squared distances of row i with their indices, in
 *    ascending (distance, index) lexicographic order.
 *
 * All arrays are dense row-major.  `rows` selects which output rows to
 * compute (NULL = rows 0..nrows-1); outputs are written for the selected rows
 * in order.  Return value: 0 on success, -1 on an invalid argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* |x_i - y_j|^2 in double: [README] D_ij = ((x_i - y_j)**2).sum(dim=2). */
static double sq_dist(const float *xi, const float *yj, int D) {
    double s = 0.0;
    for (int d = 0; d < D; ++d) {
        double t = (double)xi[d] - (double)yj[d];
        s += t * t;
    }
    return s;
}

static int check_common(int64_t M, int64_t N, int D, int64_t nrows, const int64_t *rows) {
    if (M < 0 || N < 0 || D < 1 || nrows < 0) return -1;
    if (!rows && nrows > M) return -1;
    if (rows)
        for (int64_t r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= M) return -1;
    return 0;
}

/*
 * Gaussian kernel sum  a_ie = sum_j exp(-|x_i - y_j|^2 / sigma^2) * b_je
 * ([KO-GPU] §1 "Target operation": a_i = sum_j k(x_i, y_j) b_j with a Gaussian
 * k of deviation sigma > 0; [README] a_i = K_ij.sum(dim=1)).
 * Also returns the normaliser  norm_ie = sum_j |K_ij * b_je|  used by the
 * per-row relative tolerance.
 */
int oracle_gauss_sum(const float *x, const float *y, const float *b,
                     int64_t M, int64_t N, int D, int E, double sigma,
                     const int64_t *rows, int64_t nrows,
                     double *out, double *norm) {
    if (check_common(M, N, D, nrows, rows) || E < 1 || !(sigma > 0.0)) return -1;
    const double inv_s2 = 1.0 / (sigma * sigma);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = rows ? rows[r] : r;
        /* the row's accumulators live on the thread's stack: threads writing
         * neighbouring rows of `out` would otherwise share its cache lines */
        double o[E], nacc[E];
        double *nm = norm ? nacc : NULL;
        for (int e = 0; e < E; ++e) { o[e] = 0.0; if (nm) nm[e] = 0.0; }
        for (int64_t j = 0; j < N; ++j) {
            const double k = exp(-sq_dist(x + i * D, y + j * D, D) * inv_s2);
            for (int e = 0; e < E; ++e) {
                const double t = k * (double)b[j * E + e];
                o[e] += t;
                if (nm) nm[e] += fabs(t);
            }
        }
        for (int e = 0; e < E; ++e) { out[r * E + e] = o[e]; if (norm) norm[r * E + e] = nacc[e]; }
    }
    return 0;
}

/*
 * LogSumExp reduction  l_ie = log sum_j exp(v_ije),  v_ije = -|x_i-y_j|^2/sigma^2 + b_je
 * ([KO-GPU] §2 reductions "sum, max, argmin, and log-sum-exp"; [README]
 * .logsumexp()).  Textbook two-pass form: m = max_j v, then
 * l = m + log sum_j exp(v - m).  N = 0 gives -inf.
 */
int oracle_gauss_lse(const float *x, const float *y, const float *b,
                     int64_t M, int64_t N, int D, int E, double sigma,
                     const int64_t *rows, int64_t nrows, double *out) {
    if (check_common(M, N, D, nrows, rows) || E < 1 || !(sigma > 0.0)) return -1;
    const double inv_s2 = 1.0 / (sigma * sigma);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = rows ? rows[r] : r;
        for (int e = 0; e < E; ++e) {
            double m = -INFINITY;
            for (int64_t j = 0; j < N; ++j) {
                const double v = -sq_dist(x + i * D, y + j * D, D) * inv_s2 + (double)b[j * E + e];
                if (v > m) m = v;
            }
            double s = 0.0;
            if (m > -INFINITY) {
                for (int64_t j = 0; j < N; ++j) {
                    const double v = -sq_dist(x + i * D, y + j * D, D) * inv_s2 + (double)b[j * E + e];
                    s += exp(v - m);
                }
                out[r * E + e] = m + log(s);
            } else {
                out[r * E + e] = -INFINITY;
            }
        }
    }
    return 0;
}

/*
 * Gradient of L with respect to x, given the cotangent g = dL/da of the sum
 * reduction ([KO-GPU] §2 "Performance and differentiation": autodiff through
 * torch.autograd; [README] torch.autograd.grad((a_i ** 2).sum(), [x])).
 * Differentiating a_ie = sum_j exp(-|x_i-y_j|^2/sigma^2) b_je with respect to
 * x_id gives
 *   G_id = sum_j (-2/sigma^2) K_ij <g_i, b_j> (x_id - y_jd).
 * Also returns  nu_id = sum_j |(2/sigma^2) K_ij <g_i, b_j> (x_id - y_jd)|.
 */
int oracle_gauss_grad_x(const float *x, const float *y, const float *b, const float *g,
                        int64_t M, int64_t N, int D, int E, double sigma,
                        const int64_t *rows, int64_t nrows,
                        double *out, double *nu) {
    if (check_common(M, N, D, nrows, rows) || E < 1 || !(sigma > 0.0)) return -1;
    const double inv_s2 = 1.0 / (sigma * sigma);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = rows ? rows[r] : r;
        double o[D], nacc[D];               /* stack accumulators, as in the sum */
        double *n = nu ? nacc : NULL;
        for (int d = 0; d < D; ++d) { o[d] = 0.0; if (n) n[d] = 0.0; }
        for (int64_t j = 0; j < N; ++j) {
            const double k = exp(-sq_dist(x + i * D, y + j * D, D) * inv_s2);
            double gb = 0.0;
            for (int e = 0; e < E; ++e) gb += (double)g[i * E + e] * (double)b[j * E + e];
            for (int d = 0; d < D; ++d) {
                const double t = -2.0 * inv_s2 * k * gb * ((double)x[i * D + d] - (double)y[j * D + d]);
                o[d] += t;
                if (n) n[d] += fabs(t);
            }
        }
        for (int d = 0; d < D; ++d) { out[r * D + d] = o[d]; if (nu) nu[r * D + d] = nacc[d]; }
    }
    return 0;
}

/*
 * Gradient of L = sum_ie g_ie a_ie with respect to y (the transposed
 * reduction: one output per point y_j, summed over the rows i).  [KO-GPU] §2
 * "Performance and differentiation": the reductions are differentiable with
 * respect to every input variable; differentiating
 * a_ie = sum_j exp(-|x_i - y_j|^2/sigma^2) b_je in y_jd gives
 *   Gy_jd = sum_i (2/sigma^2) K_ij <g_i, b_j> (x_id - y_jd).
 * `cols` selects which points j to compute (NULL = 0..ncols-1).  Also returns
 * nu_jd = sum_i |(2/sigma^2) K_ij <g_i, b_j> (x_id - y_jd)|.
 */
int oracle_gauss_grad_y(const float *x, const float *y, const float *b, const float *g,
                        int64_t M, int64_t N, int D, int E, double sigma,
                        const int64_t *cols, int64_t ncols,
                        double *out, double *nu) {
    if (check_common(N, M, D, ncols, cols) || E < 1 || !(sigma > 0.0)) return -1;
    const double inv_s2 = 1.0 / (sigma * sigma);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t c = 0; c < ncols; ++c) {
        const int64_t j = cols ? cols[c] : c;
        double o[D], nacc[D];               /* stack accumulators, as in the sum */
        double *n = nu ? nacc : NULL;
        for (int d = 0; d < D; ++d) { o[d] = 0.0; if (n) n[d] = 0.0; }
        for (int64_t i = 0; i < M; ++i) {
            const double k = exp(-sq_dist(x + i * D, y + j * D, D) * inv_s2);
            double gb = 0.0;
            for (int e = 0; e < E; ++e) gb += (double)g[i * E + e] * (double)b[j * E + e];
            for (int d = 0; d < D; ++d) {
                const double t = 2.0 * inv_s2 * k * gb * ((double)x[i * D + d] - (double)y[j * D + d]);
                o[d] += t;
                if (n) n[d] += fabs(t);
            }
        }
        for (int d = 0; d < D; ++d) { out[c * D + d] = o[d]; if (nu) nu[c * D + d] = nacc[d]; }
    }
    return 0;
}

/*
 * Gradient of L = sum_ie g_ie a_ie with respect to b (same passage): a is
 * linear in b, so
 *   Gb_je = sum_i K_ij g_ie,
 * with nu_je = sum_i |K_ij g_ie|.  `cols` as for oracle_gauss_grad_y.
 */
int oracle_gauss_grad_b(const float *x, const float *y, const float *g,
                        int64_t M, int64_t N, int D, int E, double sigma,
                        const int64_t *cols, int64_t ncols,
                        double *out, double *nu) {
    if (check_common(N, M, D, ncols, cols) || E < 1 || !(sigma > 0.0)) return -1;
    const double inv_s2 = 1.0 / (sigma * sigma);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t c = 0; c < ncols; ++c) {
        const int64_t j = cols ? cols[c] : c;
        double o[E], nacc[E];               /* stack accumulators, as in the sum */
        double *n = nu ? nacc : NULL;
        for (int e = 0; e < E; ++e) { o[e] = 0.0; if (n) n[e] = 0.0; }
        for (int64_t i = 0; i < M; ++i) {
            const double k = exp(-sq_dist(x + i * D, y + j * D, D) * inv_s2);
            for (int e = 0; e < E; ++e) {
                const double t = k * (double)g[i * E + e];
                o[e] += t;
                if (n) n[e] += fabs(t);
            }
        }
        for (int e = 0; e < E; ++e) { out[c * E + e] = o[e]; if (nu) nu[c * E + e] = nacc[e]; }
    }
    return 0;
}

/*
 * K-min reduction with indices ([KO-GPU] §2 "argmin, and argKmin"; [README]
 * "ArgMin, ArgMax or K-min reductions").  For row i: the K smallest values of
 * delta_ij = |x_i - y_j|^2 (double), ordered by (delta, j) lexicographically,
 * ascending.  Kept as a sorted list of length K into which each j is inserted
 * when it precedes the current K-th entry.  Requires 1 <= K <= N.
 */
int oracle_kmin(const float *x, const float *y,
                int64_t M, int64_t N, int D, int K,
                const int64_t *rows, int64_t nrows,
                double *out_d, int64_t *out_idx) {
    if (check_common(M, N, D, nrows, rows) || K < 1 || (int64_t)K > N) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = rows ? rows[r] : r;
        double *bd = out_d + r * K;
        int64_t *bj = out_idx + r * K;
        int count = 0;
        for (int64_t j = 0; j < N; ++j) {
            const double dj = sq_dist(x + i * D, y + j * D, D);
            /* does (dj, j) precede the last kept entry? */
            if (count == K && !(dj < bd[K - 1] || (dj == bd[K - 1] && j < bj[K - 1]))) continue;
            int pos = (count < K) ? count : K - 1;
            while (pos > 0 && (dj < bd[pos - 1] || (dj == bd[pos - 1] && j < bj[pos - 1]))) {
                bd[pos] = bd[pos - 1];
                bj[pos] = bj[pos - 1];
                --pos;
            }
            bd[pos] = dj;
            bj[pos] = j;
            if (count < K) ++count;
        }
    }
    return 0;
}

/* delta(i, j) = |x_i - y_j|^2 in double for a list of (i, j) pairs, to judge
 * the GPU's K-min picks one by one. */
int oracle_sq_dist_pairs(const float *x, const float *y, int D,
                         const int64_t *ii, const int64_t *jj, int64_t npairs, double *out) {
    if (D < 1 || npairs < 0) return -1;
    for (int64_t p = 0; p < npairs; ++p) out[p] = sq_dist(x + ii[p] * D, y + jj[p] * D, D);
    return 0;
}

/*
 * The Gaussian kernel matrix itself, K[i*N + j] = exp(-|x_i - y_j|^2/sigma^2)
 * in double, for the dense linear solve that stands for the conjugate
 * gradient solver ([README] feature list: a conjugate gradient solver for
 * spline interpolation or kriging) on small inputs.
 */
int oracle_gauss_matrix(const float *x, const float *y, int64_t M, int64_t N, int D, double sigma,
                        double *out) {
    if (M < 0 || N < 0 || D < 1 || !(sigma > 0.0)) return -1;
    const double inv_s2 = 1.0 / (sigma * sigma);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) out[i * N + j] = exp(-sq_dist(x + i * D, y + j * D, D) * inv_s2);
    return 0;
}

/*
 * Block-sparse reductions ([KO-GPU] §3 "Applications": cluster-wise
 * block-sparsity for large kernel linear systems; §4: the block-sparse
 * truncation rule; [README] feature list: an interface for block-sparse
 * strategies).  The kept pairs are given as ranges: row range c covers rows
 * [ranges_i[2c], ranges_i[2c+1]) and meets the j ranges
 * [redranges_j[2k], redranges_j[2k+1]) for k from slices_i[c-1] (0 when c = 0)
 * up to slices_i[c] - 1.  The reductions are the definitions above restricted
 * to the kept pairs, j visited range by range in the listed order; a j listed
 * in two ranges of one row range counts twice.  Rows in no row range get the
 * empty reduction (0 for the sum, -inf for LogSumExp).  Row ranges must not
 * overlap (-1 otherwise), and every range must lie inside [0, M) or [0, N).
 */
static int check_ranges(int64_t M, int64_t N, const int64_t *ranges_i, int64_t nri, const int64_t *slices_i,
                        const int64_t *redranges_j, int64_t nrj) {
    if (M < 0 || N < 0 || nri < 0 || nrj < 0) return -1;
    if (nri > 0 && (!ranges_i || !slices_i)) return -1;
    if (nrj > 0 && !redranges_j) return -1;
    int64_t prev = 0;
    for (int64_t c = 0; c < nri; ++c) {
        const int64_t lo = ranges_i[2 * c], hi = ranges_i[2 * c + 1];
        if (lo < 0 || lo > hi || hi > M) return -1;
        if (slices_i[c] < prev || slices_i[c] > nrj) return -1;
        prev = slices_i[c];
        for (int64_t d = 0; d < c; ++d)   /* row ranges pairwise disjoint */
            if (lo < ranges_i[2 * d + 1] && ranges_i[2 * d] < hi) return -1;
    }
    for (int64_t k = 0; k < nrj; ++k) {
        const int64_t lo = redranges_j[2 * k], hi = redranges_j[2 * k + 1];
        if (lo < 0 || lo > hi || hi > N) return -1;
    }
    return 0;
}

int oracle_gauss_sum_ranges(const float *x, const float *y, const float *b,
                            int64_t M, int64_t N, int D, int E, double sigma,
                            const int64_t *ranges_i, int64_t nri, const int64_t *slices_i,
                            const int64_t *redranges_j, int64_t nrj,
                            double *out, double *norm) {
    if (D < 1 || E < 1 || !(sigma > 0.0) || check_ranges(M, N, ranges_i, nri, slices_i, redranges_j, nrj))
        return -1;
    const double inv_s2 = 1.0 / (sigma * sigma);
    for (int64_t q = 0; q < M * E; ++q) { out[q] = 0.0; if (norm) norm[q] = 0.0; }
    for (int64_t c = 0; c < nri; ++c) {
        const int64_t k0 = c == 0 ? 0 : slices_i[c - 1], k1 = slices_i[c];
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t i = ranges_i[2 * c]; i < ranges_i[2 * c + 1]; ++i) {
            double o[E], nacc[E];           /* stack accumulators, as in the sum */
            double *nm = norm ? nacc : NULL;
            for (int e = 0; e < E; ++e) { o[e] = 0.0; nacc[e] = 0.0; }
            for (int64_t k = k0; k < k1; ++k)
                for (int64_t j = redranges_j[2 * k]; j < redranges_j[2 * k + 1]; ++j) {
                    const double kv = exp(-sq_dist(x + i * D, y + j * D, D) * inv_s2);
                    for (int e = 0; e < E; ++e) {
                        const double t = kv * (double)b[j * E + e];
                        o[e] += t;
                        if (nm) nm[e] += fabs(t);
                    }
                }
            for (int e = 0; e < E; ++e) { out[i * E + e] = o[e]; if (norm) norm[i * E + e] = nacc[e]; }
        }
    }
    return 0;
}

int oracle_gauss_lse_ranges(const float *x, const float *y, const float *b,
                            int64_t M, int64_t N, int D, int E, double sigma,
                            const int64_t *ranges_i, int64_t nri, const int64_t *slices_i,
                            const int64_t *redranges_j, int64_t nrj, double *out) {
    if (D < 1 || E < 1 || !(sigma > 0.0) || check_ranges(M, N, ranges_i, nri, slices_i, redranges_j, nrj))
        return -1;
    const double inv_s2 = 1.0 / (sigma * sigma);
    for (int64_t q = 0; q < M * E; ++q) out[q] = -INFINITY;
    for (int64_t c = 0; c < nri; ++c) {
        const int64_t k0 = c == 0 ? 0 : slices_i[c - 1], k1 = slices_i[c];
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t i = ranges_i[2 * c]; i < ranges_i[2 * c + 1]; ++i) {
            for (int e = 0; e < E; ++e) {
                double m = -INFINITY;
                for (int64_t k = k0; k < k1; ++k)
                    for (int64_t j = redranges_j[2 * k]; j < redranges_j[2 * k + 1]; ++j) {
                        const double v = -sq_dist(x + i * D, y + j * D, D) * inv_s2 + (double)b[j * E + e];
                        if (v > m) m = v;
                    }
                if (!(m > -INFINITY)) continue;
                double s = 0.0;
                for (int64_t k = k0; k < k1; ++k)
                    for (int64_t j = redranges_j[2 * k]; j < redranges_j[2 * k + 1]; ++j)
                        s += exp(-sq_dist(x + i * D, y + j * D, D) * inv_s2 + (double)b[j * E + e] - m);
                out[i * E + e] = m + log(s);
            }
        }
    }
    return 0;
}

/*
 * Max / ArgMax reduction of the kernel product ([KO-GPU] §2 reductions list
 * "sum, max, argmin, and log-sum-exp"; [README] feature list "Sum, LogSumExp,
 * Min, Max but also ArgMin, ArgMax").  For row i and column e:
 *   out_ie = max_j  sgn * K_ij b_je,  idx_ie = the smallest j reaching it,
 * so sgn = +1 is Max / ArgMax of K b and sgn = -1 gives -(Min / ArgMin of
 * K b).  N = 0 gives -inf and index -1.  The comparison is in double.
 */
int oracle_gauss_max(const float *x, const float *y, const float *b,
                     int64_t M, int64_t N, int D, int E, double sigma, int sgn,
                     const int64_t *rows, int64_t nrows, double *out, int64_t *idx) {
    if (check_common(M, N, D, nrows, rows) || E < 1 || !(sigma > 0.0) || (sgn != 1 && sgn != -1)) return -1;
    const double inv_s2 = 1.0 / (sigma * sigma);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = rows ? rows[r] : r;
        for (int e = 0; e < E; ++e) { out[r * E + e] = -INFINITY; idx[r * E + e] = -1; }
        for (int64_t j = 0; j < N; ++j) {
            const double k = exp(-sq_dist(x + i * D, y + j * D, D) * inv_s2);
            for (int e = 0; e < E; ++e) {
                const double v = (double)sgn * k * (double)b[j * E + e];
                if (v > out[r * E + e]) { out[r * E + e] = v; idx[r * E + e] = j; }
            }
        }
    }
    return 0;
}

/*
 * Laplacian kernel sum ([README] feature list: a wide range of formulas; the
 * pages name Gaussian and other kernels for kernel methods):
 *   a_ie = sum_j exp(-|x_i - y_j| / sigma) b_je,  |.| the Euclidean norm,
 * with norm_ie = sum_j |exp(-|x_i - y_j|/sigma) b_je|.
 */
int oracle_laplace_sum(const float *x, const float *y, const float *b,
                       int64_t M, int64_t N, int D, int E, double sigma,
                       const int64_t *rows, int64_t nrows, double *out, double *norm) {
    if (check_common(M, N, D, nrows, rows) || E < 1 || !(sigma > 0.0)) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = rows ? rows[r] : r;
        double o[E], nacc[E];               /* stack accumulators, as in the sum */
        for (int e = 0; e < E; ++e) { o[e] = 0.0; nacc[e] = 0.0; }
        for (int64_t j = 0; j < N; ++j) {
            const double k = exp(-sqrt(sq_dist(x + i * D, y + j * D, D)) / sigma);
            for (int e = 0; e < E; ++e) {
                const double t = k * (double)b[j * E + e];
                o[e] += t;
                nacc[e] += fabs(t);
            }
        }
        for (int e = 0; e < E; ++e) { out[r * E + e] = o[e]; if (norm) norm[r * E + e] = nacc[e]; }
    }
    return 0;
}

