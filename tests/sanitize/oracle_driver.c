/* Runs every oracle routine on small seeded inputs in buffers of exactly the sizes
 * the routines are documented to touch, so that an address/undefined-behaviour
 * sanitizer build reports any out-of-bounds access, overflow or uninitialised
 * read.  Test infrastructure: built and run by tests/test_sanitizers.py. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_gauss_sum(const float *, const float *, const float *, int64_t, int64_t, int, int, double,
                     const int64_t *, int64_t, double *, double *);
int oracle_gauss_lse(const float *, const float *, const float *, int64_t, int64_t, int, int, double,
                     const int64_t *, int64_t, double *);
int oracle_gauss_grad_x(const float *, const float *, const float *, const float *, int64_t, int64_t, int, int,
                        double, const int64_t *, int64_t, double *, double *);
int oracle_gauss_grad_y(const float *, const float *, const float *, const float *, int64_t, int64_t, int, int,
                        double, const int64_t *, int64_t, double *, double *);
int oracle_gauss_grad_b(const float *, const float *, const float *, int64_t, int64_t, int, int, double,
                        const int64_t *, int64_t, double *, double *);
int oracle_kmin(const float *, const float *, int64_t, int64_t, int, int, const int64_t *, int64_t, double *,
                int64_t *);
int oracle_sq_dist_pairs(const float *, const float *, int, const int64_t *, const int64_t *, int64_t, double *);
int oracle_gauss_matrix(const float *, const float *, int64_t, int64_t, int, double, double *);
int oracle_gauss_sum_ranges(const float *, const float *, const float *, int64_t, int64_t, int, int, double,
                            const int64_t *, int64_t, const int64_t *, const int64_t *, int64_t, double *, double *);
int oracle_gauss_lse_ranges(const float *, const float *, const float *, int64_t, int64_t, int, int, double,
                            const int64_t *, int64_t, const int64_t *, const int64_t *, int64_t, double *);
int oracle_gauss_max(const float *, const float *, const float *, int64_t, int64_t, int, int, double, int,
                     const int64_t *, int64_t, double *, int64_t *);
int oracle_laplace_sum(const float *, const float *, const float *, int64_t, int64_t, int, int, double,
                       const int64_t *, int64_t, double *, double *);

static uint64_t state = 88172645463325252ull;
static float rnd(void) {            /* xorshift64, uniform in [-1, 1) */
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return (float)((double)(state >> 11) / 9007199254740992.0 * 2.0 - 1.0);
}
static float *fbuf(int64_t n) {
  float *p = (float *)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
  for (int64_t k = 0; k < n; ++k) p[k] = rnd();
  return p;
}
static double *dbuf(int64_t n) { return (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double)); }
static int64_t *ibuf(int64_t n) { return (int64_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(int64_t)); }

static int fails = 0;
static void expect(int rc, const char *what) {
  if (rc != 0) {
    fprintf(stderr, "%s returned %d\n", what, rc);
    ++fails;
  }
}

static void one_shape(int64_t M, int64_t N, int D, int E, int K) {
  float *x = fbuf(M * D), *y = fbuf(N * D), *b = fbuf(N * E), *g = fbuf(M * E);
  /* a row subset: every other row, backwards */
  const int64_t nr = (M + 1) / 2;
  int64_t *rows = ibuf(nr);
  for (int64_t k = 0; k < nr; ++k) rows[k] = M - 1 - 2 * k;
  for (int sub = 0; sub < 2; ++sub) {
    const int64_t *r = sub ? rows : NULL;
    const int64_t n = sub ? nr : M;
    double *o1 = dbuf(n * E), *o2 = dbuf(n * E), *od = dbuf(n * D), *nd = dbuf(n * D);
    expect(oracle_gauss_sum(x, y, b, M, N, D, E, 0.7, r, n, o1, o2), "gauss_sum");
    expect(oracle_gauss_lse(x, y, b, M, N, D, E, 0.7, r, n, o1), "gauss_lse");
    expect(oracle_gauss_grad_x(x, y, b, g, M, N, D, E, 0.7, r, n, od, nd), "gauss_grad_x");
    expect(oracle_laplace_sum(x, y, b, M, N, D, E, 0.7, r, n, o1, o2), "laplace_sum");
    int64_t *ix = ibuf(n * E);
    expect(oracle_gauss_max(x, y, b, M, N, D, E, 0.7, 1, r, n, o1, ix), "gauss_max");
    expect(oracle_gauss_max(x, y, b, M, N, D, E, 0.7, -1, r, n, o1, ix), "gauss_min");
    free(ix);
    if (K >= 1 && K <= N) {
      double *kd = dbuf(n * K);
      int64_t *ki = ibuf(n * K);
      expect(oracle_kmin(x, y, M, N, D, K, r, n, kd, ki), "kmin");
      free(kd);
      free(ki);
    }
    free(o1); free(o2); free(od); free(nd);
  }
  /* the transposed gradients reduce over i for a subset of j */
  const int64_t nc = (N + 2) / 3;
  int64_t *cols = ibuf(nc);
  for (int64_t k = 0; k < nc; ++k) cols[k] = 3 * k;
  double *gy = dbuf(nc * D), *ny = dbuf(nc * D), *gb = dbuf(nc * E), *nb = dbuf(nc * E);
  expect(oracle_gauss_grad_y(x, y, b, g, M, N, D, E, 0.7, cols, nc, gy, ny), "gauss_grad_y");
  expect(oracle_gauss_grad_b(x, y, g, M, N, D, E, 0.7, cols, nc, gb, nb), "gauss_grad_b");
  free(cols); free(gy); free(ny); free(gb); free(nb);
  if (M * N <= 4096) {
    double *km = dbuf(M * N);
    expect(oracle_gauss_matrix(x, y, M, N, D, 0.7, km), "gauss_matrix");
    free(km);
  }
  if (M > 0 && N > 0) {
    int64_t ii[5], jj[5];
    double pd[5];
    for (int k = 0; k < 5; ++k) { ii[k] = (k * 7) % M; jj[k] = (k * 11) % N; }
    expect(oracle_sq_dist_pairs(x, y, D, ii, jj, 5, pd), "sq_dist_pairs");
    /* block-sparse: two row ranges, three j ranges (one repeated, one empty) */
    const int64_t ri[4] = {0, M / 2, M / 2, M};
    const int64_t si[2] = {2, 3};
    const int64_t rj[6] = {0, N / 3, N / 3, N, N / 2, N / 2};
    double *o1 = dbuf(M * E), *o2 = dbuf(M * E);
    expect(oracle_gauss_sum_ranges(x, y, b, M, N, D, E, 0.7, ri, 2, si, rj, 3, o1, o2), "gauss_sum_ranges");
    expect(oracle_gauss_lse_ranges(x, y, b, M, N, D, E, 0.7, ri, 2, si, rj, 3, o1), "gauss_lse_ranges");
    free(o1); free(o2);
  }
  free(x); free(y); free(b); free(g); free(rows);
}

int main(void) {
  one_shape(1, 1, 1, 1, 1);
  one_shape(7, 13, 3, 1, 5);
  one_shape(33, 65, 3, 2, 13);
  one_shape(20, 40, 8, 4, 16);
  one_shape(9, 17, 50, 1, 17);    /* K = N */
  one_shape(5, 0, 3, 1, 0);       /* N = 0 */
  one_shape(0, 4, 3, 1, 2);       /* M = 0 */
  if (fails) return 1;
  printf("oracle sanitizer driver: ok\n");
  return 0;
}
