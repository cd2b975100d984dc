// Drives the C ABI's host-side argument validation -- every rule of the header,
// block-sparse range arrays included -- in a sanitizer build of the API source, on a
// host without a GPU: every call below either fails validation before any HIP call
// or reaches the first HIP call, which fails without a device.  Device pointers are
// stand-in addresses that validation never dereferences; host arrays (the ranges) are
// allocated at exactly their documented sizes.  Test infrastructure: built and run by
// tests/test_sanitizers.py.
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "keops_mi355x.h"

namespace {

int fails = 0;
void expect(bool ok, const char *what, int line) {
  if (!ok) {
    std::fprintf(stderr, "line %d: %s\n", line, what);
    ++fails;
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)

float *dev(uintptr_t a) { return reinterpret_cast<float *>(a); }
const int kHip = KEOPS_ERR_HIP;   // the first HIP call fails on a host without a GPU

}  // namespace

int main() {
  // The stand-in device addresses below must never reach a kernel: on a host with a
  // GPU the calls that pass validation would launch.  Refuse to run there.
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0) {
    std::printf("skipped: a GPU is visible\n");
    return 77;
  }
  float *X = dev(0x10000), *Y = dev(0x20000000), *B = dev(0x40000000), *O = dev(0x60000000);
  // ---- dense reductions: every validation rule
  EXPECT(keops_gauss_sum(nullptr, nullptr, nullptr, -1, 0, 3, 1, 1.0f, nullptr, nullptr) == KEOPS_ERR_INVALID_ARG);
  EXPECT(keops_gauss_sum(nullptr, nullptr, nullptr, 0, -1, 3, 1, 1.0f, nullptr, nullptr) == KEOPS_ERR_INVALID_ARG);
  EXPECT(keops_gauss_sum(X, Y, B, 5, 7, 0, 1, 1.0f, O, nullptr) == KEOPS_ERR_INVALID_ARG);
  EXPECT(keops_gauss_lse(X, Y, B, 5, 7, 3, 0, 1.0f, O, nullptr) == KEOPS_ERR_INVALID_ARG);
  EXPECT(keops_gauss_lse(X, Y, B, 5, 7, 3, 1, -1.0f, O, nullptr) == KEOPS_ERR_INVALID_ARG);
  EXPECT(keops_gauss_sum(X, Y, B, 5, 7, 3, 1, 1.0f / 0.0f, O, nullptr) == KEOPS_ERR_INVALID_ARG);
  EXPECT(keops_gauss_sum(nullptr, Y, B, 5, 7, 3, 1, 1.0f, O, nullptr) == KEOPS_ERR_INVALID_ARG);
  EXPECT(keops_gauss_sum(X, Y, B, 5, 7, 3, 1, 1.0f, X, nullptr) == KEOPS_ERR_INVALID_ARG);      // overlap
  EXPECT(keops_gauss_sum(dev(0x10002), Y, B, 5, 7, 3, 1, 1.0f, O, nullptr) == KEOPS_ERR_INVALID_ARG);
  EXPECT(keops_gauss_sum(X, Y, B, 0, 0, 9, 1, 1.0f, O, nullptr) == KEOPS_ERR_UNSUPPORTED);
  EXPECT(keops_gauss_sum(X, Y, B, 0, 7, 3, 1, 1.0f, O, nullptr) == KEOPS_OK);                // M = 0
  EXPECT(keops_gauss_sum(X, Y, B, 5, 7, 3, 1, 1.0f, O, nullptr) == kHip);
  EXPECT(keops_gauss_sum_noalloc(X, Y, B, 5, 7, 50, 1, 1.0f, O, nullptr) == kHip);
  EXPECT(keops_gauss_sum_noalloc(dev(1ull << 40), dev(1ull << 48), dev(1ull << 48), int64_t(1) << 36, 10, 50, 1,
                                 1.0f, dev(1ull << 52), nullptr) == KEOPS_ERR_SCRATCH);
  EXPECT(keops_gauss_grad_x(X, Y, B, nullptr, 5, 7, 3, 1, 1.0f, O, nullptr) == KEOPS_ERR_INVALID_ARG);
  EXPECT(keops_gauss_grad_y(X, Y, nullptr, B, 5, 7, 3, 1, 1.0f, O, nullptr) == KEOPS_ERR_INVALID_ARG);
  EXPECT(keops_gauss_grad_b(X, Y, nullptr, 5, 7, 3, 1, 1.0f, O, nullptr) == KEOPS_ERR_INVALID_ARG);
  EXPECT(keops_gauss_max(X, Y, B, 5, 7, 3, 1, 1.0f, O, nullptr, nullptr) == KEOPS_ERR_INVALID_ARG);
  EXPECT(keops_gauss_min(X, Y, B, 5, 7, 3, 1, 1.0f, O, reinterpret_cast<int64_t *>(0x70000004), nullptr) ==
         KEOPS_ERR_INVALID_ARG);
  EXPECT(keops_laplace_sum(X, Y, B, 5, 7, 99, 1, 1.0f, O, nullptr) == KEOPS_ERR_UNSUPPORTED);
  // ---- K-min
  int64_t *I = reinterpret_cast<int64_t *>(0x70000000);
  EXPECT(keops_kmin(X, Y, nullptr, 5, 7, 3, 0, 1.0f, O, I, nullptr) == KEOPS_ERR_INVALID_ARG);
  EXPECT(keops_kmin(X, Y, nullptr, 5, 7, 3, 8, 1.0f, O, I, nullptr) == KEOPS_ERR_INVALID_ARG);    // K > N
  EXPECT(keops_kmin(X, Y, nullptr, 5, 100, 3, 17, 1.0f, O, I, nullptr) == KEOPS_ERR_UNSUPPORTED);
  EXPECT(keops_kmin(X, Y, nullptr, 5, 7, 3, 2, 0.0f / 0.0f, O, I, nullptr) == kHip);           // b, sigma unread
  // ---- CG
  int32_t it = 0;
  float res[4] = {0, 0, 0, 0};
  EXPECT(keops_gauss_cg(X, B, 10, 3, 1, 1.0f, -1.0f, 1e-5f, 10, O, &it, res, nullptr) == KEOPS_ERR_INVALID_ARG);
  EXPECT(keops_gauss_cg(X, B, 10, 3, 5, 1.0f, 1.0f, 1e-5f, 10, O, &it, res, nullptr) == KEOPS_ERR_UNSUPPORTED);
  EXPECT(keops_gauss_cg(nullptr, nullptr, 0, 3, 2, 1.0f, 0.0f, 1e-5f, 10, nullptr, &it, res, nullptr) == KEOPS_OK);
  // ---- block-sparse ranges: random valid and invalid host arrays of exact sizes
  std::mt19937_64 rng(7);
  int valid = 0, invalid = 0;
  for (int rep = 0; rep < 400; ++rep) {
    const int64_t M = 1 + rng() % 300, N = 1 + rng() % 300;
    const int64_t nri = rng() % 6, nrj = rng() % 8;
    std::vector<int64_t> ri(2 * nri), si(nri), rj(2 * nrj);
    int64_t lo = 0;
    for (int64_t c = 0; c < nri; ++c) {         // disjoint ascending row ranges
      const int64_t a = lo + (int64_t)(rng() % 20), e = a + (int64_t)(rng() % 60);
      ri[2 * c] = a;
      ri[2 * c + 1] = e;
      lo = e;
      si[c] = nrj ? (int64_t)(rng() % (nrj + 1)) : 0;
    }
    for (int64_t c = 1; c < nri; ++c) si[c] = si[c] < si[c - 1] ? si[c - 1] : si[c];   // non-decreasing
    for (int64_t k = 0; k < nrj; ++k) {
      const int64_t a = (int64_t)(rng() % (N + 1)), e = a + (int64_t)(rng() % (N - a + 1));
      rj[2 * k] = a;
      rj[2 * k + 1] = e;
    }
    // a mutation in one of four reps: out of range, reversed, overlapping or decreasing
    const int mut = rng() % 8;
    if (mut == 0 && nri) ri[2 * nri - 1] = M + 5;
    if (mut == 1 && nrj) { rj[0] = 3; rj[1] = 2; }
    if (mut == 2 && nri > 1) ri[2] = ri[1] > 0 ? ri[1] - 1 : ri[2];
    if (mut == 3 && nri > 1) si[0] = si[nri - 1] + 1;
    const int rc = keops_gauss_sum_ranges(X, Y, B, M, N, 3, 1, 1.0f, nri ? ri.data() : nullptr, nri,
                                          nri ? si.data() : nullptr, nrj ? rj.data() : nullptr, nrj, O, nullptr);
    EXPECT(rc == KEOPS_ERR_INVALID_ARG || rc == kHip);
    (rc == KEOPS_ERR_INVALID_ARG ? invalid : valid) += 1;
    const int rl = keops_gauss_lse_ranges(X, Y, B, M, N, 3, 2, 1.0f, nri ? ri.data() : nullptr, nri,
                                          nri ? si.data() : nullptr, nrj ? rj.data() : nullptr, nrj, O, nullptr);
    EXPECT(rl == rc);
  }
  EXPECT(valid > 50 && invalid > 20);
  // ---- options and status strings
  EXPECT(keops_set_option(99, 1) == KEOPS_ERR_INVALID_ARG);
  EXPECT(keops_set_option(KEOPS_OPT_WS_CACHE, 3) == KEOPS_ERR_INVALID_ARG);
  for (int s = -6; s <= 0; ++s) EXPECT(keops_status_string(s) != nullptr);
  double ms = 0;
  int64_t n = 0;
  EXPECT(keops_profile_read(&ms, &n) == KEOPS_OK && n == 0);
  if (fails) return 1;
  std::printf("ABI host sanitizer driver: ok (%d valid, %d invalid range sets)\n", valid, invalid);
  return 0;
}
