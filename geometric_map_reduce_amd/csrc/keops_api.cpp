// keops_api.cpp -- the C ABI of include/keops_mi355x.h: argument validation,
// the launch plan (rows per lane, j-splits), stream-ordered workspace and
// kernel dispatch.  No HIP call is made before the arguments are validated,
// so argument errors never touch the device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <memory>
#include <mutex>
#include <vector>

#include "keops_mi355x.h"
#include "launch.h"

// Device scratch of keops_gauss_sum_noalloc (split-j partials and form flags): a
// fixed array in the library's code object, one copy per GPU, held until the process
// ends.  Host code never passes `scratch` itself to a kernel or a copy: on the host
// the name stands for a shadow, not a device address; the address of each GPU's copy
// comes from hipGetSymbolAddress (scratch_of_device below).
static constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace kmi {
namespace {

std::atomic<int64_t> g_opt_split{0}, g_opt_form{0}, g_opt_rows{0}, g_opt_profile{0}, g_opt_wg_target{0},
    g_opt_mfma{0}, g_opt_ws_cache{1}, g_opt_fail_alloc{0};

// ---- pass-1 timing (KEOPS_OPT_PROFILE)
struct EventPair { hipEvent_t start, stop; };
std::mutex g_prof_mu;
std::vector<EventPair> g_prof_events;
constexpr size_t kMaxProfiled = 4096;

// Records the start event when profiling is on; returns the pair index or -1.
int prof_begin(hipStream_t st) {
  if (g_opt_profile.load(std::memory_order_relaxed) != 1) return -1;
  // timing-only events: no system-scope fence (its cache write-back and invalidation
  // cost a few microseconds of GPU time per event, visible on small calls)
  EventPair e{};
  if (hipEventCreateWithFlags(&e.start, hipEventDisableSystemFence) != hipSuccess) return -1;
  if (hipEventCreateWithFlags(&e.stop, hipEventDisableSystemFence) != hipSuccess) {
    (void)hipEventDestroy(e.start);
    return -1;
  }
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (g_prof_events.size() >= kMaxProfiled) {
    (void)hipEventDestroy(e.start);
    (void)hipEventDestroy(e.stop);
    return -1;
  }
  (void)hipEventRecord(e.start, st);
  g_prof_events.push_back(e);
  return (int)g_prof_events.size() - 1;
}

void prof_end(int idx, hipStream_t st) {
  if (idx < 0) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if ((size_t)idx < g_prof_events.size()) (void)hipEventRecord(g_prof_events[idx].stop, st);
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];
std::once_flag g_pool_once[kMaxDevices];

// Compute units of the current device (cached).  Also raises the release
// threshold of the device's default memory pool once, so that stream-ordered
// workspace allocations are served from the pool instead of the driver.
int device_setup(int *cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KEOPS_ERR_HIP;
  int c = g_cu_count[dev].load(std::memory_order_relaxed);
  if (c <= 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
      return KEOPS_ERR_HIP;
    g_cu_count[dev].store(c, std::memory_order_relaxed);
  }
  std::call_once(g_pool_once[dev], [dev] {
    hipMemPool_t pool;
    if (hipDeviceGetDefaultMemPool(&pool, dev) == hipSuccess) {
      uint64_t thr = UINT64_MAX;
      (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &thr);
    }
  });
  *cus = c;
  return KEOPS_OK;
}

// Address of this device's copy of `scratch`, looked up once per device with that
// device current (each GPU holds its own copy at its own address).
std::mutex g_scratch_mu;
std::atomic<char *> g_scratch_ptr[kMaxDevices];

int scratch_of_device(char **ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KEOPS_ERR_HIP;
  char *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      void *q = nullptr;
      if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) {
        (void)hipGetLastError();
        return KEOPS_ERR_HIP;
      }
      p = (char *)q;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return KEOPS_OK;
}

// Workspace of one call: allocated stream-ordered (arena null), or carved from a
// fixed device buffer of `cap` bytes (the no-allocation entry point).
struct Arena {
  char *base;
  size_t cap;
};

// ---- workspace cache
// Each (device, stream, slot) keeps one grow-only device buffer, which the calls on
// that stream reuse in stream order: after the first call of a given size a call
// neither allocates nor waits on the host (a stream-ordered allocation and free per
// call made every small call wait for the GPU).  Growing or evicting an idle buffer
// frees it with hipFree, which waits for the device's pending work first.  A buffer
// held by another host thread's call on the same stream is never shared (the two
// calls' kernels could interleave): such a call allocates its own for the occasion.
// Slot 0: the reductions' split partials; slot 1: the CG solver's vectors (its
// products take slot 0 on the same stream).  KEOPS_OPT_WS_CACHE = 0 allocates per
// call instead and frees the idle cached buffers.
struct WsEntry {
  int dev;
  hipStream_t st;
  int slot;
  char *ptr;
  size_t cap;
  int busy;
  uint64_t tick;
};
std::mutex g_ws_mu;
std::vector<std::unique_ptr<WsEntry>> g_ws;
uint64_t g_ws_tick = 0;
constexpr size_t kWsMaxEntries = 32;

// Frees every cached buffer no call holds (caller holds g_ws_mu).
void ws_trim_locked() {
  for (size_t k = 0; k < g_ws.size();) {
    if (g_ws[k]->busy == 0) {
      int cur = 0;
      (void)hipGetDevice(&cur);
      (void)hipSetDevice(g_ws[k]->dev);
      (void)hipFree(g_ws[k]->ptr);
      (void)hipSetDevice(cur);
      g_ws.erase(g_ws.begin() + (ptrdiff_t)k);
    } else {
      ++k;
    }
  }
  (void)hipGetLastError();
}

class Workspace {
 public:
  Workspace() = default;
  Workspace(const Workspace &) = delete;
  Workspace &operator=(const Workspace &) = delete;
  ~Workspace() { release(); }

  // A device buffer of at least `bytes` for work enqueued on `st` (null for 0 bytes).
  // Returns KEOPS_OK or KEOPS_ERR_ALLOC (nothing enqueued).
  int acquire(hipStream_t st, int slot, size_t bytes) {
    release();
    if (bytes == 0) return KEOPS_OK;
    if (g_opt_fail_alloc.load(std::memory_order_relaxed) == 1) return KEOPS_ERR_ALLOC;
    bytes = (bytes + 255) / 256 * 256;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
      (void)hipGetLastError();
      return KEOPS_ERR_ALLOC;
    }
    if (g_opt_ws_cache.load(std::memory_order_relaxed) == 1) {
      std::lock_guard<std::mutex> lk(g_ws_mu);
      WsEntry *e = nullptr;
      for (auto &u : g_ws)
        if (u->dev == dev && u->st == st && u->slot == slot) { e = u.get(); break; }
      if (!e && g_ws.size() >= kWsMaxEntries) {
        // evict the least recently used idle buffer
        size_t lru = g_ws.size();
        for (size_t k = 0; k < g_ws.size(); ++k)
          if (g_ws[k]->busy == 0 && (lru == g_ws.size() || g_ws[k]->tick < g_ws[lru]->tick)) lru = k;
        if (lru < g_ws.size()) {
          (void)hipSetDevice(g_ws[lru]->dev);
          (void)hipFree(g_ws[lru]->ptr);
          (void)hipSetDevice(dev);
          g_ws.erase(g_ws.begin() + (ptrdiff_t)lru);
        }
      }
      if (!e && g_ws.size() < kWsMaxEntries) {
        g_ws.push_back(std::unique_ptr<WsEntry>(new WsEntry{dev, st, slot, nullptr, 0, 0, 0}));
        e = g_ws.back().get();
      }
      if (e && e->busy == 0) {
        if (e->cap < bytes) {
          const size_t cap = std::max(bytes, (e->cap + e->cap / 4 + 255) / 256 * 256);
          if (e->ptr) (void)hipFree(e->ptr);
          e->ptr = nullptr;
          e->cap = 0;
          if (hipMalloc((void **)&e->ptr, cap) != hipSuccess || !e->ptr) {
            (void)hipGetLastError();
            e->ptr = nullptr;
            // an empty entry is dropped again; the per-call allocation below may still fit
            for (size_t k = 0; k < g_ws.size(); ++k)
              if (g_ws[k].get() == e) { g_ws.erase(g_ws.begin() + (ptrdiff_t)k); break; }
            e = nullptr;
          } else {
            e->cap = cap;
          }
        }
        if (e) {
          e->busy = 1;
          e->tick = ++g_ws_tick;
          entry_ = e;
          ptr_ = e->ptr;
          return KEOPS_OK;
        }
      }
    }
    if (hipMallocAsync((void **)&ptr_, bytes, st) != hipSuccess || !ptr_) {
      (void)hipGetLastError();
      ptr_ = nullptr;
      return KEOPS_ERR_ALLOC;
    }
    owned_ = true;
    st_ = st;
    return KEOPS_OK;
  }

  char *ptr() const { return ptr_; }

 private:
  void release() {
    if (owned_ && ptr_) (void)hipFreeAsync(ptr_, st_);
    if (entry_) {
      std::lock_guard<std::mutex> lk(g_ws_mu);
      entry_->busy = 0;
      if (g_opt_ws_cache.load(std::memory_order_relaxed) != 1) ws_trim_locked();
    }
    ptr_ = nullptr;
    entry_ = nullptr;
    owned_ = false;
  }

  char *ptr_ = nullptr;
  hipStream_t st_ = nullptr;
  WsEntry *entry_ = nullptr;
  bool owned_ = false;
};

bool overlaps(const void *a, int64_t abytes, const void *b, int64_t bbytes) {
  if (!a || !b || abytes <= 0 || bbytes <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

using GaussDispatch = int (*)(int, int, int, VariantInfo *, dim3, const GaussArgs *, hipStream_t);
using KminDispatch = int (*)(int, int, VariantInfo *, dim3, const KminArgs *, hipStream_t);

const GaussDispatch kGaussUnits[5][2] = {
    {gauss_dispatch_sum_small, gauss_dispatch_sum_large},
    {gauss_dispatch_lse_small, gauss_dispatch_lse_large},
    {gauss_dispatch_grad_small, gauss_dispatch_grad_large},
    {gauss_dispatch_max_small, gauss_dispatch_max_large},
    {laplace_dispatch_sum_small, laplace_dispatch_sum_large},
};
const KminDispatch kKminUnits[3] = {kmin_dispatch_d1_4, kmin_dispatch_d5_8, kmin_dispatch_large};

int gauss_find(int op, int D, int E, int wide, VariantInfo *info, GaussDispatch *fn) {
  for (GaussDispatch f : kGaussUnits[op])
    if (f(D, E, wide, info, dim3(), nullptr, nullptr) == 0) { *fn = f; return 0; }
  return KEOPS_ERR_UNSUPPORTED;
}

int kmin_find(int D, int K, VariantInfo *info, KminDispatch *fn) {
  for (KminDispatch f : kKminUnits)
    if (f(D, K, info, dim3(), nullptr, nullptr) == 0) { *fn = f; return 0; }
  return KEOPS_ERR_UNSUPPORTED;
}

// Default work-groups per CU for each kernel family, from sweeps at the
// 1M x 1M (D = 3), 100k x 10M (D = 50) and 1M x 1M K-min shapes: the VALU sum,
// LSE and grad gain 7-8 % going from 4 to 24 and, with 4 rows per lane, another
// 1.5-2 % at 64 (sum 136.6 -> 134.0 ms, LogSumExp 134.6 -> 132.2, Max 107.0 -> 104.5,
// grad_y 232.9 -> 228.8); with the sum and grad at 2 rows per lane, 128 gains about
// 1 % more on each of them (sum 128.6 -> 127.4 ms, LogSumExp 126.8 -> 126.1, Max
// 100.9 -> 100.0, grad_y 219.1 -> 217.1; 256 about 0.3 % beyond that, with twice
// the partial sums); the MFMA sum gains 7 % from 4 to 16;
// K-min's partial lists are larger, and every split starts its lists empty (the
// early candidates nearly all insert): at 1M x 1M, D = 3, one split (4 per CU)
// ran 112 ms against 115 ms with two (8 per CU) and 114 ms with 16 per CU.
constexpr int64_t kGaussWgsPerCu = 128;
// Block-sparse launches spread the kept pairs over this many work-groups per CU.
constexpr int64_t kRangesWgsPerCu = 24;
constexpr int64_t kMfmaSumWgsPerCu = 16;
constexpr int64_t kKminWgsPerCu = 4;
constexpr int64_t kKminMfmaWgsPerCu = 4;
// Rows from which the sum and LSE take the wide variant (several rows per lane):
// at 50k rows and above it was faster than one row per lane by 3-20 %, at 20k
// and below slower (too few row blocks to fill the GPU).  grad_x keeps one row
// per lane until the wide variant fills every CU: it was the faster one up to
// 200k rows.
constexpr int64_t kWideMinRows = 40000;
// below this many work-groups per CU, the j split may go down to one tile per split
constexpr int64_t kSmallGridWgsPerCu = 8;

struct Plan {
  int wide;
  int64_t rows_wg; // rows per work-group
  int tile_j;
  int64_t nblk;    // work-groups along i
  int nsplit;      // j-splits
  int64_t jps;     // j per split (multiple of tile_j)
};

// Work-groups along i and splits along j.  The split count is chosen so that
// the grid holds about `wgs_per_cu` work-groups per CU (each of four waves), with
// at least two tiles per split.  Many short work-groups let the hardware
// dispatcher even out the CUs' finishing times: the last round of a grid whose
// size is not a multiple of the resident capacity leaves CUs idle, and at a
// handful of work-groups per CU that tail costs several per cent.
Plan make_plan(int64_t M, int64_t N, int cus, int64_t rows_wide, int64_t rows_narrow, int tile_j,
               int64_t wgs_per_cu, int64_t wide_min_rows, int64_t max_split = 65535) {
  const int64_t target = g_opt_wg_target.load();
  if (target > 0) wgs_per_cu = target;
  if (rows_wide < 1) rows_wide = 1;
  if (rows_narrow < 1) rows_narrow = 1;
  if (tile_j < 1) tile_j = 1;
  const int64_t want_wgs = (int64_t)cus * (wgs_per_cu > 0 ? wgs_per_cu : 1);
  Plan p{};
  const int64_t opt_rows = g_opt_rows.load();
  p.wide = opt_rows == 1 ? 0 : (opt_rows == 2 ? 1 : (M >= wide_min_rows));
  p.rows_wg = p.wide ? rows_wide : rows_narrow;
  p.tile_j = tile_j;
  p.nblk = (M + p.rows_wg - 1) / p.rows_wg;
  const int64_t ntiles = (N + tile_j - 1) / tile_j;
  int64_t s = 1;
  const int64_t forced = g_opt_split.load();
  if (forced > 0) {
    s = forced;
  } else if (p.nblk < want_wgs) {
    s = (want_wgs + p.nblk - 1) / p.nblk;
    // at least 4 j tiles per split (with 2-3, the CG solve at 100k x 100k ran 2 %
    // slower), unless that leaves fewer than kSmallGridWgsPerCu work-groups per CU:
    // then down to one tile per split (1k x 1k sum: 13 against 31 us)
    int64_t max_s = ntiles / 4 > 1 ? ntiles / 4 : 1;
    if (p.nblk * max_s < (int64_t)cus * kSmallGridWgsPerCu) max_s = ntiles;
    if (s > max_s) s = max_s;
  }
  if (s > ntiles) s = ntiles;
  if (s > max_split) s = max_split;
  if (s < 1) s = 1;
  if (s > 65535) s = 65535;
  const int64_t tiles_per = (ntiles + s - 1) / s;
  p.jps = tiles_per * tile_j;
  p.nsplit = (int)((N + p.jps - 1) / p.jps);
  return p;
}

int check_launch() { return hipGetLastError() == hipSuccess ? KEOPS_OK : KEOPS_ERR_HIP; }

// Few rows, many j: lanes own j, rows sit in LDS (M <= kStreamMaxRows by default).
// Work-groups along j: about kStreamWgsPerCu per CU over all row groups, between
// 4 and kStreamMaxSteps steps each (the latter bounds the terms one lane adds up).
constexpr int64_t kStreamMaxRows = 64;
constexpr int64_t kStreamWgsPerCu = 8;
constexpr int64_t kStreamMaxSteps = 128;

// Returns kStreamNoFit (nothing enqueued) when `arena` cannot hold its workspace.
constexpr int kStreamNoFit = 1;

int gauss_stream_entry(int op, const float *x, const float *y, const float *b, const float *gv, int64_t M, int64_t N,
                       int D, int E, float sigma, float *out, hipStream_t st, int cus, const VariantInfo &info,
                       int form, const Arena *arena) {
  const int64_t step = info.tile_j;
  const int64_t groups = (M + info.rows_per_wg - 1) / info.rows_per_wg;
  const int64_t nsteps = (N + step - 1) / step;
  const int64_t target = g_opt_wg_target.load() > 0 ? g_opt_wg_target.load() : kStreamWgsPerCu;
  int64_t wgs = ((int64_t)cus * target + groups - 1) / groups;
  const int64_t lo = (nsteps + kStreamMaxSteps - 1) / kStreamMaxSteps;
  const int64_t hi = std::max<int64_t>(1, nsteps / 4);
  wgs = std::max(lo, std::min(wgs, hi));
  if (wgs > nsteps) wgs = nsteps;
  if (wgs < 1) wgs = 1;
  const int64_t jpw = (nsteps + wgs - 1) / wgs * step;
  wgs = (N + jpw - 1) / jpw;
  // one-dimensional grid, 8 x groups x ceil(wgs / 8) ids: the kernels place the row
  // groups of one chunk together on one XCD (the padding ids exit at once)
  const int64_t nblk = 8 * groups * ((wgs + 7) / 8);
  if (nblk > 0x7fffffff) return KEOPS_ERR_UNSUPPORTED;

  // workspace: partials, then (sum: underflow guard, expanded form allowed) the row
  // factors and the maxima of |b| per j chunk (taken by pass 1 from the b it streams)
  const bool guard = op == OP_SUM && form == 0;
  const int PW = op == OP_SUM ? E : (op == OP_LSE ? 2 * E : D);
  float *ws = nullptr;
  const size_t part_bytes = ((size_t)wgs * M * PW * sizeof(float) + 255) / 256 * 256;
  const size_t fac_bytes = guard ? ((size_t)M * sizeof(float) + 255) / 256 * 256 : 0;
  const size_t bmax_bytes = guard ? (size_t)wgs * sizeof(float) : 0;
  Workspace wsp;
  if (arena) {
    if (part_bytes + fac_bytes + bmax_bytes > arena->cap) return kStreamNoFit;
    ws = (float *)arena->base;
  } else {
    if (int rc = wsp.acquire(st, 0, part_bytes + fac_bytes + bmax_bytes)) return rc;
    ws = (float *)wsp.ptr();
  }
  StreamArgs a{};
  a.x = x; a.y = y; a.b = b;
  a.M = M; a.N = N;
  a.scale = (float)std::sqrt(1.4426950408889634 / ((double)sigma * (double)sigma));
  a.j_per_wg = jpw;
  a.part = ws;
  a.form = form == 1 ? FORM_DIRECT : FORM_AUTO;
  a.g = gv;
  a.coef = (float)(-2.0 / ((double)sigma * (double)sigma));
  // pass 2 recomputes an output directly when the guard flags it, or when the sum of
  // its partials is not finite (the shifted accumulators can overflow)
  StreamGuard g{};
  g.x = x; g.y = y; g.b = b;
  g.N = N; g.D = D; g.E = E;
  g.scale = a.scale;
  g.nparts = (int)wgs;
  g.log2n = (float)std::ceil(std::log2((double)N));
  g.g = gv;
  g.coef = a.coef;
  if (guard) {
    a.row_fac = (float *)((char *)ws + part_bytes);
    a.chunk_bmax = (float *)((char *)ws + part_bytes + fac_bytes);
    g.row_fac = a.row_fac;
    g.chunk_bmax = a.chunk_bmax;
  }
  const dim3 grid((unsigned)nblk);
  const int prof = prof_begin(st);
  if (op == OP_SUM) gauss_dispatch_sum_stream(D, E, info.rows_per_wg, nullptr, grid, &a, st);
  else if (op == OP_LSE) gauss_dispatch_lse_stream(D, E, info.rows_per_wg, nullptr, grid, &a, st);
  else gauss_dispatch_grad_stream(D, E, info.rows_per_wg, nullptr, grid, &a, st);
  prof_end(prof, st);
  if (op == OP_SUM) launch_stream_combine(ws, (int)wgs, M * E, out, g, st);
  else if (op == OP_LSE) launch_lse_combine_rows(ws, (int)wgs, M, E, out, st);
  else launch_stream_grad_combine(ws, (int)wgs, M, out, g, st);
  return check_launch();
}

int gauss_entry(int op, const float *x, const float *y, const float *b, const float *g, int64_t M, int64_t N,
                int32_t D, int32_t E, float sigma, float *out, void *stream, int64_t *out_idx = nullptr,
                float max_sign = 1.0f, bool no_alloc = false) {
  // ---- validation (host only)
  if (M < 0 || N < 0 || D < 1 || E < 1) return KEOPS_ERR_INVALID_ARG;
  if (!std::isfinite(sigma) || !(sigma > 0.0f)) return KEOPS_ERR_INVALID_ARG;
  if (M > 0 && (!x || !out)) return KEOPS_ERR_INVALID_ARG;
  if (N > 0 && (!y || !b)) return KEOPS_ERR_INVALID_ARG;
  if (op == OP_GRAD && M > 0 && !g) return KEOPS_ERR_INVALID_ARG;
  if (op == OP_MAX && M > 0 && (!out_idx || ((uintptr_t)out_idx & 7u))) return KEOPS_ERR_INVALID_ARG;
  for (const void *p : {(const void *)x, (const void *)y, (const void *)b, (const void *)g, (const void *)out})
    if (p && !aligned4(p)) return KEOPS_ERR_INVALID_ARG;
  const int W = op == OP_GRAD ? D : E;
  if (M > 0) {
    const int64_t ob = M * W * 4;
    if (overlaps(out, ob, x, M * D * 4) || overlaps(out, ob, y, N * D * 4) || overlaps(out, ob, b, N * E * 4) ||
        (op == OP_GRAD && overlaps(out, ob, g, M * E * 4)))
      return KEOPS_ERR_INVALID_ARG;
    if (op == OP_MAX) {
      const int64_t ib = M * E * 8;
      if (overlaps(out_idx, ib, x, M * D * 4) || overlaps(out_idx, ib, y, N * D * 4) ||
          overlaps(out_idx, ib, b, N * E * 4) || overlaps(out_idx, ib, out, ob))
        return KEOPS_ERR_INVALID_ARG;
    }
  }
  if (op == OP_MAX && N > 0x7fffffffLL) return KEOPS_ERR_UNSUPPORTED;   // indices are int32 inside
  VariantInfo wide_info{}, narrow_info{}, mfma_info{};
  GaussDispatch fn = nullptr;
  if (gauss_find(op, D, E, 1, &wide_info, &fn) || gauss_find(op, D, E, 0, &narrow_info, &fn))
    return KEOPS_ERR_UNSUPPORTED;
  // fp32-MFMA cross term where the contraction is large enough (D >= 32), unless
  // switched off: the sum, the LogSumExp and the gradient with respect to x
  const int64_t form = g_opt_form.load();
  const GaussDispatch mfma_fn = op == OP_SUM ? gauss_dispatch_sum_mfma
                                : (op == OP_LSE ? gauss_dispatch_lse_mfma
                                                : (op == OP_GRAD ? gauss_dispatch_grad_mfma : nullptr));
  const bool use_mfma = mfma_fn && D >= 32 && form == 0 && g_opt_mfma.load() == 0 &&
                        mfma_fn(D, E, 0, &mfma_info, dim3(), nullptr, nullptr) == 0;
  // no-allocation calls: the MFMA path's work-group flags (one per 256-row block and
  // j split) must fit the scratch (split-j partials are then sized to what is left)
  if (no_alloc && use_mfma &&
      (size_t)((M + mfma_info.rows_per_wg - 1) / mfma_info.rows_per_wg) * sizeof(int) + 1024 > kNoAllocScratchBytes)
    return KEOPS_ERR_SCRATCH;
  if (M == 0) return KEOPS_OK;

  // ---- device work
  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();
  Arena arena{nullptr, 0};
  if (no_alloc) {
    if (int rc = scratch_of_device(&arena.base)) return rc;
    arena.cap = kNoAllocScratchBytes;
  }
  if (N == 0) {
    launch_fill(out, M * W, op == OP_LSE ? -INFINITY : (op == OP_MAX ? -max_sign * INFINITY : 0.0f), st);
    if (op == OP_MAX) launch_fill_i64(out_idx, M * E, -1, st);
    return check_launch();
  }
  int cus = 0;
  if (int rc = device_setup(&cus)) return rc;
  // few rows (sum, LogSumExp, gradient; D <= 8): lanes own j, the rows sit in LDS
  if ((op == OP_SUM || op == OP_LSE || op == OP_GRAD) && !use_mfma) {
    VariantInfo sinfo{};
    const int64_t rows_opt = g_opt_rows.load();
    const int mr = M <= 4 ? 4 : (op == OP_GRAD ? stream_grad_mr_large(D) : stream_rows_large(D, E));
    const auto sfn = op == OP_SUM ? gauss_dispatch_sum_stream
                                  : (op == OP_LSE ? gauss_dispatch_lse_stream : gauss_dispatch_grad_stream);
    if ((rows_opt == 3 || (rows_opt == 0 && M <= kStreamMaxRows)) &&
        sfn(D, E, mr, &sinfo, dim3(), nullptr, nullptr) == 0 &&
        (M + sinfo.rows_per_wg - 1) / sinfo.rows_per_wg <= 65535) {
      const int rc = gauss_stream_entry(op, x, y, b, g, M, N, D, E, sigma, out, st, cus, sinfo, (int)form,
                                        no_alloc ? &arena : nullptr);
      if (rc != kStreamNoFit) return rc;   // else: the row-per-lane layout below
    }
  }
  // The MFMA kernel and its direct-form companion both use 256-row work-groups
  // (the narrow VALU variant) and j-splits on the larger of the two tiles.
  const int PW = (op == OP_SUM || op == OP_LAPLACE) ? E : ((op == OP_LSE || op == OP_MAX) ? 2 * E : D);
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  auto plan = [&](int64_t max_split) {
    return use_mfma ? make_plan(M, N, cus, mfma_info.rows_per_wg, mfma_info.rows_per_wg,
                                std::max(mfma_info.tile_j, narrow_info.tile_j), kMfmaSumWgsPerCu, 0, max_split)
                    : make_plan(M, N, cus, wide_info.rows_per_wg, narrow_info.rows_per_wg, wide_info.tile_j,
                                kGaussWgsPerCu, op == OP_GRAD ? wide_info.rows_per_wg * cus : kWideMinRows, max_split);
  };
  auto flag_bytes_of = [&](const Plan &q) { return use_mfma ? al((size_t)q.nblk * q.nsplit * sizeof(int)) : 0; };
  Plan p = plan(65535);
  if (no_alloc && p.nsplit > 1 && al((size_t)p.nsplit * M * PW * sizeof(float)) + flag_bytes_of(p) > arena.cap) {
    // as many j-splits as the scratch holds partials and flags for (one: no partials)
    const size_t per = (size_t)M * PW * sizeof(float) + (use_mfma ? (size_t)p.nblk * sizeof(int) : 0);
    const int64_t fit = (int64_t)((arena.cap > 1024 ? arena.cap - 1024 : 0) / per);
    p = plan(fit >= 2 ? fit : 1);
  }
  const size_t flag_bytes = flag_bytes_of(p);

  const double s2 = (double)sigma * (double)sigma;
  // Laplacian: scale^2 = log2(e) / sigma multiplies |x - y|
  const double scale = op == OP_LAPLACE ? std::sqrt(1.4426950408889634 / (double)sigma)
                                        : std::sqrt(1.4426950408889634 / s2);
  GaussArgs a{};
  a.x = x; a.y = y; a.b = b; a.g = g;
  a.M = M; a.N = N;
  a.scale = (float)scale;
  a.grad_coef = (float)(-2.0 / s2 / scale);
  a.grad_coef_direct = (float)(-2.0 / s2);
  a.j_per_split = p.jps;
  a.nsplit = p.nsplit;
  a.form = form == 1 ? FORM_DIRECT : FORM_AUTO;
  a.wg_flags = nullptr;
  a.out_idx = out_idx;
  a.max_sign = max_sign;

  // workspace: split-j partials, then (MFMA path) one flag per work-group.  The range
  // checks of the expanded and direct forms happen inside each work-group.
  float *ws = nullptr;
  const size_t part_bytes = p.nsplit > 1 ? al((size_t)p.nsplit * M * PW * sizeof(float)) : 0;
  const size_t ws_bytes = part_bytes + flag_bytes;
  Workspace wsp;
  if (ws_bytes > 0) {
    if (no_alloc) {
      if (ws_bytes > arena.cap) return KEOPS_ERR_SCRATCH;
      ws = (float *)arena.base;
    } else {
      if (int rc = wsp.acquire(st, 0, ws_bytes)) return rc;
      ws = (float *)wsp.ptr();
    }
  }
  a.out = p.nsplit > 1 ? ws : out;
  const dim3 grid((unsigned)p.nblk, (unsigned)p.nsplit);
  const int prof = prof_begin(st);
  if (use_mfma) {
    a.wg_flags = (int *)((char *)ws + part_bytes);
    mfma_fn(D, E, 0, nullptr, grid, &a, st);
    prof_end(prof, st);
    GaussArgs b2 = a;            // direct-form VALU pass over the work-groups the MFMA kernel left
    b2.form = FORM_DIRECT;
    fn(D, E, 0, nullptr, grid, &b2, st);
  } else {
    fn(D, E, p.wide, nullptr, grid, &a, st);
    prof_end(prof, st);
  }
  if (p.nsplit > 1) {
    if (op == OP_LSE) launch_lse_combine(ws, p.nsplit, M, E, out, st);
    else if (op == OP_MAX) launch_max_combine(ws, p.nsplit, M, E, max_sign, out, out_idx, st);
    else launch_sum_combine(ws, p.nsplit, M * PW, out, st);
  }
  return check_launch();
}

// ---- block-sparse launches
// Most split slots per row in a block-sparse launch.
constexpr int64_t kMaxRangeSlots = 16;

// Checks the host range arrays: row ranges inside [0, M) and pairwise disjoint,
// slice ends non-decreasing up to nrj, j ranges inside [0, N).
bool ranges_valid(int64_t M, int64_t N, const int64_t *ri, int64_t nri, const int64_t *si, const int64_t *rj,
                  int64_t nrj) {
  if (nri < 0 || nrj < 0 || (nri > 0 && (!ri || !si)) || (nrj > 0 && !rj)) return false;
  std::vector<std::pair<int64_t, int64_t>> rows;
  rows.reserve((size_t)nri);
  int64_t prev = 0;
  for (int64_t c = 0; c < nri; ++c) {
    const int64_t lo = ri[2 * c], hi = ri[2 * c + 1];
    if (lo < 0 || lo > hi || hi > M) return false;
    if (si[c] < prev || si[c] > nrj) return false;
    prev = si[c];
    if (lo < hi) rows.emplace_back(lo, hi);
  }
  std::sort(rows.begin(), rows.end());
  for (size_t c = 1; c < rows.size(); ++c)
    if (rows[c].first < rows[c - 1].second) return false;
  for (int64_t k = 0; k < nrj; ++k)
    if (rj[2 * k] < 0 || rj[2 * k] > rj[2 * k + 1] || rj[2 * k + 1] > N) return false;
  return true;
}

int gauss_ranges_entry(int op, const float *x, const float *y, const float *b, const float *g, int64_t M,
                       int64_t N, int32_t D, int32_t E, float sigma, const int64_t *ranges_i, int64_t nri,
                       const int64_t *slices_i, const int64_t *redranges_j, int64_t nrj, float *out, void *stream) {
  // ---- validation (host only): the same rules as the dense calls, plus the ranges
  if (M < 0 || N < 0 || D < 1 || E < 1) return KEOPS_ERR_INVALID_ARG;
  if (!std::isfinite(sigma) || !(sigma > 0.0f)) return KEOPS_ERR_INVALID_ARG;
  if (M > 0 && (!x || !out)) return KEOPS_ERR_INVALID_ARG;
  if (N > 0 && (!y || !b)) return KEOPS_ERR_INVALID_ARG;
  if (op == OP_GRAD && M > 0 && !g) return KEOPS_ERR_INVALID_ARG;
  for (const void *p : {(const void *)x, (const void *)y, (const void *)b, (const void *)g, (const void *)out})
    if (p && !aligned4(p)) return KEOPS_ERR_INVALID_ARG;
  const int W = op == OP_GRAD ? D : E;
  if (M > 0) {
    const int64_t ob = M * W * 4;
    if (overlaps(out, ob, x, M * D * 4) || overlaps(out, ob, y, N * D * 4) || overlaps(out, ob, b, N * E * 4) ||
        (op == OP_GRAD && overlaps(out, ob, g, M * E * 4)))
      return KEOPS_ERR_INVALID_ARG;
  }
  if (!ranges_valid(M, N, ranges_i, nri, slices_i, redranges_j, nrj)) return KEOPS_ERR_INVALID_ARG;
  VariantInfo wide_info{}, narrow_info{};
  GaussDispatch fn = nullptr;
  if (gauss_find(op, D, E, 1, &wide_info, &fn) || gauss_find(op, D, E, 0, &narrow_info, &fn))
    return KEOPS_ERR_UNSUPPORTED;
  if (M == 0) return KEOPS_OK;

  // ---- plan on the host: rows per work-group from the mean row-range size,
  // j portions (split slots) from the kept pairs per row range
  int64_t covered = 0, nonempty = 0;
  double pairs = 0.0;
  std::vector<int64_t> tj((size_t)nri, 0);
  for (int64_t c = 0; c < nri; ++c) {
    const int64_t len = ranges_i[2 * c + 1] - ranges_i[2 * c];
    for (int64_t k = c == 0 ? 0 : slices_i[c - 1]; k < slices_i[c]; ++k) tj[c] += redranges_j[2 * k + 1] - redranges_j[2 * k];
    if (len > 0 && tj[c] > 0) { covered += len; ++nonempty; pairs += (double)len * (double)tj[c]; }
  }
  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();
  const float empty = op == OP_LSE ? -INFINITY : 0.0f;
  if (nonempty == 0) {
    launch_fill(out, M * W, empty, st);
    return check_launch();
  }
  int cus = 0;
  if (int rc = device_setup(&cus)) return rc;
  const bool wide = g_opt_rows.load() == 2 || (g_opt_rows.load() == 0 && covered / nonempty >= 2 * wide_info.rows_per_wg);
  const int64_t rw = wide ? wide_info.rows_per_wg : narrow_info.rows_per_wg;
  const int tile = wide_info.tile_j;
  const int64_t target = g_opt_wg_target.load() > 0 ? g_opt_wg_target.load() : kRangesWgsPerCu;
  // j per item: the kept pairs spread over ~target work-groups per CU, at least four tiles
  const double jt = std::max(4.0 * tile, pairs / ((double)target * cus * (double)rw));
  const int64_t forced = g_opt_split.load();
  std::vector<BsItem> items;
  int64_t smax = 1;
  for (int64_t c = 0; c < nri; ++c) {
    const int64_t lo = ranges_i[2 * c], hi = ranges_i[2 * c + 1];
    if (lo >= hi || tj[c] == 0) continue;
    const int64_t k0 = c == 0 ? 0 : slices_i[c - 1], k1 = slices_i[c];
    int64_t sc = forced > 0 ? forced : (int64_t)std::ceil((double)tj[c] / jt);
    sc = std::max<int64_t>(1, std::min(sc, std::min(kMaxRangeSlots, tj[c])));
    smax = std::max(smax, sc);
    // the flat position f of the row range's j list as (range k, j)
    auto locate = [&](int64_t f, bool end, int64_t *kk, int64_t *jj) {
      int64_t acc = 0;
      for (int64_t k = k0; k < k1; ++k) {
        const int64_t len = redranges_j[2 * k + 1] - redranges_j[2 * k];
        if (f < acc + len || (end && f == acc + len && len > 0)) { *kk = k; *jj = redranges_j[2 * k] + (f - acc); return; }
        acc += len;
      }
      *kk = k1 - 1;
      *jj = redranges_j[2 * (k1 - 1) + 1];
    };
    for (int64_t s = 0; s < sc; ++s) {
      const int64_t f0 = tj[c] * s / sc, f1 = tj[c] * (s + 1) / sc;
      if (f0 >= f1) continue;
      BsItem it{};
      locate(f0, false, &it.k0, &it.j0);
      locate(f1, true, &it.k1, &it.j1);
      it.slot = (int32_t)s;
      for (int64_t r = lo; r < hi; r += rw) {
        it.row_lo = r;
        it.row_hi = std::min(r + rw, hi);
        items.push_back(it);
      }
    }
  }
  if (items.size() > 0x7fffffffu) return KEOPS_ERR_UNSUPPORTED;

  // ---- workspace: items, j ranges, then (several slots) the partials
  const int PW = op == OP_SUM ? E : (op == OP_LSE ? 2 * E : D);
  const size_t ib = (items.size() * sizeof(BsItem) + 255) / 256 * 256;
  const size_t rb = ((size_t)nrj * 2 * sizeof(int64_t) + 255) / 256 * 256;
  const size_t pb = smax > 1 ? (size_t)smax * M * PW * sizeof(float) : 0;
  Workspace wsp;
  if (int rc = wsp.acquire(st, 0, ib + rb + pb)) return rc;
  char *ws = wsp.ptr();
  std::vector<char> host(ib + rb);
  std::memcpy(host.data(), items.data(), items.size() * sizeof(BsItem));
  if (nrj > 0) std::memcpy(host.data() + ib, redranges_j, (size_t)nrj * 2 * sizeof(int64_t));
  // the host copy must outlive the transfer: wait for it
  if (hipMemcpyAsync(ws, host.data(), ib + rb, hipMemcpyHostToDevice, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return KEOPS_ERR_HIP;
  float *part = smax > 1 ? (float *)(ws + ib + rb) : nullptr;
  // rows outside every kept range (and slots a row range does not use) hold the empty reduction
  if (smax > 1) {
    if (op == OP_LSE) launch_fill2(part, smax * M * E, -3.0e38f, 0.0f, st);
    else launch_fill(part, smax * M * PW, 0.0f, st);
  } else {
    launch_fill(out, M * W, empty, st);
  }

  const double s2 = (double)sigma * (double)sigma;
  const double scale = std::sqrt(1.4426950408889634 / s2);
  GaussArgs a{};
  a.x = x; a.y = y; a.b = b; a.g = g;
  a.M = M; a.N = N;
  a.scale = (float)scale;
  a.grad_coef = (float)(-2.0 / s2 / scale);
  a.grad_coef_direct = (float)(-2.0 / s2);
  a.j_per_split = 0;
  a.nsplit = (int)smax;
  a.form = g_opt_form.load() == 1 ? FORM_DIRECT : FORM_AUTO;
  a.items = (const BsItem *)ws;
  a.redr = (const int64_t *)(ws + ib);
  a.out = smax > 1 ? part : out;
  const int prof = prof_begin(st);
  fn(D, E, wide ? 1 : 0, nullptr, dim3((unsigned)items.size(), 1), &a, st);
  prof_end(prof, st);
  if (smax > 1) {
    if (op == OP_LSE) launch_lse_combine(part, (int)smax, M, E, out, st);
    else launch_sum_combine(part, (int)smax, M * PW, out, st);
  }
  return check_launch();
}

}  // namespace
}  // namespace kmi

using namespace kmi;

extern "C" {

int keops_gauss_sum(const float *x, const float *y, const float *b, int64_t M, int64_t N, int32_t D, int32_t E,
                    float sigma, float *out, void *stream) {
  return gauss_entry(OP_SUM, x, y, b, nullptr, M, N, D, E, sigma, out, stream);
}

int keops_gauss_sum_noalloc(const float *x, const float *y, const float *b, int64_t M, int64_t N, int32_t D,
                            int32_t E, float sigma, float *out, void *stream) {
  return gauss_entry(OP_SUM, x, y, b, nullptr, M, N, D, E, sigma, out, stream, nullptr, 1.0f, true);
}

int keops_gauss_lse(const float *x, const float *y, const float *b, int64_t M, int64_t N, int32_t D, int32_t E,
                    float sigma, float *out, void *stream) {
  return gauss_entry(OP_LSE, x, y, b, nullptr, M, N, D, E, sigma, out, stream);
}

int keops_gauss_grad_x(const float *x, const float *y, const float *b, const float *g, int64_t M, int64_t N,
                       int32_t D, int32_t E, float sigma, float *out, void *stream) {
  return gauss_entry(OP_GRAD, x, y, b, g, M, N, D, E, sigma, out, stream);
}

// The transposed reductions run the row-side kernels with the roles exchanged:
// the points y become the rows, x the columns; for grad_y the payload is g and
// the cotangent b, and the sign of (x - y) flips with the roles, so
//   sum_i (-2/s^2) K <b_j, g_i> (y_j - x_i) = sum_i (2/s^2) K <g_i, b_j> (x_i - y_j).
int keops_gauss_grad_y(const float *x, const float *y, const float *b, const float *g, int64_t M, int64_t N,
                       int32_t D, int32_t E, float sigma, float *out, void *stream) {
  return gauss_entry(OP_GRAD, y, x, g, b, N, M, D, E, sigma, out, stream);
}

int keops_gauss_grad_b(const float *x, const float *y, const float *g, int64_t M, int64_t N, int32_t D,
                       int32_t E, float sigma, float *out, void *stream) {
  return gauss_entry(OP_SUM, y, x, g, nullptr, N, M, D, E, sigma, out, stream);
}

int keops_gauss_cg(const float *x, const float *b, int64_t N, int32_t D, int32_t E, float sigma, float lambda,
                   float rtol, int32_t max_iter, float *out, int32_t *iters, float *rel_residual, void *stream) {
  // ---- validation (host only)
  if (N < 0 || D < 1 || E < 1 || max_iter < 0) return KEOPS_ERR_INVALID_ARG;
  if (!std::isfinite(sigma) || !(sigma > 0.0f) || !std::isfinite(lambda) || lambda < 0.0f) return KEOPS_ERR_INVALID_ARG;
  if (!std::isfinite(rtol) || rtol < 0.0f) return KEOPS_ERR_INVALID_ARG;
  if (N > 0 && (!x || !b || !out)) return KEOPS_ERR_INVALID_ARG;
  for (const void *p : {(const void *)x, (const void *)b, (const void *)out})
    if (p && !aligned4(p)) return KEOPS_ERR_INVALID_ARG;
  if (N > 0 && (overlaps(out, N * E * 4, x, N * D * 4) || overlaps(out, N * E * 4, b, N * E * 4)))
    return KEOPS_ERR_INVALID_ARG;
  if (E > 4) return KEOPS_ERR_UNSUPPORTED;
  {
    VariantInfo vi{};
    GaussDispatch fn = nullptr;
    if (gauss_find(OP_SUM, D, E, 1, &vi, &fn)) return KEOPS_ERR_UNSUPPORTED;
  }
  if (iters) *iters = 0;
  if (rel_residual)
    for (int e = 0; e < E; ++e) rel_residual[e] = 0.0f;
  if (N == 0) return KEOPS_OK;

  // ---- device work: r, p, q [N][E] fp32; partials [kCgBlocks][E] and scalars
  // bb, rr (two slots), pq, rt [E] in double
  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();
  const size_t vec = ((size_t)N * E * sizeof(float) + 255) / 256 * 256;
  const size_t part_bytes = (size_t)kCgBlocks * E * sizeof(double);
  const size_t scal_bytes = 5 * 4 * sizeof(double);
  Workspace wsp;
  if (int rc = wsp.acquire(st, 1, 3 * vec + part_bytes + scal_bytes)) return rc;
  char *ws = wsp.ptr();
  float *r = (float *)ws, *p = (float *)(ws + vec), *q = (float *)(ws + 2 * vec);
  double *part = (double *)(ws + 3 * vec);
  double *sc = (double *)(ws + 3 * vec + part_bytes);
  double *bb = sc, *rr[2] = {sc + 4, sc + 8}, *pq = sc + 12, *rt = sc + 16;
  double h_bb[4] = {0, 0, 0, 0}, h_rr[4] = {0, 0, 0, 0};
  int rc = KEOPS_OK;
  auto fetch = [&](double *host, const double *dev) -> int {
    if (hipMemcpyAsync(host, dev, E * sizeof(double), hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
      return KEOPS_ERR_HIP;
    return KEOPS_OK;
  };
  auto converged = [&](const double *v) {
    for (int e = 0; e < E; ++e)
      if (!(v[e] <= (double)rtol * (double)rtol * h_bb[e])) return false;
    return true;
  };

  launch_cg_init(b, N, E, out, r, p, part, bb, st);
  rc = fetch(h_bb, bb);
  int it = 0;
  int cur = 0;
  if (rc == KEOPS_OK && hipMemcpyAsync(rr[0], bb, E * sizeof(double), hipMemcpyDeviceToDevice, st) != hipSuccess)
    rc = KEOPS_ERR_HIP;
  bool done = converged(h_bb);                       // b = 0 (or rtol >= 1): a = 0
  while (rc == KEOPS_OK && !done && it < max_iter) {
    rc = gauss_entry(OP_SUM, x, x, p, nullptr, N, N, D, E, sigma, q, stream);     // q = K p
    if (rc != KEOPS_OK) break;
    launch_cg_apply(p, q, lambda, N, E, part, pq, st);                            // q += lam p; <p, q>
    launch_cg_step(out, r, p, q, rr[cur], pq, N, E, part, rr[cur ^ 1], st);       // a, r; <r, r>
    ++it;
    rc = fetch(h_rr, rr[cur ^ 1]);
    if (rc != KEOPS_OK) break;
    done = converged(h_rr);
    if (!done) launch_cg_direction(p, r, rr[cur ^ 1], rr[cur], N, E, st);          // p = r + beta p
    cur ^= 1;
  }
  // ---- the true residual |b - (K + lam I) a| / |b| of the returned solution
  if (rc == KEOPS_OK && rel_residual) {
    rc = gauss_entry(OP_SUM, x, x, out, nullptr, N, N, D, E, sigma, q, stream);
    if (rc == KEOPS_OK) {
      launch_cg_apply(out, q, lambda, N, E, part, pq, st);
      launch_cg_residual(b, q, N, E, part, rt, st);
      double h_rt[4] = {0, 0, 0, 0};
      rc = fetch(h_rt, rt);
      for (int e = 0; e < E && rc == KEOPS_OK; ++e)
        rel_residual[e] = h_bb[e] > 0.0 ? (float)std::sqrt(h_rt[e] / h_bb[e]) : 0.0f;
    }
  }
  if (iters) *iters = it;
  if (rc == KEOPS_OK) rc = check_launch();
  if (rc == KEOPS_OK && hipStreamSynchronize(st) != hipSuccess) rc = KEOPS_ERR_HIP;
  return rc;
}

int keops_gauss_sum_ranges(const float *x, const float *y, const float *b, int64_t M, int64_t N, int32_t D,
                           int32_t E, float sigma, const int64_t *ranges_i, int64_t nri, const int64_t *slices_i,
                           const int64_t *redranges_j, int64_t nrj, float *out, void *stream) {
  return gauss_ranges_entry(OP_SUM, x, y, b, nullptr, M, N, D, E, sigma, ranges_i, nri, slices_i, redranges_j, nrj,
                            out, stream);
}

int keops_gauss_lse_ranges(const float *x, const float *y, const float *b, int64_t M, int64_t N, int32_t D,
                           int32_t E, float sigma, const int64_t *ranges_i, int64_t nri, const int64_t *slices_i,
                           const int64_t *redranges_j, int64_t nrj, float *out, void *stream) {
  return gauss_ranges_entry(OP_LSE, x, y, b, nullptr, M, N, D, E, sigma, ranges_i, nri, slices_i, redranges_j, nrj,
                            out, stream);
}

int keops_gauss_grad_x_ranges(const float *x, const float *y, const float *b, const float *g, int64_t M, int64_t N,
                              int32_t D, int32_t E, float sigma, const int64_t *ranges_i, int64_t nri,
                              const int64_t *slices_i, const int64_t *redranges_j, int64_t nrj, float *out,
                              void *stream) {
  return gauss_ranges_entry(OP_GRAD, x, y, b, g, M, N, D, E, sigma, ranges_i, nri, slices_i, redranges_j, nrj, out,
                            stream);
}

int keops_gauss_max(const float *x, const float *y, const float *b, int64_t M, int64_t N, int32_t D, int32_t E,
                    float sigma, float *out, int64_t *out_idx, void *stream) {
  return gauss_entry(OP_MAX, x, y, b, nullptr, M, N, D, E, sigma, out, stream, out_idx, 1.0f);
}

int keops_gauss_min(const float *x, const float *y, const float *b, int64_t M, int64_t N, int32_t D, int32_t E,
                    float sigma, float *out, int64_t *out_idx, void *stream) {
  return gauss_entry(OP_MAX, x, y, b, nullptr, M, N, D, E, sigma, out, stream, out_idx, -1.0f);
}

int keops_laplace_sum(const float *x, const float *y, const float *b, int64_t M, int64_t N, int32_t D, int32_t E,
                      float sigma, float *out, void *stream) {
  return gauss_entry(OP_LAPLACE, x, y, b, nullptr, M, N, D, E, sigma, out, stream);
}

// Few-rows K-min: row groups x chunks of j, about kKminStreamWgsPerCu work-groups per
// CU (three waves per SIMD fit; at 1e8 j, D = 3: 3 per CU ran fastest for K <= 16 and
// 2 for K = 32, whose lists and merges are larger), each chunk at least
// kKminStreamMinSteps steps; a chunk count of 8 or more is kept a multiple of 8, which
// lets the kernel put the row groups of one chunk on one XCD.
constexpr int64_t kKminStreamWgsPerCu = 3;
constexpr int64_t kKminStreamWgsPerCuWideK = 2;
constexpr int64_t kKminStreamMinSteps = 8;

int kmin_stream_entry(const float *x, const float *y, int64_t M, int64_t N, int D, int K, float *out_d,
                      int64_t *out_idx, hipStream_t st, int cus, const VariantInfo &info) {
  const int64_t groups = (M + info.rows_per_wg - 1) / info.rows_per_wg;
  const int64_t nsteps = (N + info.tile_j - 1) / info.tile_j;
  const int64_t target = g_opt_wg_target.load() > 0 ? g_opt_wg_target.load()
                                                    : (K > 16 ? kKminStreamWgsPerCuWideK : kKminStreamWgsPerCu);
  int64_t C = ((int64_t)cus * target + groups - 1) / groups;
  C = std::min(C, std::max<int64_t>(1, nsteps / kKminStreamMinSteps));
  if (C >= 8) C = C / 8 * 8;
  if (g_opt_split.load() > 0) C = g_opt_split.load();   // chunks past N stay empty
  if (groups * C > 0x7fffffff) return KEOPS_ERR_UNSUPPORTED;
  KminArgs a{};
  a.x = x; a.y = y; a.M = M; a.N = N;
  a.nsplit = (int)C;
  a.j_per_split = (N + C - 1) / C;
  const size_t n = (size_t)C * M * K;
  Workspace wsp;
  if (int rc = wsp.acquire(st, 0, n * (sizeof(float) + sizeof(int32_t)))) return rc;
  a.out_d = (float *)wsp.ptr();
  a.part_idx = (int32_t *)((float *)wsp.ptr() + n);
  const int prof = prof_begin(st);
  kmin_dispatch_stream(D, K, nullptr, dim3((unsigned)(groups * C)), &a, st);
  prof_end(prof, st);
  launch_kmin_stream_combine(a.out_d, a.part_idx, (int)C, M, K, out_d, out_idx, st);
  return check_launch();
}

int keops_kmin(const float *x, const float *y, const float * /*b: not read*/, int64_t M, int64_t N, int32_t D,
               int32_t K, float /*sigma: not read*/, float *out_d, int64_t *out_idx, void *stream) {
  if (M < 0 || N < 0 || D < 1 || K < 1) return KEOPS_ERR_INVALID_ARG;
  if ((int64_t)K > N) return KEOPS_ERR_INVALID_ARG;
  if (M > 0 && (!x || !out_d || !out_idx)) return KEOPS_ERR_INVALID_ARG;
  if (!y) return KEOPS_ERR_INVALID_ARG;   // N >= K >= 1
  for (const void *p : {(const void *)x, (const void *)y, (const void *)out_d})
    if (p && !aligned4(p)) return KEOPS_ERR_INVALID_ARG;
  if (out_idx && ((uintptr_t)out_idx & 7u)) return KEOPS_ERR_INVALID_ARG;
  if (M > 0) {
    const int64_t db = M * K * 4, ib = M * K * 8;
    if (overlaps(out_d, db, x, M * D * 4) || overlaps(out_d, db, y, N * D * 4) || overlaps(out_idx, ib, x, M * D * 4) ||
        overlaps(out_idx, ib, y, N * D * 4) || overlaps(out_d, db, out_idx, ib))
      return KEOPS_ERR_INVALID_ARG;
  }
  if (N >= ((int64_t)1 << 31)) return KEOPS_ERR_UNSUPPORTED;
  VariantInfo info{};
  KminDispatch fn = nullptr;
  if (kmin_find(D, K, &info, &fn)) return KEOPS_ERR_UNSUPPORTED;
  // matrix-core prefilter at D >= 32 (the result is the same direct-form K-min):
  // the split-bf16 form by default, the fp32 form when KEOPS_OPT_MFMA is 2
  VariantInfo mfma_info{};
  const int opt_mfma = g_opt_mfma.load();
  const KminDispatch mfma_fn = opt_mfma == 2 ? kmin_dispatch_mfma : kmin_dispatch_mfma_split;
  if (D >= 32 && g_opt_form.load() == 0 && opt_mfma != 1 &&
      mfma_fn(D, K, &mfma_info, dim3(), nullptr, nullptr) == 0) {
    fn = mfma_fn;
    info = mfma_info;
  }
  if (M == 0) return KEOPS_OK;

  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();
  int cus = 0;
  if (int rc = device_setup(&cus)) return rc;
  // few rows: lanes own j, each keeps K-lists for a group of rows
  {
    VariantInfo sinfo{};
    const int64_t rows_opt = g_opt_rows.load();
    if ((rows_opt == 3 || (rows_opt == 0 && M <= kStreamMaxRows)) &&
        kmin_dispatch_stream(D, K, &sinfo, dim3(), nullptr, nullptr) == 0)
      return kmin_stream_entry(x, y, M, N, D, K, out_d, out_idx, st, cus, sinfo);
  }
  const Plan p = make_plan(M, N, cus, info.rows_per_wg, info.rows_per_wg, info.tile_j,
                           (fn == kmin_dispatch_mfma || fn == kmin_dispatch_mfma_split) ? kKminMfmaWgsPerCu : kKminWgsPerCu, 0);
  KminArgs a{};
  a.x = x; a.y = y; a.M = M; a.N = N;
  a.j_per_split = p.jps;
  a.nsplit = p.nsplit;
  Workspace wsp;
  if (p.nsplit > 1) {
    const size_t n = (size_t)p.nsplit * M * K;
    if (int rc = wsp.acquire(st, 0, n * (sizeof(float) + sizeof(int32_t)))) return rc;
    a.out_d = (float *)wsp.ptr();
    a.part_idx = (int32_t *)((float *)wsp.ptr() + n);
  } else {
    a.out_d = out_d;
    a.out_idx = out_idx;
  }
  const int prof = prof_begin(st);
  fn(D, K, nullptr, dim3((unsigned)p.nblk, (unsigned)p.nsplit), &a, st);
  prof_end(prof, st);
  if (p.nsplit > 1) {
    launch_kmin_combine(a.out_d, a.part_idx, p.nsplit, M, K, out_d, out_idx, st);
  }
  return check_launch();
}

const char *keops_status_string(int status) {
  switch (status) {
    case KEOPS_OK: return "ok";
    case KEOPS_ERR_INVALID_ARG: return "invalid argument";
    case KEOPS_ERR_UNSUPPORTED: return "unsupported D, E or K";
    case KEOPS_ERR_ALLOC: return "workspace allocation failed";
    case KEOPS_ERR_HIP: return "HIP error";
    case KEOPS_ERR_SCRATCH: return "the call needs more device scratch than the no-allocation entry point holds";
    default: return "unknown status";
  }
}

int keops_set_option(int option, int64_t value) {
  switch (option) {
    case KEOPS_OPT_SPLIT_J:
      if (value < 0 || value > 65535) return KEOPS_ERR_INVALID_ARG;
      g_opt_split.store(value);
      return KEOPS_OK;
    case KEOPS_OPT_FORM:
      if (value < 0 || value > 1) return KEOPS_ERR_INVALID_ARG;
      g_opt_form.store(value);
      return KEOPS_OK;
    case KEOPS_OPT_ROWS:
      if (value < 0 || value > 3) return KEOPS_ERR_INVALID_ARG;
      g_opt_rows.store(value);
      return KEOPS_OK;
    case KEOPS_OPT_PROFILE:
      if (value < 0 || value > 1) return KEOPS_ERR_INVALID_ARG;
      g_opt_profile.store(value);
      return KEOPS_OK;
    case KEOPS_OPT_WG_TARGET:
      if (value < 0 || value > 4096) return KEOPS_ERR_INVALID_ARG;
      g_opt_wg_target.store(value);
      return KEOPS_OK;
    case KEOPS_OPT_MFMA:
      if (value < 0 || value > 2) return KEOPS_ERR_INVALID_ARG;
      g_opt_mfma.store(value);
      return KEOPS_OK;
    case KEOPS_OPT_WS_CACHE:
      // 0 = 1 here: the cache is on unless switched off
      if (value < 0 || value > 2) return KEOPS_ERR_INVALID_ARG;
      g_opt_ws_cache.store(value == 2 ? 0 : 1);
      if (value == 2) {
        std::lock_guard<std::mutex> lk(g_ws_mu);
        ws_trim_locked();
      }
      return KEOPS_OK;
    case KEOPS_OPT_FAIL_ALLOC:
      if (value < 0 || value > 1) return KEOPS_ERR_INVALID_ARG;
      g_opt_fail_alloc.store(value);
      return KEOPS_OK;
    default:
      return KEOPS_ERR_INVALID_ARG;
  }
}

int keops_profile_read(double *total_ms, int64_t *launches) {
  if (!total_ms || !launches) return KEOPS_ERR_INVALID_ARG;
  std::vector<EventPair> ev;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    ev.swap(g_prof_events);
  }
  double tot = 0.0;
  int rc = KEOPS_OK;
  for (const EventPair &e : ev) {
    float ms = 0.0f;
    if (hipEventSynchronize(e.stop) != hipSuccess || hipEventElapsedTime(&ms, e.start, e.stop) != hipSuccess)
      rc = KEOPS_ERR_HIP;
    tot += ms;
    (void)hipEventDestroy(e.start);
    (void)hipEventDestroy(e.stop);
  }
  *total_ms = tot;
  *launches = (int64_t)ev.size();
  return rc;
}

int keops_version(void) { return 100; }

}  // extern "C"
