// extern "C" entry points of libkvpage.so: host-side validation, then
// launches on the caller's stream.  Declarations and the contract of every
// argument are in include/kvpage.h.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <vector>

#include "kvpage_common.h"

// Workspace of kvpage_decode_step_noalloc: one copy per device, at its own
// address on each.  Host code never passes this name to a kernel (on the
// host it is only a stand-in for the symbol); it uses the device address
// that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[KVPAGE_NOALLOC_WORKSPACE_BYTES];

namespace kvpage {
hipError_t launch_build_queue(const kvpage_shape&, const int32_t*, kvpage_task*, int32_t, int32_t*,
                              int32_t*, hipStream_t);
hipError_t launch_gather_offsets(const kvpage_shape&, const int32_t*, const kvpage_task*,
                                 const int32_t*, int32_t, int64_t*, hipStream_t);
hipError_t launch_split_attn(const kvpage_shape&, const void*, const void*, const void*,
                             const int32_t*, const kvpage_task*, const int32_t*, int32_t, void*,
                             const kvpage_budget*, hipStream_t, hipEvent_t, hipEvent_t,
                             const int32_t*, kvpage_task*, int32_t*, int32_t*, int32_t,
                             const int32_t*);
bool split_attn_can_fuse_queue(const kvpage_shape&);
hipError_t launch_append(const kvpage_shape&, const void*, const void*, void*, void*, int32_t*,
                         const int32_t*, int32_t*, const int32_t*, const int32_t*, int32_t*,
                         int32_t*, hipStream_t);
int split_attn_waves_per_cu();
int split_attn_chunk_max(int split_tokens);
hipError_t launch_merge(const kvpage_shape&, const int32_t*, int32_t, const void*, void*, float*,
                        hipStream_t);
hipError_t launch_merge_finish(const kvpage_shape&, const kvpage_budget&, const void*,
                               const int32_t*, const int32_t*, int32_t, const void*, void*, float*,
                               hipStream_t);
hipError_t launch_check_inputs(const kvpage_shape&, const int32_t*, const int32_t*,
                               const kvpage_task*, const int32_t*, const int32_t*, int32_t, int32_t*,
                               hipStream_t);
hipError_t launch_page_mass(const kvpage_shape&, const kvpage_budget&, const void*, const float*,
                            const int32_t*, const int32_t*, int32_t, const void*, hipStream_t);
hipError_t launch_budget_decide(const kvpage_shape&, const float*, const int32_t*, float, int32_t*,
                                float*, int32_t*, int32_t*, int32_t*, hipStream_t);
int decide_max_pages();

namespace {

// Structural checks every entry point shares.  Returns a kvpage_status.
int check_shape(const kvpage_shape* s) {
  if (!s) return KVPAGE_ERR_INVALID_ARG;
  if (s->B < 0 || s->Hq <= 0 || s->Hkv <= 0 || s->d <= 0 || s->page_size <= 0 ||
      s->split_tokens <= 0 || s->max_pages <= 0 || s->num_pages <= 0)
    return KVPAGE_ERR_INVALID_ARG;
  if (s->Hq % s->Hkv != 0) return KVPAGE_ERR_INVALID_ARG;
  if (s->split_tokens % s->page_size != 0) return KVPAGE_ERR_INVALID_ARG;
  if (!(s->scale > 0.0f) || !isfinite(s->scale)) return KVPAGE_ERR_INVALID_ARG;
  if (s->dtype != KVPAGE_F16 && s->dtype != KVPAGE_BF16) return KVPAGE_ERR_INVALID_ARG;
  if ((s->flags & ~KVPAGE_FLAG_STREAM_KV) != 0) return KVPAGE_ERR_INVALID_ARG;
  // Token indices (including one split past the end) must fit in int32.
  if ((int64_t)s->max_pages * s->page_size + s->split_tokens > INT32_MAX)
    return KVPAGE_ERR_INVALID_ARG;
  if ((int64_t)s->B * s->Hq * s->max_pages > INT64_MAX / 8) return KVPAGE_ERR_INVALID_ARG;
  return KVPAGE_OK;
}

// What the attention kernels are built for.
int check_supported(const kvpage_shape* s) {
  if (s->page_size != kPage) return KVPAGE_ERR_UNSUPPORTED;
  if (s->d != 64 && s->d != 128) return KVPAGE_ERR_UNSUPPORTED;
  const int G = s->Hq / s->Hkv;
  if (G < 1 || G > 8) return KVPAGE_ERR_UNSUPPORTED;
  // Splits up to 16 pages, or whole multiples of 16 pages up to 256 pages
  // (run as pieces of 16 pages).
  if (s->split_tokens > 16 * kPage &&
      (s->split_tokens % (16 * kPage) != 0 || s->split_tokens > 256 * kPage))
    return KVPAGE_ERR_UNSUPPORTED;
  if ((int64_t)s->B * s->Hq > INT32_MAX) return KVPAGE_ERR_UNSUPPORTED;
  return KVPAGE_OK;
}

int64_t capacity_of(const kvpage_shape* s) {
  const int64_t tokens = (int64_t)s->max_pages * s->page_size;
  const int64_t splits = (tokens + s->split_tokens - 1) / s->split_tokens;
  return (int64_t)s->B * s->Hkv * splits;
}

int check_capacity(const kvpage_shape* s, int32_t capacity) {
  if (capacity < 0) return KVPAGE_ERR_INVALID_ARG;
  if ((int64_t)capacity < capacity_of(s)) return KVPAGE_ERR_CAPACITY;
  return KVPAGE_OK;
}

int check_budget(const kvpage_budget* b) {
  if (!b->page_mass || !b->s_prev || !b->s_next || !b->page_max) return KVPAGE_ERR_INVALID_ARG;
  if (b->s_prev == b->s_next) return KVPAGE_ERR_INVALID_ARG;
  if (!(b->alpha_fast >= 0.0f && b->alpha_fast <= 1.0f)) return KVPAGE_ERR_INVALID_ARG;
  if (!(b->alpha_slow >= 0.0f && b->alpha_slow <= 1.0f)) return KVPAGE_ERR_INVALID_ARG;
  return KVPAGE_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? KVPAGE_OK : KVPAGE_ERR_HIP; }

#define KV_TRY(expr)          \
  do {                        \
    const int st_ = (expr);   \
    if (st_ != KVPAGE_OK) return st_; \
  } while (0)

bool aligned(const void* ptr, uintptr_t bytes) {
  return reinterpret_cast<uintptr_t>(ptr) % bytes == 0;
}

int validate_attn(const kvpage_shape* s, const void* q, const void* k_pool, const void* v_pool,
                  const int32_t* block_tables, const kvpage_task* tasks, const int32_t* n_tasks,
                  int32_t capacity, const void* workspace, const kvpage_budget* budget) {
  KV_TRY(check_shape(s));
  KV_TRY(check_supported(s));
  KV_TRY(check_capacity(s, capacity));
  if (!q || !k_pool || !v_pool || !block_tables || !tasks || !n_tasks || !workspace)
    return KVPAGE_ERR_INVALID_ARG;
  // 16-byte vector loads of query rows, pool tiles and workspace partials.
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(workspace, 16))
    return KVPAGE_ERR_INVALID_ARG;
  if (budget) KV_TRY(check_budget(budget));
  return KVPAGE_OK;
}

// Device address of `scratch` on the current device, looked up on the first
// call per device and kept.  Concurrent first calls may both look it up;
// they store the same address.
int scratch_address(void** out) {
  static std::atomic<void*> addr[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KVPAGE_ERR_HIP;
  if (dev < 0 || dev >= 64) return KVPAGE_ERR_UNSUPPORTED;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVPAGE_ERR_HIP;
    addr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return KVPAGE_OK;
}

}  // namespace
}  // namespace kvpage

using namespace kvpage;

extern "C" {

int32_t kvpage_queue_capacity(const kvpage_shape* s) {
  const int st = check_shape(s);
  if (st != KVPAGE_OK) return st;
  const int64_t cap = capacity_of(s);
  if (cap > INT32_MAX) return KVPAGE_ERR_UNSUPPORTED;
  return (int32_t)cap;
}

int64_t kvpage_workspace_bytes(const kvpage_shape* s, int32_t capacity) {
  int st = check_shape(s);
  if (st == KVPAGE_OK) st = check_supported(s);
  if (st == KVPAGE_OK) st = check_capacity(s, capacity);
  if (st != KVPAGE_OK) return st;
  return (int64_t)ws_bytes(capacity, s->Hq / s->Hkv, s->d);
}

int kvpage_check_inputs(const kvpage_shape* s, const int32_t* ctx_lens,
                        const int32_t* block_tables, const kvpage_task* tasks,
                        const int32_t* group_offsets, const int32_t* n_tasks, int32_t capacity,
                        int32_t* status, hipStream_t stream) {
  KV_TRY(check_shape(s));
  if (!ctx_lens || !block_tables || !status) return KVPAGE_ERR_INVALID_ARG;
  const bool queue = tasks || group_offsets || n_tasks;
  if (queue) {
    if (!tasks || !group_offsets || !n_tasks) return KVPAGE_ERR_INVALID_ARG;
    KV_TRY(check_capacity(s, capacity));
  }
  return status_of(launch_check_inputs(*s, ctx_lens, block_tables, queue ? tasks : nullptr,
                                       group_offsets, n_tasks, capacity, status, stream));
}

int kvpage_build_queue(const kvpage_shape* s, const int32_t* ctx_lens, kvpage_task* tasks,
                       int32_t capacity, int32_t* group_offsets, int32_t* n_tasks,
                       hipStream_t stream) {
  KV_TRY(check_shape(s));
  KV_TRY(check_capacity(s, capacity));
  if (!ctx_lens || !tasks || !group_offsets || !n_tasks) return KVPAGE_ERR_INVALID_ARG;
  if (s->B == 0) return KVPAGE_OK;
  return status_of(launch_build_queue(*s, ctx_lens, tasks, capacity, group_offsets, n_tasks, stream));
}

int kvpage_split_attn(const kvpage_shape* s, const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_tables, const int32_t* ctx_lens,
                      const kvpage_task* tasks, const int32_t* n_tasks, int32_t capacity,
                      void* workspace, const kvpage_budget* budget, hipStream_t stream) {
  KV_TRY(validate_attn(s, q, k_pool, v_pool, block_tables, tasks, n_tasks, capacity, workspace,
                       budget));
  if (!ctx_lens) return KVPAGE_ERR_INVALID_ARG;
  if (s->B == 0 || capacity == 0) return KVPAGE_OK;
  return status_of(launch_split_attn(*s, q, k_pool, v_pool, block_tables, tasks, n_tasks, capacity,
                                     workspace, budget, stream, nullptr, nullptr, nullptr, nullptr,
                                     nullptr, nullptr, 0, nullptr));
}

int kvpage_merge_splits(const kvpage_shape* s, const int32_t* group_offsets, int32_t capacity,
                        const void* workspace, void* out, float* lse, hipStream_t stream) {
  KV_TRY(check_shape(s));
  KV_TRY(check_supported(s));
  KV_TRY(check_capacity(s, capacity));
  if (!group_offsets || !workspace || !out || !lse) return KVPAGE_ERR_INVALID_ARG;
  if (!aligned(workspace, 16) || !aligned(out, 8)) return KVPAGE_ERR_INVALID_ARG;
  if (s->B == 0) return KVPAGE_OK;
  return status_of(launch_merge(*s, group_offsets, capacity, workspace, out, lse, stream));
}

int kvpage_decode_attn(const kvpage_shape* s, const void* q, const void* k_pool, const void* v_pool,
                       const int32_t* block_tables, const int32_t* ctx_lens,
                       const kvpage_task* tasks, const int32_t* group_offsets,
                       const int32_t* n_tasks, int32_t capacity, void* workspace,
                       const kvpage_budget* budget, void* out, float* lse, hipStream_t stream) {
  KV_TRY(validate_attn(s, q, k_pool, v_pool, block_tables, tasks, n_tasks, capacity, workspace,
                       budget));
  if (!ctx_lens || !group_offsets || !out || !lse) return KVPAGE_ERR_INVALID_ARG;
  if (!aligned(out, 8)) return KVPAGE_ERR_INVALID_ARG;
  if (s->B == 0) return KVPAGE_OK;
  if (capacity > 0) {
    KV_TRY(status_of(launch_split_attn(*s, q, k_pool, v_pool, block_tables, tasks, n_tasks,
                                       capacity, workspace, budget, stream, nullptr, nullptr,
                                       nullptr, nullptr, nullptr, nullptr, 0, nullptr)));
  }
  return status_of(launch_merge(*s, group_offsets, capacity, workspace, out, lse, stream));
}

int kvpage_decode_step(const kvpage_shape* s, const void* q, const void* k_pool,
                       const void* v_pool, const int32_t* block_tables, const int32_t* ctx_lens,
                       kvpage_task* tasks, int32_t* group_offsets, int32_t* n_tasks,
                       int32_t capacity, void* workspace, const kvpage_budget* budget, void* out,
                       float* lse, const kvpage_launch_opts* opts, hipStream_t stream) {
  KV_TRY(validate_attn(s, q, k_pool, v_pool, block_tables, tasks, n_tasks, capacity, workspace,
                       budget));
  if (!ctx_lens || !group_offsets || !out || !lse) return KVPAGE_ERR_INVALID_ARG;
  if (!aligned(out, 8)) return KVPAGE_ERR_INVALID_ARG;
  if (s->B == 0) return KVPAGE_OK;
  hipEvent_t t0 = opts ? opts->attn_start : nullptr;
  hipEvent_t t1 = opts ? opts->attn_stop : nullptr;
  const int max_wg = opts ? opts->max_workgroups : 0;
  if (max_wg < 0) return KVPAGE_ERR_INVALID_ARG;
  // Shared leading pages matter only with streaming loads (else every load
  // goes through the caches already).
  const int32_t* shared =
      (opts && (s->flags & KVPAGE_FLAG_STREAM_KV)) ? opts->shared_pages : nullptr;
  if (capacity > 0 && split_attn_can_fuse_queue(*s)) {
    // The attention kernel builds the queue itself (same content, same order).
    KV_TRY(status_of(launch_split_attn(*s, q, k_pool, v_pool, block_tables, tasks, n_tasks,
                                       capacity, workspace, budget, stream, t0, t1, ctx_lens,
                                       tasks, group_offsets, n_tasks, max_wg, shared)));
  } else {
    KV_TRY(status_of(launch_build_queue(*s, ctx_lens, tasks, capacity, group_offsets, n_tasks,
                                        stream)));
    if (capacity > 0) {
      KV_TRY(status_of(launch_split_attn(*s, q, k_pool, v_pool, block_tables, tasks, n_tasks,
                                         capacity, workspace, budget, stream, t0, t1, nullptr,
                                         nullptr, nullptr, nullptr, max_wg, shared)));
    }
  }
  if (budget)
    return status_of(launch_merge_finish(*s, *budget, q, ctx_lens, group_offsets, capacity,
                                         workspace, out, lse, stream));
  return status_of(launch_merge(*s, group_offsets, capacity, workspace, out, lse, stream));
}

int kvpage_decode_step_noalloc(const kvpage_shape* s, const void* q, const void* k_pool,
                               const void* v_pool, const int32_t* block_tables,
                               const int32_t* ctx_lens, kvpage_task* tasks,
                               int32_t* group_offsets, int32_t* n_tasks, int32_t capacity,
                               const kvpage_budget* budget, void* out, float* lse,
                               const kvpage_launch_opts* opts, hipStream_t stream) {
  KV_TRY(check_shape(s));
  KV_TRY(check_supported(s));
  KV_TRY(check_capacity(s, capacity));
  if (ws_bytes(capacity, s->Hq / s->Hkv, s->d) > (size_t)KVPAGE_NOALLOC_WORKSPACE_BYTES)
    return KVPAGE_ERR_SCRATCH;
  void* ws = nullptr;
  KV_TRY(scratch_address(&ws));
  return kvpage_decode_step(s, q, k_pool, v_pool, block_tables, ctx_lens, tasks, group_offsets,
                            n_tasks, capacity, ws, budget, out, lse, opts, stream);
}

int kvpage_page_mass(const kvpage_shape* s, const kvpage_budget* budget, const void* q,
                     const float* lse, const int32_t* ctx_lens, const int32_t* group_offsets,
                     int32_t capacity, const void* workspace, hipStream_t stream) {
  KV_TRY(check_shape(s));
  KV_TRY(check_supported(s));
  KV_TRY(check_capacity(s, capacity));
  if (!budget) return KVPAGE_ERR_INVALID_ARG;
  KV_TRY(check_budget(budget));
  if (!q || !lse || !ctx_lens || !group_offsets || !workspace) return KVPAGE_ERR_INVALID_ARG;
  if (s->B == 0) return KVPAGE_OK;
  return status_of(launch_page_mass(*s, *budget, q, lse, ctx_lens, group_offsets, capacity,
                                    workspace, stream));
}

int kvpage_debug_gather_offsets(const kvpage_shape* s, const int32_t* block_tables,
                                const kvpage_task* tasks, const int32_t* n_tasks,
                                int32_t capacity, int64_t* offsets, hipStream_t stream) {
  KV_TRY(check_shape(s));
  KV_TRY(check_capacity(s, capacity));
  if (!block_tables || !tasks || !n_tasks || !offsets) return KVPAGE_ERR_INVALID_ARG;
  if (s->B == 0 || capacity == 0) return KVPAGE_OK;
  return status_of(launch_gather_offsets(*s, block_tables, tasks, n_tasks, capacity, offsets, stream));
}

int kvpage_append_kv(const kvpage_shape* s, const void* k_new, const void* v_new, void* k_pool,
                     void* v_pool, int32_t* block_tables, const int32_t* ctx_lens,
                     int32_t* ctx_lens_out, const int32_t* free_pages, const int32_t* free_count,
                     int32_t* free_count_out, int32_t* status, hipStream_t stream) {
  KV_TRY(check_shape(s));
  KV_TRY(check_supported(s));
  if (!k_new || !v_new || !k_pool || !v_pool || !block_tables || !ctx_lens || !ctx_lens_out ||
      !free_pages || !free_count || !free_count_out || !status)
    return KVPAGE_ERR_INVALID_ARG;
  if (ctx_lens == ctx_lens_out || free_count == free_count_out) return KVPAGE_ERR_INVALID_ARG;
  // 16-byte row copies: the rows of one token are d halves (d is 64 or 128).
  for (const void* ptr : {k_new, v_new, (const void*)k_pool, (const void*)v_pool})
    if (!aligned(ptr, 16)) return KVPAGE_ERR_INVALID_ARG;
  return status_of(launch_append(*s, k_new, v_new, k_pool, v_pool, block_tables, ctx_lens,
                                 ctx_lens_out, free_pages, free_count, free_count_out, status,
                                 stream));
}

int kvpage_budget_decide(const kvpage_shape* s, const float* page_max, const int32_t* ctx_lens,
                         float tau, int32_t* ws_size, float* ws_level, int32_t* ws_union,
                         int32_t* decision, int32_t* victim, hipStream_t stream) {
  KV_TRY(check_shape(s));
  if (s->page_size != kPage) return KVPAGE_ERR_UNSUPPORTED;
  if (s->max_pages > decide_max_pages()) return KVPAGE_ERR_UNSUPPORTED;
  if ((int64_t)2 * s->B * s->Hkv > INT32_MAX) return KVPAGE_ERR_UNSUPPORTED;
  if (!(tau > 0.0f && tau <= 1.0f)) return KVPAGE_ERR_INVALID_ARG;
  if (!page_max || !ctx_lens || !ws_size || !ws_level || !ws_union || !decision || !victim)
    return KVPAGE_ERR_INVALID_ARG;
  if (s->B == 0) return KVPAGE_OK;
  return status_of(launch_budget_decide(*s, page_max, ctx_lens, tau, ws_size, ws_level, ws_union,
                                        decision, victim, stream));
}

// ---- Split policy --------------------------------------------------------
//
// The attention kernel is bound by HBM: with every wavefront streaming, each
// gets an equal share of the bandwidth, and once some have finished the rest
// stream faster, up to kWaveRateCap times that share (measured on MI355X: a
// wavefront reads 0.77 pages/us when 1024 stream and 1.37 pages/us when 256
// do; the value below fits the split timings of the B1, B4, B8 and B64
// workloads best).  A split is priced by simulating the kernel's schedule:
// each wavefront's pages plus a fixed cost per queue position, then the
// time to finish when every unfinished wavefront streams at
// min(cap, wavefronts / unfinished) (water filling), in units of one page at
// the equal share.
constexpr double kWaveRateCap = 1.43;
constexpr int64_t kSimRoundsMax = 8;   // past this, the wavefronts' loads are taken as equal

static double water_fill(std::vector<double>& load) {
  std::sort(load.begin(), load.end());
  const double n = (double)load.size();
  double t = 0.0, done = 0.0;
  for (size_t i = 0; i < load.size(); ++i) {
    const double active = n - (double)i;
    const double rate = std::min(kWaveRateCap, n / active);
    t += (load[i] - done) / rate;
    done = load[i];
  }
  return t;
}

// Cost of split S (tokens, a multiple of the page size), or a negative value
// if its queue has fewer tasks than wavefronts.  The schedule mirrors the
// attention kernel's: with more than one sequence, at most 64 (fused queue
// build), Hkv a multiple of 8 and wavefronts a multiple of 32, 8 classes of
// KV heads each on its own wavefronts (identical, so one is simulated);
// chunks of c positions per class, at most 16 pieces of 16 pages each.
static double split_cost(const kvpage_shape& t, const int32_t* ctx, int32_t S, int64_t waves,
                         double fixed) {
  const int P = t.page_size;
  const int ncls = (t.B >= 2 && t.B <= 64 && t.Hkv % 8 == 0 && waves % 32 == 0) ? 8 : 1;
  const int64_t hpc = t.Hkv / ncls, nwc = waves / ncls;
  // Per sequence: class positions and pages before it (prefix sums).
  std::vector<int64_t> pos(t.B + 1, 0), pages(t.B + 1, 0);
  for (int b = 0; b < t.B; ++b) {
    pos[b + 1] = pos[b] + hpc * ((ctx[b] + S - 1) / S);
    pages[b + 1] = pages[b] + hpc * ((ctx[b] + P - 1) / P);
  }
  const int64_t T = pos[t.B];
  if (T * ncls < waves) return -1.0;
  const int64_t cmax = split_attn_chunk_max(S);
  int64_t rounds = 1, c;
  if (T <= nwc * cmax) {
    c = (T + nwc - 1) / nwc;
  } else {
    rounds = (T + nwc * cmax - 1) / (nwc * cmax);
    c = (T + nwc * rounds - 1) / (nwc * rounds);
  }
  if (rounds > kSimRoundsMax)   // many chunks per wavefront: equal loads
    return ((double)pages[t.B] + fixed * (double)T) / (double)nwc;
  // Pages of class positions [0, p): sequence b holds positions
  // [pos[b], pos[b+1]), hpc KV heads of n tasks each, all full splits but
  // the last.
  auto prefix = [&](int64_t p) -> int64_t {
    const int b = (int)(std::upper_bound(pos.begin(), pos.end(), p) - pos.begin()) - 1;
    if (b >= t.B) return pages[t.B];
    const int64_t n = (ctx[b] + S - 1) / S;
    const int64_t r = p - pos[b], gi = r / n, j = r - gi * n;
    return pages[b] + gi * ((ctx[b] + P - 1) / P) + j * (S / P);
  };
  std::vector<double> load(nwc, 0.0);
  for (int64_t k = 0; k * c < T; ++k) {
    const int64_t a = k * c, e = std::min(a + c, T);
    load[k % nwc] += (double)(prefix(e) - prefix(a)) + fixed * (double)(e - a);
  }
  return water_fill(load);
}

int32_t kvpage_choose_split(const kvpage_shape* s, const int32_t* ctx_lens_host,
                            int32_t wavefronts) {
  if (!s) return KVPAGE_ERR_INVALID_ARG;
  // The shape is checked as if split at the page size (the split is the output).
  kvpage_shape t = *s;
  t.split_tokens = t.page_size;
  KV_TRY(check_shape(&t));
  KV_TRY(check_supported(&t));
  if (t.B > 0 && !ctx_lens_host) return KVPAGE_ERR_INVALID_ARG;
  const int64_t max_ctx = (int64_t)t.max_pages * t.page_size;
  int64_t total = 0;
  for (int b = 0; b < t.B; ++b) {
    if (ctx_lens_host[b] < 0 || ctx_lens_host[b] > max_ctx) return KVPAGE_ERR_INVALID_ARG;
    total += ctx_lens_host[b];
  }
  int64_t waves = wavefronts;
  if (waves <= 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return KVPAGE_ERR_HIP;
    waves = (int64_t)cus * split_attn_waves_per_cu();
  }
  if (total == 0) return 16 * t.page_size;
  // Candidates from the longest split down to the page size; only splits
  // whose queue holds a task for every resident wavefront qualify; the
  // cheapest wins, ties to the longer split; none qualifies: the page size.
  // The fixed cost of a queue position is measured: half a page with
  // streaming loads, one and a half with cached ones.  Where pages may be
  // shared (cached loads) splits stay at 16 pages or less: wavefronts
  // running side by side then read a shared prefix's pages close together
  // in time, from L2 (B64 with a shared prefix: 256 tokens 4.4% faster than
  // 1024).
  const bool streaming = (t.flags & KVPAGE_FLAG_STREAM_KV) != 0;
  const int32_t longest = (streaming ? 256 : 16) * t.page_size;
  const double fixed = streaming ? 0.5 : 1.5;
  int32_t best = 0;
  double best_cost = 0.0;
  for (int32_t split = longest; split >= t.page_size; split /= 2) {
    const double cost = split_cost(t, ctx_lens_host, split, waves, fixed);
    if (cost < 0.0) continue;
    if (best == 0 || cost < best_cost) {
      best_cost = cost;
      best = split;
    }
  }
  return best ? best : t.page_size;
}

const char* kvpage_status_string(int status) {
  switch (status) {
    case KVPAGE_OK: return "ok";
    case KVPAGE_ERR_INVALID_ARG: return "invalid argument";
    case KVPAGE_ERR_UNSUPPORTED: return "unsupported shape";
    case KVPAGE_ERR_CAPACITY: return "task capacity too small";
    case KVPAGE_ERR_HIP: return "HIP runtime error";
    case KVPAGE_ERR_SCRATCH: return "workspace larger than the static no-allocation workspace";
    default: return "unknown status";
  }
}

}  // extern "C"
