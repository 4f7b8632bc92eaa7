// extern "C" entry points of libkvpage.so: host-side validation, then
// launches on the caller's stream.  Declarations and the contract of every
// argument are in include/kvpage.h.
#include <math.h>
#include <stdint.h>

#include "kvpage_common.h"

namespace kvpage {
hipError_t launch_build_queue(const kvpage_shape&, const int32_t*, kvpage_task*, int32_t, int32_t*,
                              int32_t*, hipStream_t);
hipError_t launch_gather_offsets(const kvpage_shape&, const int32_t*, const kvpage_task*,
                                 const int32_t*, int32_t, int64_t*, hipStream_t);
hipError_t launch_split_attn(const kvpage_shape&, const void*, const void*, const void*,
                             const int32_t*, const kvpage_task*, const int32_t*, int32_t, void*,
                             const kvpage_budget*, hipStream_t, hipEvent_t, hipEvent_t,
                             const int32_t*, kvpage_task*, int32_t*, int32_t*, int32_t);
bool split_attn_can_fuse_queue(const kvpage_shape&);
hipError_t launch_append(const kvpage_shape&, const void*, const void*, void*, void*, int32_t*,
                         const int32_t*, int32_t*, const int32_t*, const int32_t*, int32_t*,
                         int32_t*, hipStream_t);
int split_attn_waves_per_cu();
int split_attn_chunk_max();
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
  if (s->split_tokens > 16 * kPage) return KVPAGE_ERR_UNSUPPORTED;
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
                                     nullptr, nullptr, 0));
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
                                       nullptr, nullptr, nullptr, nullptr, 0)));
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
  if (capacity > 0 && split_attn_can_fuse_queue(*s)) {
    // The attention kernel builds the queue itself (same content, same order).
    KV_TRY(status_of(launch_split_attn(*s, q, k_pool, v_pool, block_tables, tasks, n_tasks,
                                       capacity, workspace, budget, stream, t0, t1, ctx_lens,
                                       tasks, group_offsets, n_tasks, max_wg)));
  } else {
    KV_TRY(status_of(launch_build_queue(*s, ctx_lens, tasks, capacity, group_offsets, n_tasks,
                                        stream)));
    if (capacity > 0) {
      KV_TRY(status_of(launch_split_attn(*s, q, k_pool, v_pool, block_tables, tasks, n_tasks,
                                         capacity, workspace, budget, stream, t0, t1, nullptr,
                                         nullptr, nullptr, nullptr, max_wg)));
    }
  }
  if (budget)
    return status_of(launch_merge_finish(*s, *budget, q, ctx_lens, group_offsets, capacity,
                                         workspace, out, lse, stream));
  return status_of(launch_merge(*s, group_offsets, capacity, workspace, out, lse, stream));
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
  const int32_t longest = 16 * t.page_size;
  if (total == 0) return longest;
  // Among the splits whose queue holds a task for every resident wavefront,
  // the one whose busiest wavefront has the least work under the attention
  // kernel's schedule (rounds of chunks of at most chunk_max positions):
  // its tasks times (pages per task + a task's fixed cost), the fixed cost
  // measured at half a page with streaming tile loads and one and a half
  // with cached ones.  Ties go to the longer split; none qualifies: the page
  // size.
  const int64_t chunk_max = split_attn_chunk_max();
  const int64_t task_cost2 = (t.flags & KVPAGE_FLAG_STREAM_KV) ? 1 : 3;   // twice the fixed cost
  int32_t best = 0;
  int64_t best_cost = INT64_MAX;
  for (int32_t split = longest; split >= t.page_size; split /= 2) {
    int64_t tasks = 0;
    for (int b = 0; b < t.B; ++b) tasks += (ctx_lens_host[b] + split - 1) / split;
    tasks *= t.Hkv;
    if (tasks < waves) continue;
    const int64_t rounds = (tasks + waves * chunk_max - 1) / (waves * chunk_max);
    const int64_t c = (tasks + waves * rounds - 1) / (waves * rounds);
    const int64_t cost = c * rounds * (2 * (split / t.page_size) + task_cost2);   // twice the work
    if (cost < best_cost) {
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
    default: return "unknown status";
  }
}

}  // extern "C"
