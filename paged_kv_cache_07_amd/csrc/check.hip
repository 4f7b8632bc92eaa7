// Debug checks of the data-dependent preconditions of the decode calls.
//
// The attention, merge and page-mass kernels clamp every length, page id and
// queue entry they read into the shape instead of reporting it (a violation
// gives wrong values for its rows, never an access outside the buffers).  A
// caller that wants to know runs this pass: it reads the lengths, the
// block-table entries the sequences use and, if given, the queue, and
// writes a status word with one bit per kind of violation.  It is separate
// from the hot path and costs nothing when not called.
#include "kvpage_common.h"

namespace kvpage {

struct CheckParams {
  const int32_t* ctx_lens;
  const int32_t* block_tables;
  const kvpage_task* tasks;
  const int32_t* group_offsets;
  const int32_t* n_tasks;
  int32_t* status;
  int32_t B, Hkv, max_pages, num_pages, split_tokens, capacity;
};

constexpr int kCheckThreads = 256;

__global__ void __launch_bounds__(kWave) check_clear_kernel(int32_t* status) {
  if (threadIdx.x == 0) status[0] = 0;
}

// Grid-stride over the lengths, the table cells and the (sequence, KV head)
// groups; a thread that finds a violation ORs its bits into the status word.
__global__ void __launch_bounds__(kCheckThreads) check_inputs_kernel(const CheckParams c) {
  const int64_t tid = (int64_t)blockIdx.x * kCheckThreads + threadIdx.x;
  const int64_t nthr = (int64_t)gridDim.x * kCheckThreads;
  const int64_t max_tok = (int64_t)c.max_pages * kPage;
  uint32_t bits = 0;

  // Lengths inside [0, max_pages * P].
  for (int64_t b = tid; b < c.B; b += nthr) {
    const int32_t ctx = c.ctx_lens[b];
    if (ctx < 0 || ctx > max_tok) bits |= KVPAGE_CHECK_LENGTH;
  }
  // The first ceil(ctx / P) entries of each row (ctx clamped) inside the pool.
  const int64_t cells = (int64_t)c.B * c.max_pages;
  for (int64_t i = tid; i < cells; i += nthr) {
    const int64_t b = i / c.max_pages;
    const int64_t pg = i - b * c.max_pages;
    if (pg * kPage < clamp_ctx(c.ctx_lens[b], c.max_pages)) {
      const int32_t id = c.block_tables[i];
      if (id < 0 || id >= c.num_pages) bits |= KVPAGE_CHECK_PAGE;
    }
  }
  // The queue kvpage_build_queue writes for the clamped lengths: group
  // (b, g) holds tasks [offsets[b*Hkv+g], offsets[b*Hkv+g+1]), ceil(ctx_b / S)
  // of them, the j-th covering tokens [j*S, min(ctx_b, (j+1)*S)); offsets
  // start at 0 and end at n_tasks <= capacity.
  if (c.tasks) {
    const int64_t groups = (int64_t)c.B * c.Hkv;
    const int64_t nt = c.n_tasks[0];
    const int64_t S = c.split_tokens;
    if (tid == 0 && (nt < 0 || nt > c.capacity || c.group_offsets[0] != 0 ||
                     c.group_offsets[groups] != nt))
      bits |= KVPAGE_CHECK_QUEUE;
    const int64_t limit = nt < c.capacity ? nt : c.capacity;
    for (int64_t q = tid; q < groups; q += nthr) {
      const int64_t b = q / c.Hkv;
      const int32_t g = (int32_t)(q - b * c.Hkv);
      const int64_t ctx = clamp_ctx(c.ctx_lens[b], c.max_pages);
      const int64_t ns = (ctx + S - 1) / S;
      const int64_t lo = c.group_offsets[q], hi = c.group_offsets[q + 1];
      if (hi - lo != ns || lo < 0 || hi > limit) {
        bits |= KVPAGE_CHECK_QUEUE;
        continue;
      }
      for (int64_t j = 0; j < ns; ++j) {
        const kvpage_task t = c.tasks[lo + j];
        const int64_t end = ctx < (j + 1) * S ? ctx : (j + 1) * S;
        if (t.seq != b || t.kv_head != g || t.tok_begin != j * S || t.tok_end != end) {
          bits |= KVPAGE_CHECK_QUEUE;
          break;
        }
      }
    }
  }
  if (bits) atomicOr(c.status, (int32_t)bits);
}

hipError_t launch_check_inputs(const kvpage_shape& s, const int32_t* ctx_lens,
                               const int32_t* block_tables, const kvpage_task* tasks,
                               const int32_t* group_offsets, const int32_t* n_tasks,
                               int32_t capacity, int32_t* status, hipStream_t stream) {
  hipLaunchKernelGGL(check_clear_kernel, dim3(1), dim3(kWave), 0, stream, status);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || s.B == 0) return err;
  CheckParams c;
  c.ctx_lens = ctx_lens;
  c.block_tables = block_tables;
  c.tasks = tasks;
  c.group_offsets = group_offsets;
  c.n_tasks = n_tasks;
  c.status = status;
  c.B = s.B;
  c.Hkv = s.Hkv;
  c.max_pages = s.max_pages;
  c.num_pages = s.num_pages;
  c.split_tokens = s.split_tokens;
  c.capacity = capacity;
  int64_t work = (int64_t)s.B * s.max_pages;
  if ((int64_t)s.B * s.Hkv > work) work = (int64_t)s.B * s.Hkv;
  int64_t blocks = (work + kCheckThreads - 1) / kCheckThreads;
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(check_inputs_kernel, dim3((unsigned)blocks), dim3(kCheckThreads), 0, stream, c);
  return hipGetLastError();
}

}  // namespace kvpage
