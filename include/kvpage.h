/*
 * kvpage.h -- C ABI of libkvpage.so: one decode step of paged grouped-query
 * attention (GQA) over a block-table KV cache, for AMD Instinct MI355X
 * (gfx950).
 *
 * What a step computes (sources are the web pages this library follows):
 *
 *   - "PersistentKV: Page-Aware Decode Scheduling for Long-Context LLM
 *     Serving on Commodity GPUs" (aissential.tech summary), Summary and
 *     Method: a native block-table decode attention for GQA that reuses each
 *     K/V tile across the query heads of a KV-head group, reads KV through
 *     per-sequence page tables, and runs a compact workqueue holding only
 *     non-empty (sequence, KV head, sequence split) tasks.
 *   - "GrowPage: On-Demand KV Budgeting for Efficient LLM Reasoning Serving"
 *     (mlsanity.com entry, Abstract; aitrending.vip article, Technical
 *     Details): page-level KV budgeting driven by dual-timescale query
 *     summaries.  The step therefore also emits per-page attention mass and,
 *     for a fast and a slow summary of each KV group's queries, the largest
 *     scaled summary-key dot product on every page.
 *
 * Around the step: kvpage_append_kv is the step before it (append one token
 * per sequence, taking a page from a free list at a page boundary),
 * kvpage_budget_decide turns the step's summary page maxima into GrowPage's
 * compress-or-acquire decision,
 * kvpage_choose_split is a host-side policy that picks the split size for a
 * batch's context lengths, and kvpage_check_inputs reports violated
 * preconditions of the integer inputs (debug checks).
 *
 * Problem statement and data layout (every tensor row-major, contiguous):
 *
 *   q            [B, Hq, d]                     f16 or bf16 (shape.dtype)
 *   k_pool       [num_pages, Hkv, d/8, P, 8]    same dtype; P = page_size; each
 *                                               (page, KV head) tile holds its
 *                                               P keys as 16-byte chunks, chunk
 *                                               c of every token together:
 *                                               element (page, g, c, s, x) is
 *                                               key element 8c + x of slot s
 *   v_pool       [num_pages, Hkv, P, d]         same dtype, row-major tiles
 *   block_tables int32 [B, max_pages]           logical page -> physical page
 *   ctx_lens     int32 [B]                      tokens attended by sequence b
 *   out          [B, Hq, d]                     q's dtype, round to nearest even
 *   lse          float32 [B, Hq]                natural-log sum of exp(scores)
 *
 * The K tile order is the one vLLM's PagedAttention uses for its key cache
 * (the head dimension split into 16-byte pieces outside the block's tokens):
 * a load of four chunk rows of a tile is 1 KiB of contiguous memory that
 * lands in the attention kernel's MFMA operand layout as it is, where a
 * row-major key tile needs 64-byte pieces of 16 rows per load (measured 7%
 * slower at one sequence of 32768 tokens, 8% on a batch of 8).
 *
 * Query head h reads KV head h / (Hq / Hkv).  Token t of sequence b is slot
 * t % P of physical page block_tables[b][t / P].  Scores are
 * scale * dot(q, k).  A sequence with ctx_lens[b] == 0 has no tasks; its out
 * rows are 0 and its lse is -inf.
 *
 * Ownership and threading: the caller owns every buffer and the stream.
 * Struct arguments (kvpage_shape, kvpage_budget) are HOST pointers read
 * during the call; every other pointer is a DEVICE pointer.  Calls enqueue
 * work on `stream` and return without synchronizing; the library never
 * allocates, frees or synchronizes and keeps no per-call state (only a
 * per-device count of resident workgroups, found on first use, and the static
 * device workspace of kvpage_decode_step_noalloc).  Calls that
 * may run at the same time (other streams) need their own queue, workspace
 * and output buffers; inputs may be shared.  Every call can be captured in
 * a HIP graph: it enqueues kernels only (no memset, copy or allocation).
 *
 * Alignment: q, k_pool, v_pool and the workspace must be 16-byte aligned,
 * out 8-byte aligned (vector loads and stores); anything else is
 * KVPAGE_ERR_INVALID_ARG.
 *
 * Errors: arguments are validated on the host before anything is enqueued;
 * a failed check returns a negative kvpage_status and enqueues nothing.  A
 * failed kernel launch returns KVPAGE_ERR_HIP.  Data-dependent preconditions
 * (0 <= ctx_lens[b] <= max_pages * P, 0 <= block-table entries < num_pages
 * for the pages a sequence uses, queue entries as kvpage_build_queue writes
 * them) are the caller's and are not reported, but every kernel clamps what
 * it reads into the shape: lengths to [0, max_pages * P], page ids to
 * [0, num_pages), queue entries to a sequence, a KV head and at most
 * split_tokens tokens inside the table row, task counts to `capacity`.  A
 * violation therefore gives wrong values for the rows it touches and never
 * an access outside the buffers described here.  (kvpage_append_kv checks
 * its page ids and lengths and reports them in its status word.)  A caller
 * who wants the violations reported runs kvpage_check_inputs, a separate
 * read-only pass that writes them to a device status word (debug checks).
 */
#ifndef KVPAGE_H
#define KVPAGE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVPAGE_OK = 0,
  KVPAGE_ERR_INVALID_ARG = -1, /* null pointer, inconsistent or out-of-range shape */
  KVPAGE_ERR_UNSUPPORTED = -2, /* valid shape the library has no kernel for       */
  KVPAGE_ERR_CAPACITY = -3,    /* task capacity below kvpage_queue_capacity()     */
  KVPAGE_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed       */
  KVPAGE_ERR_SCRATCH = -5      /* workspace larger than the library's static one  */
} kvpage_status;

typedef enum { KVPAGE_F16 = 0, KVPAGE_BF16 = 1 } kvpage_dtype;

/* One queue entry: tokens [tok_begin, tok_end) of KV head kv_head of sequence
 * seq (PersistentKV summary, Method: row/sequence, KV head, split tasks). */
typedef struct {
  int32_t seq, kv_head, tok_begin, tok_end;
} kvpage_task;

/* Shape flags.
 *   KVPAGE_FLAG_STREAM_KV  the caller promises that no K/V page is referenced
 *       by more than one sequence in the call (no prefix sharing).  The
 *       attention kernel then marks its K/V tile loads non-temporal so they
 *       stream past the caches.  It changes no result, only speed: 2-7%
 *       faster when the step has at least about one task per wavefront of
 *       the GPU (Hkv * sum_b ceil(ctx_b / split_tokens) >= 4 per compute
 *       unit, which kvpage_choose_split aims for), ~6% slower on shorter
 *       steps.  Leave it clear when block tables share pages: shared pages
 *       are then served from cache (15% faster on a batch of 64 sequences
 *       sharing 128 prefix pages than with the flag set). */
#define KVPAGE_FLAG_STREAM_KV 1u

/* Problem shape.  Supported by the kernels: page_size == 16; d in {64, 128};
 * 1 <= Hq / Hkv <= 8; split_tokens a multiple of page_size in [16, 256]
 * or a multiple of 256 in [512, 4096] (run as consecutive 16-page pieces);
 * dtype f16 or bf16; scale finite and > 0.  flags: 0 or
 * KVPAGE_FLAG_STREAM_KV (any other bit is KVPAGE_ERR_INVALID_ARG). */
typedef struct {
  int32_t B, Hq, Hkv, d, page_size, split_tokens, max_pages, num_pages;
  int32_t dtype; /* kvpage_dtype */
  float scale;   /* usually 1/sqrt(d) */
  uint32_t flags;
} kvpage_shape;

/* Budgeting outputs (GrowPage, Abstract: dual-timescale query summaries and
 * page-level budgeting).  All device pointers, float32, none may be NULL.
 *   page_mass [B, Hq, max_pages]  softmax weight of each logical page; 0 past
 *                                 the sequence's last page
 *   s_prev    [2, B, Hkv, d]      summaries before this step (0 fast, 1 slow)
 *   s_next    [2, B, Hkv, d]      s <- (1 - a) s + a * mean_h(q); must not
 *                                 overlap s_prev (swap the two between steps)
 *   page_max  [2, B, Hkv, max_pages]  max over a page's keys of
 *                                 scale * dot(s_next, k); -inf past the last page
 * alpha_fast / alpha_slow in [0, 1] (0.5 and 0.05 in the reference workload). */
typedef struct {
  float* page_mass;
  const float* s_prev;
  float* s_next;
  float alpha_fast, alpha_slow;
  float* page_max;
} kvpage_budget;

/* Task capacity for `shape`: B * Hkv * ceil(max_pages * page_size /
 * split_tokens), the most tasks any ctx_lens within max_pages can produce.
 * Returns a negative kvpage_status for an invalid shape. */
int32_t kvpage_queue_capacity(const kvpage_shape* shape);

/* Bytes of device workspace kvpage_split_attn / kvpage_merge_splits /
 * kvpage_page_mass / kvpage_decode_step need for `capacity` tasks: the split
 * partials (an unnormalised output row, a reference max and a sum of
 * exponentials per query head for each run of consecutive tasks of one
 * (sequence, KV head) that a wavefront processed) and a small header.  It
 * does not depend on budgeting: raw page sums and page maxima go straight
 * into the caller's page_mass / page_max buffers.  Negative kvpage_status on
 * error. */
int64_t kvpage_workspace_bytes(const kvpage_shape* shape, int32_t capacity);

/* Build the compact task queue (PersistentKV summary, Summary: only
 * non-empty tasks).  For b in order, KV head g in order, split j in order:
 * one task {b, g, j*S, min(ctx_b, (j+1)*S)} for each j < ceil(ctx_b / S),
 * S = split_tokens.  Writes tasks[0 .. n), group_offsets[b*Hkv + g] = index
 * of the first task of (b, g), group_offsets[B*Hkv] = n, and n_tasks[0] = n.
 * tasks: [capacity]; group_offsets: [B*Hkv + 1]; n_tasks: [1]; all device. */
int kvpage_build_queue(const kvpage_shape* shape, const int32_t* ctx_lens, kvpage_task* tasks,
                       int32_t capacity, int32_t* group_offsets, int32_t* n_tasks,
                       hipStream_t stream);

/* Split attention (PersistentKV summary, Summary/Method: per KV-head group,
 * each K/V page tile serves all Hq/Hkv query heads).  For the queued tasks
 * writes into `workspace` the split partials of each of the group's query
 * heads (one per run of consecutive tasks a wavefront processed): reference
 * max, sum of exponentials and the unnormalised weighted V row.  With
 * `budget` non-NULL it also writes, for the tasks' pages, page_mass relative
 * to the reference max of the run holding the page (finished by
 * kvpage_page_mass) and the final summary page_max.  budget may be NULL. */
int kvpage_split_attn(const kvpage_shape* shape, const void* q, const void* k_pool,
                      const void* v_pool, const int32_t* block_tables, const int32_t* ctx_lens,
                      const kvpage_task* tasks, const int32_t* n_tasks, int32_t capacity,
                      void* workspace, const kvpage_budget* budget, hipStream_t stream);

/* Log-sum-exp merge of the split partials of each (sequence, query head),
 * over its group's task range in split order: out = sum_j w_j o_j / sum_j w_j
 * l_j with w_j = exp(m_j - max m), lse = max m + ln(sum_j w_j l_j).  The
 * pages do not give the merge; splitting a sequence's tokens into tasks
 * (PersistentKV summary, Method: sequence-split tasks) needs one, and this is
 * the standard flash-decoding log-sum-exp combination, which gives the
 * softmax over the whole context up to rounding.  out: [B, Hq, d] in q's
 * dtype; lse: float32 [B, Hq]; group_offsets as kvpage_build_queue wrote
 * them; workspace as kvpage_split_attn left it. */
int kvpage_merge_splits(const kvpage_shape* shape, const int32_t* group_offsets, int32_t capacity,
                        const void* workspace, void* out, float* lse, hipStream_t stream);

/* Decode attention over the queued tasks (PersistentKV summary, Summary:
 * block-table decode attention for GQA, K/V tiles shared by the query heads
 * of a KV-head group; Method: sequence-split tasks):
 * kvpage_split_attn followed by kvpage_merge_splits on the same stream.
 * Arguments as for those two calls; with `budget` the page values are left
 * for kvpage_page_mass to finish. */
int kvpage_decode_attn(const kvpage_shape* shape, const void* q, const void* k_pool,
                       const void* v_pool, const int32_t* block_tables, const int32_t* ctx_lens,
                       const kvpage_task* tasks, const int32_t* group_offsets,
                       const int32_t* n_tasks, int32_t capacity, void* workspace,
                       const kvpage_budget* budget, void* out, float* lse, hipStream_t stream);

/* Optional launch settings for kvpage_decode_step.
 *   attn_start / attn_stop: events the split-attention kernel's own dispatch
 *     records at its start and end (NULL: none).
 *   max_workgroups: cap on the attention kernel's persistent grid (0: as many
 *     as are resident on the device).  Fewer workgroups give each wavefront a
 *     longer contiguous stretch of the queue, which it folds into fewer run
 *     partials: results agree to rounding whatever the cap, the bits of out,
 *     lse and page mass depend on it.
 *   shared_pages: NULL, or DEVICE int32 [B]: the first shared_pages[b] logical
 *     pages of sequence b's table row may also be referenced by other
 *     sequences (a shared prompt prefix, as prefix caching keeps it; GrowPage,
 *     mlsanity.com entry, Abstract: budgeting that keeps prefix caching).
 *     Used only with KVPAGE_FLAG_STREAM_KV, whose promise it narrows: no page
 *     outside those leading pages is referenced twice.  Pieces of work (up to
 *     16 pages) that start on a shared page then load through the caches, so
 *     a shared page read by several sequences is served from cache, and the
 *     rest stream.  It changes no result, only speed (B64 with 128 shared
 *     prefix pages: 6% faster than all loads cached). */
typedef struct {
  hipEvent_t attn_start, attn_stop;
  int32_t max_workgroups;
  const int32_t* shared_pages;
} kvpage_launch_opts;

/* One whole decode step in one call, on `stream`: the queue build (as
 * kvpage_build_queue), split attention (as kvpage_split_attn) and the merge
 * (as kvpage_merge_splits); with `budget` the merge also finishes the
 * budgeting outputs exactly as kvpage_page_mass would, in the same kernel.
 * Outputs equal those of kvpage_build_queue + kvpage_decode_attn (+
 * kvpage_page_mass): the queue, page maxima and summaries bit for bit; out,
 * lse and page mass bit for bit as well when B == 1, B > 64 or Hkv is not a
 * multiple of 8, and to rounding otherwise (there the attention kernel runs
 * each KV head's tasks on one XCD and so folds them into different runs).
 * Repeated calls with the same inputs and opts give the same bits.
 * tasks, group_offsets and n_tasks are written.  opts may be NULL. */
int kvpage_decode_step(const kvpage_shape* shape, const void* q, const void* k_pool,
                       const void* v_pool, const int32_t* block_tables, const int32_t* ctx_lens,
                       kvpage_task* tasks, int32_t* group_offsets, int32_t* n_tasks,
                       int32_t capacity, void* workspace, const kvpage_budget* budget, void* out,
                       float* lse, const kvpage_launch_opts* opts, hipStream_t stream);

/* Bytes of the static device workspace of kvpage_decode_step_noalloc. */
#define KVPAGE_NOALLOC_WORKSPACE_BYTES (64u << 20)

/* kvpage_decode_step for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same kernels, with the workspace taken from a static
 * device array of KVPAGE_NOALLOC_WORKSPACE_BYTES (64 MiB) that the library
 * holds on every device it runs on until the process ends; the caller still
 * passes inputs, queue and outputs.  Arguments are those of
 * kvpage_decode_step without `workspace`; outputs are bit for bit those of
 * kvpage_decode_step.  The workspace is the current device's (the stream
 * must belong to it).  Nothing in it has to start at zero, so nothing is
 * cleared; every call on a device shares that device's array and leaves it
 * holding the last call's split partials, so calls that may overlap on one
 * device (other streams, other threads) race and must be serialised by the
 * caller.  Returns KVPAGE_ERR_SCRATCH, enqueueing nothing, when
 * kvpage_workspace_bytes(shape, capacity) exceeds the static size (for
 * example B = 1, Hq = 32, Hkv = 8, d = 128, 2048 pages of 16 tokens, split
 * 256: 2.1 MB; 8 sequences of up to 65536 tokens at split 256: 34 MB).  The
 * call allocates and frees nothing; its first call on a device looks up that
 * device's address of the array (hipGetSymbolAddress). */
int kvpage_decode_step_noalloc(const kvpage_shape* shape, const void* q, const void* k_pool,
                               const void* v_pool, const int32_t* block_tables,
                               const int32_t* ctx_lens, kvpage_task* tasks,
                               int32_t* group_offsets, int32_t* n_tasks, int32_t capacity,
                               const kvpage_budget* budget, void* out, float* lse,
                               const kvpage_launch_opts* opts, hipStream_t stream);

/* Finish the budgeting outputs (GrowPage, mlsanity.com entry, Abstract:
 * page-level KV budgeting driven by dual-timescale query summaries;
 * aitrending.vip article, Technical Details) after kvpage_decode_attn ran
 * with the same budget, queue and workspace: page_mass[b,h,p] becomes the
 * softmax weight of page p (using the merged lse), entries past each
 * sequence's last page are set (mass 0, page_max -inf), and s_next is
 * written for every (b, g), including sequences with no tokens.  The page
 * values are addressed by logical page: page p of (b, g) lies in the task
 * group_offsets[b*Hkv + g] + p*P/split_tokens, whose run the workspace
 * header locates, so the queue itself is not read; `capacity` is the one the
 * workspace was laid out for.  lse: float32 [B, Hq] as the merge wrote it;
 * q: [B, Hq, d]; ctx_lens: [B]. */
int kvpage_page_mass(const kvpage_shape* shape, const kvpage_budget* budget, const void* q,
                     const float* lse, const int32_t* ctx_lens, const int32_t* group_offsets,
                     int32_t capacity, const void* workspace, hipStream_t stream);

/* Test support (PersistentKV summary, Summary: native page tables): the pool
 * element offsets each queued task reads for each of its tokens.  They are
 * built from kvpage_split_attn's own addressing: the (page, KV head) tile
 * offset, then the place the kernel's K and V lane maps load for the
 * token's slot, after checking that those lanes' pieces lie at that slot's
 * places and cover its d elements exactly once (else -2).  Which lane holds
 * which piece of a token is checked only by that coverage test and by the
 * outputs.
 * offsets: int64 [capacity, split_tokens, 2]; entry (i, j) holds, for token
 * tok_begin + j of task i, the element offset of its first key element in
 * k_pool ([0], chunk 0 of its slot) and of its value row in v_pool ([1]), or
 * -1, -1 past tok_end.  Rows >= n_tasks untouched. */
int kvpage_debug_gather_offsets(const kvpage_shape* shape, const int32_t* block_tables,
                                const kvpage_task* tasks, const int32_t* n_tasks,
                                int32_t capacity, int64_t* offsets, hipStream_t stream);

/* Split size for one decode step, chosen per workload (PersistentKV
 * summary, Summary: its throughput gains come from a policy that picks the
 * decode configuration for each workload).  Candidates: S in {4096, 2048,
 * ..., 32, 16} tokens with KVPAGE_FLAG_STREAM_KV in shape.flags, {256, ...,
 * 16} without (pages that may be shared are then read by wavefronts running
 * side by side close together in time, from cache: on a batch sharing a
 * prefix, 256 ran 1.7% faster than 1024).  Only splits whose queue holds at
 * least one task per resident wavefront of the attention kernel
 * (Hkv * sum_b ceil(ctx_b / S) >= wavefronts) qualify.  Each is priced by
 * simulating the kernel's schedule (per-XCD classes of KV heads where the
 * kernel uses them; chunks of positions, at most 16 / ceil(S / 256) per
 * chunk): every wavefront's pages plus a fixed cost per queue position
 * (measured: half a page with streaming loads, one and a half cached), then
 * the time to finish when each unfinished wavefront streams at
 * min(1.43, wavefronts / unfinished) times its equal share of HBM (water
 * filling: the kernel is bound by HBM, and a wavefront streams up to ~1.4-1.8x
 * faster once others have finished).  Returns the cheapest, ties to the
 * longer split; the page size (16) if no split fills the wavefronts, 256 if
 * every context is empty.  Measured on MI355X against 256: 4 long + 4 short
 * sequences 1024 (2.3% faster attention), Zipf lengths 2048 (4.1%), 4
 * bimodal sequences 1024 (2.8%); one 32768-token sequence keeps 256 (512
 * leaves half the wavefronts idle: 26% slower), and so do 64 sequences of
 * 2-14K private tokens (1024: 6.8% slower, many wavefronts with six 64-page
 * tasks).  Host cost: ~0.1 ms per call.
 *   shape: B, Hq, Hkv, d, page_size, max_pages, num_pages, dtype, scale and
 *     flags as for the other calls: KVPAGE_FLAG_STREAM_KV set only when no
 *     page is shared at all.  A step that names shared leading pages
 *     (kvpage_launch_opts.shared_pages) still shares them: ask with the flag
 *     clear (B64 with a shared prefix and shared_pages: 256 tokens 4.4%
 *     faster than 1024).  split_tokens is ignored.
 *   ctx_lens_host: HOST array of B context lengths, each in [0, max_pages *
 *     page_size].
 *   wavefronts: resident wavefronts to fill; <= 0 queries the current device
 *     (4 per compute unit).
 * Returns the split in tokens, or a negative kvpage_status (KVPAGE_ERR_HIP
 * if the device query fails).  Enqueues nothing. */
int32_t kvpage_choose_split(const kvpage_shape* shape, const int32_t* ctx_lens_host,
                            int32_t wavefronts);

/* Status bits kvpage_check_inputs writes to its device status word. */
enum {
  KVPAGE_CHECK_LENGTH = 1,   /* a length outside [0, max_pages * page_size] */
  KVPAGE_CHECK_PAGE = 2,     /* a block-table entry a sequence uses outside [0, num_pages) */
  KVPAGE_CHECK_QUEUE = 4     /* the queue differs from the one kvpage_build_queue writes */
};

/* Debug checks of the data-dependent preconditions that the other calls
 * assume and do not report (they clamp instead; see Errors above).  A
 * read-only pass, separate from the decode kernels, for a caller who wants
 * violations reported:
 *   KVPAGE_CHECK_LENGTH: some ctx_lens[b] outside [0, max_pages * page_size];
 *   KVPAGE_CHECK_PAGE: some block_tables[b, p] with p * page_size < ctx_b
 *     (ctx_b clamped into that range) outside [0, num_pages);
 *   KVPAGE_CHECK_QUEUE (only when tasks, group_offsets and n_tasks are
 *     given): *n_tasks, group_offsets or one of the first *n_tasks entries of
 *     tasks differs from what kvpage_build_queue writes for the clamped
 *     lengths, or *n_tasks lies outside [0, capacity].
 *   ctx_lens: [B] int32; block_tables: [B, max_pages] int32; tasks:
 *     [capacity] kvpage_task; group_offsets: [B * Hkv + 1] int32; n_tasks:
 *     one int32; all device.  tasks, group_offsets and n_tasks are either
 *     all NULL or all given; capacity is then checked as for
 *     kvpage_build_queue.
 *   status: one int32, device, written with the KVPAGE_CHECK_* bits found
 *     (0 when every check passes).  The call enqueues two kernels (one clears
 *     the word, one checks) and reads nothing else.
 * shape: B, Hkv, page_size, split_tokens, max_pages and num_pages are used;
 * the other fields are checked as for the other calls.  Negative
 * kvpage_status on invalid arguments (nothing enqueued). */
int kvpage_check_inputs(const kvpage_shape* shape, const int32_t* ctx_lens,
                        const int32_t* block_tables, const kvpage_task* tasks,
                        const int32_t* group_offsets, const int32_t* n_tasks, int32_t capacity,
                        int32_t* status, hipStream_t stream);

/* Status bits kvpage_append_kv writes to its device status word. */
enum {
  KVPAGE_APPEND_FULL = 1,      /* a sequence's block-table row had no room left */
  KVPAGE_APPEND_NO_PAGE = 2,   /* the free list ran out */
  KVPAGE_APPEND_BAD_PAGE = 4   /* a page id outside [0, num_pages) in the free list or a table */
};

/* Append one token per sequence to the paged cache, the step before decode
 * attention (GrowPage, aitrending.vip article, Technical Details: a physical
 * page is acquired at a capacity boundary; "Elastic KV Cache for LLM
 * Serving", 2 Background and Motivation: fixed-size KV blocks handed out from
 * an integer free list).  For sequence b, in order, with t = ctx_lens[b]:
 *   t == max_pages * page_size: nothing changes for b (KVPAGE_APPEND_FULL);
 *   t % page_size == 0: b needs a page.  The k-th such sequence takes
 *     free_pages[*free_count - 1 - k] (the top of the stack) and records it in
 *     block_tables[b, t / page_size]; if k >= *free_count nothing changes for
 *     b (KVPAGE_APPEND_NO_PAGE);
 *   otherwise its page is block_tables[b, t / page_size].
 * A page id outside [0, num_pages) leaves b unchanged (a free-list entry it
 * came from is still used up; KVPAGE_APPEND_BAD_PAGE).  Then k_new[b, g, :]
 * and v_new[b, g, :] go to slot t % page_size of that page for every KV head
 * g (in the pools' layouts: the key as d/8 chunks of the chunk-major tile,
 * the value as one row), and ctx_lens_out[b] = t + 1 (t when b was left
 * unchanged).
 *   k_new, v_new: [B, Hkv, d] in the pools' dtype, device.
 *   k_pool, v_pool, block_tables: updated in place, device.
 *   ctx_lens (read) and ctx_lens_out (written): [B] int32, device, must not
 *     overlap.  Lengths must lie in [0, max_pages * page_size].
 *   free_pages: [*free_count] int32, device; free_count (read) and
 *     free_count_out (written, = free_count minus the pages taken): one int32
 *     each, device, must not overlap.
 *   status: one int32, device, written with the KVPAGE_APPEND_* bits (0 when
 *     every sequence was appended).
 * shape: B, Hkv, d, page_size, max_pages, num_pages and dtype are used; the
 * other fields are checked as for the other calls.  Negative kvpage_status on
 * invalid arguments (nothing enqueued). */
int kvpage_append_kv(const kvpage_shape* shape, const void* k_new, const void* v_new,
                     void* k_pool, void* v_pool, int32_t* block_tables, const int32_t* ctx_lens,
                     int32_t* ctx_lens_out, const int32_t* free_pages, const int32_t* free_count,
                     int32_t* free_count_out, int32_t* status, hipStream_t stream);

/* Decisions kvpage_budget_decide writes. */
enum {
  KVPAGE_DECIDE_NONE = 0,      /* not at a capacity boundary                      */
  KVPAGE_DECIDE_ACQUIRE = 1,   /* take one more physical page                     */
  KVPAGE_DECIDE_COMPRESS = 2   /* stay within the allocation; compress `victim`   */
};

/* GrowPage's budgeting decision (mlsanity.com entry, Abstract: the fast and
 * slow query summaries' relative attention working sets estimate how demand
 * evolves, and at each capacity boundary the system compresses KV within the
 * current allocation or acquires another physical page when broader demand
 * emerges; aitrending.vip article, Technical Details, on-demand page
 * allocation).  The pages give no formula; this call computes, from the
 * summary page maxima a budgeting decode step wrote:
 *   working set of (summary k, sequence b, KV head g): with x_p =
 *     page_max[k, b, g, p] for the sequence's pages p < ceil(ctx_b / P) and
 *     page weights softmax(x), every page with x_p >= L, L the highest score
 *     level whose pages scoring >= L hold at least tau of the weight (the
 *     smallest top set covering tau; equal scores enter together).
 *     ws_size[k, b, g] = its page count, ws_level[k, b, g] = L (+inf and 0
 *     pages for an empty sequence);
 *   F, S: the unions over KV heads of the fast (k = 0) and slow (k = 1) sets;
 *     ws_union[0, b] = |F|, ws_union[1, b] = |S|;
 *   decision[b]: KVPAGE_DECIDE_NONE unless ctx_b > 0 and ctx_b % P == 0 (the
 *     last page is full: a capacity boundary); there KVPAGE_DECIDE_ACQUIRE
 *     when |F| > |S| or every page lies in F or S, else
 *     KVPAGE_DECIDE_COMPRESS with victim[b] = the page outside F and S whose
 *     largest slow score over the KV heads is lowest (ties: the lowest page);
 *     victim[b] = -1 otherwise.
 * The weights are float32 exponentials summed exactly in 40-bit fixed point,
 * so a set can differ from the exact one only where the exact covered
 * fraction at its closing level lies within about 1e-5 of tau.
 *   page_max: float32 [2, B, Hkv, max_pages], finite or -inf on each
 *     sequence's pages (as the decode step writes it); ctx_lens: [B];
 *   ws_size: int32 [2, B, Hkv]; ws_level: float32 [2, B, Hkv]; ws_union:
 *     int32 [2, B]; decision, victim: int32 [B]; all device.
 *   tau in (0, 1].
 * shape: B, Hkv, page_size (16), max_pages (at most 2^23) are used; the
 * other fields are checked as for the other calls.  Two kernels; negative
 * kvpage_status on invalid arguments (nothing enqueued). */
int kvpage_budget_decide(const kvpage_shape* shape, const float* page_max, const int32_t* ctx_lens,
                         float tau, int32_t* ws_size, float* ws_level, int32_t* ws_union,
                         int32_t* decision, int32_t* victim, hipStream_t stream);

/* Static description of a status code. */
const char* kvpage_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* KVPAGE_H */
