// KV append with page acquisition: the step before decode attention.
//
// Each sequence's new token goes to slot ctx % 16 of its last page; a
// sequence at a page boundary first takes a physical page from the pool's
// integer free list (GrowPage, aitrending.vip article, Technical Details: a
// page is acquired at a capacity boundary; "Elastic KV Cache for LLM
// Serving", 2 Background and Motivation: fixed-size KV blocks handed out
// from an integer free list).  Pages go out in sequence order from the top of
// the list, so the result does not depend on scheduling.
#include "kvpage_common.h"

namespace kvpage {

struct AppendParams {
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_pool;
  uint16_t* v_pool;
  int32_t* block_tables;
  const int32_t* ctx_in;
  int32_t* ctx_out;
  const int32_t* free_pages;
  const int32_t* free_count_in;
  int32_t* free_count_out;
  int32_t* status;
  int32_t B, Hkv, d, max_pages, num_pages;
};

// The page sequence i writes to: a free-list entry if it starts a page (k =
// sequences before it that start one), else its table entry.  -1: none (row
// full or free list exhausted).
__device__ __forceinline__ int page_of(const AppendParams& p, int i, int t, int k, int fc,
                                       int max_ctx) {
  if (t < 0 || t >= max_ctx) return -1;
  if (t % kPage == 0) return k < fc ? p.free_pages[fc - 1 - k] : -1;
  return p.block_tables[(int64_t)i * p.max_pages + t / kPage];
}

// One wavefront per sequence.  It counts the sequences before it that need a
// page (a ballot per 64 lengths), which fixes the free-list entry it takes.
// Sequence 0's wavefront goes over every sequence: it writes the new free
// count and the status word (row full, free list exhausted, page id outside
// the pool).  The lengths are read from ctx_in and written to ctx_out, so no
// wavefront sees another's update.  The buffers of the first loads (lengths,
// free count), B and max_pages come first as arguments of their own, which
// gfx950 can preload into SGPRs at wave launch.
__global__ void __launch_bounds__(kWave) append_kernel(const int32_t* lead_ctx,
                                                       const int32_t* lead_fc, int32_t lead_b,
                                                       int32_t lead_max_pages,
                                                       const AppendParams p) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int max_ctx = lead_max_pages * kPage;
  const int fc = lead_fc[0];
  const int scan_end = b == 0 ? lead_b : b;
  int before = 0;   // sequences before b needing a page (all of them, for b = 0)
  int flags = 0;
  for (int base = 0; base < scan_end; base += kWave) {
    const int i = base + lane;
    const int t = i < lead_b ? lead_ctx[i] : 0;
    const bool need = i < lead_b && t >= 0 && t < max_ctx && t % kPage == 0;
    const uint64_t m = __builtin_amdgcn_ballot_w64(need);
    if (b == 0) {
      const int k = before + (int)__builtin_amdgcn_mbcnt_hi(
          (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      const int pg = i < lead_b ? page_of(p, i, t, k, fc, max_ctx) : 0;
      const bool full = i < lead_b && (t < 0 || t >= max_ctx);
      const bool starved = need && k >= fc;
      const bool bad = i < lead_b && !full && !starved && (pg < 0 || pg >= p.num_pages);
      if (__builtin_amdgcn_ballot_w64(full)) flags |= KVPAGE_APPEND_FULL;
      if (__builtin_amdgcn_ballot_w64(starved)) flags |= KVPAGE_APPEND_NO_PAGE;
      if (__builtin_amdgcn_ballot_w64(bad)) flags |= KVPAGE_APPEND_BAD_PAGE;
      before += __builtin_popcountll(m);
    } else {
      const int below = b - base;   // lanes of this chunk before sequence b
      const uint64_t mask = below >= kWave ? ~0ull : (1ull << below) - 1;
      before += __builtin_popcountll(m & mask);
    }
  }
  if (b == 0) {
    if (lane == 0) {
      p.free_count_out[0] = fc - min(before, fc);
      p.status[0] = flags;
    }
    before = 0;
  }
  const int t = lead_ctx[b];
  const int page = page_of(p, b, t, before, fc, max_ctx);
  const bool ok = page >= 0 && page < p.num_pages;
  if (ok) {
    if (t % kPage == 0 && lane == 0) p.block_tables[(int64_t)b * p.max_pages + t / kPage] = page;
    const int n = p.Hkv * p.d;   // halves of one token, all KV heads
    const int slot = t % kPage;
    for (int x = 8 * lane; x < n; x += 8 * kWave) {   // one 16-byte chunk each
      const int g = x / p.d;
      const int i = x - g * p.d;
      const int64_t tile = (int64_t)(page * p.Hkv + g) * kPage * p.d;
      const int64_t src = (int64_t)b * n + x;
      // V rows are row-major in the tile, K chunk-major ([d/8][16][8]).
      *reinterpret_cast<uint4*>(p.k_pool + tile + ((i / 8) * kPage + slot) * 8) =
          *reinterpret_cast<const uint4*>(p.k_new + src);
      *reinterpret_cast<uint4*>(p.v_pool + tile + slot * p.d + i) =
          *reinterpret_cast<const uint4*>(p.v_new + src);
    }
  }
  if (lane == 0) p.ctx_out[b] = ok ? t + 1 : t;
}

hipError_t launch_append(const kvpage_shape& s, const void* k_new, const void* v_new,
                         void* k_pool, void* v_pool, int32_t* block_tables,
                         const int32_t* ctx_in, int32_t* ctx_out, const int32_t* free_pages,
                         const int32_t* free_count_in, int32_t* free_count_out,
                         int32_t* status, hipStream_t stream) {
  if (s.B <= 0) return hipSuccess;
  AppendParams p;
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  p.k_pool = static_cast<uint16_t*>(k_pool);
  p.v_pool = static_cast<uint16_t*>(v_pool);
  p.block_tables = block_tables;
  p.ctx_in = ctx_in;
  p.ctx_out = ctx_out;
  p.free_pages = free_pages;
  p.free_count_in = free_count_in;
  p.free_count_out = free_count_out;
  p.status = status;
  p.B = s.B;
  p.Hkv = s.Hkv;
  p.d = s.d;
  p.max_pages = s.max_pages;
  p.num_pages = s.num_pages;
  hipLaunchKernelGGL(append_kernel, dim3(s.B), dim3(kWave), 0, stream, p.ctx_in, p.free_count_in,
                     p.B, p.max_pages, p);
  return hipGetLastError();
}

}  // namespace kvpage
