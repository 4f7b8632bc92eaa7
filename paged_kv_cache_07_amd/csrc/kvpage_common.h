// Device-side helpers shared by the kvpage kernels (gfx950 / CDNA4).
//
// Addressing follows the paged layout of the PersistentKV summary
// (aissential.tech, Summary: native page tables): one (page, KV head) tile
// of P tokens is P*d contiguous elements of the K pool and of the V pool.
// Inside a tile, V is row-major [P][d]; K is chunk-major [d/8][P][8] (the
// token's d elements as 16-byte chunks, chunk c of all P tokens together),
// so that one 64-lane load of four chunk rows is 1 KiB of contiguous memory
// and lands in the 16x16x32 MFMA operand layout as it is.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvpage.h"

// No product is fused into a following sum anywhere after this point (in
// every source that includes this header): each multiply and add rounds on
// its own, explicit fmaf excepted, so two instances of one kernel (or two
// copies of a body inside one) compute the same bits.
#pragma clang fp contract(off)

namespace kvpage {

// Separately rounded float operations (HIP's __fadd_rn and friends are plain
// operators compiled where they are defined, which lets them fuse).
__device__ __forceinline__ float add_rn(float a, float b) { return a + b; }
__device__ __forceinline__ float sub_rn(float a, float b) { return a - b; }
__device__ __forceinline__ float mul_rn(float a, float b) { return a * b; }

constexpr int kPage = 16;   // tokens per page: the M dimension of a 16x16 MFMA tile
constexpr int kWave = 64;   // CDNA wavefront width

// Element offset of the first element of the (physical page, KV head) tile.
__device__ __forceinline__ int64_t tile_offset(int32_t page, int32_t kv_head, int32_t Hkv,
                                               int32_t d) {
  return ((int64_t)page * Hkv + kv_head) * (int64_t)(kPage * d);
}

// Lane maps of the attention kernel's tile loads (byte offsets inside one
// (page, KV head) tile).  A wavefront's lane is (n, r) = (lane % 16, lane /
// 16).
//   K: for 16x16x32 MFMA block kb, lane (n, r) loads chunk 4 * kb + r (d
//      elements 8 * (4 * kb + r) .. + 8) of token n: the MFMA's row operand
//      (row = token); the 64 lanes read chunks 4kb .. 4kb+3 of all 16 tokens,
//      1 KiB contiguous in the chunk-major K tile.
//   V: for row group e, lane (n, r) loads token 4 * r + e, elements n * D / 16
//      .. + D / 16: whole rows per 16 lanes.
__host__ __device__ inline uint32_t k_piece_offset(int kb, int n, int r, int D) {
  (void)D;
  return (uint32_t)(((4 * kb + r) * kPage + n) * 8) * 2u;
}
__host__ __device__ inline uint32_t v_piece_offset(int e, int n, int r, int D) {
  return (uint32_t)((4 * r + e) * D + n * (D / 16)) * 2u;
}

// Lengths and page ids come from the caller's device data.  Every kernel
// clamps them into the shape (a length to [0, max_pages * P], a page id to
// [0, num_pages)), so a violated precondition gives wrong values for that
// sequence but no access outside the given buffers.
__device__ __forceinline__ int32_t clamp_ctx(int32_t ctx, int32_t max_pages) {
  return min(max(ctx, 0), max_pages * kPage);
}
__device__ __forceinline__ int32_t clamp_page(int32_t page, int32_t num_pages) {
  return min(max(page, 0), num_pages - 1);
}

// Unsigned division by a divisor fixed for a launch, as a multiply-high and
// two shifts (Granlund and Montgomery, "Division by Invariant Integers using
// Multiplication", PLDI 1994, section 4, the round-up method for 32-bit
// words): with l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1,
// t = mulhi(m, n) gives n / d = (t + ((n - t) >> min(l, 1))) >> max(l - 1, 0)
// for every 32-bit n.
struct DivMagic {
  uint32_t m, s1, s2;
};

inline DivMagic div_magic(uint32_t d) {   // d >= 1
  uint32_t l = 0;
  while (((uint64_t)1 << l) < d) ++l;
  DivMagic r;
  r.m = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d + 1);
  r.s1 = l < 1 ? l : 1;
  r.s2 = l > 1 ? l - 1 : 0;
  return r;
}

__device__ __forceinline__ uint32_t div_by(uint32_t n, DivMagic dm) {
  const uint32_t t = __umulhi(dm.m, n);
  return (t + ((n - t) >> dm.s1)) >> dm.s2;
}

// Group-mean query component: heads summed in head order, then scaled by
// 1/G.  Used by the attention kernel (summary dot products) and by the
// page-mass kernel (s_next), so both see identical bits.
template <typename LoadQ>
__device__ __forceinline__ float group_mean(LoadQ load_q, int G, float inv_g) {
  float s = load_q(0);
  for (int h = 1; h < G; ++h) s = add_rn(s, load_q(h));
  return mul_rn(s, inv_g);
}

// One exponential-moving-average step of a query summary (GrowPage:
// dual-timescale query summaries): s <- (1 - a) * s + a * qbar, rounded
// step by step (no contraction) so that every kernel agrees bitwise.
__device__ __forceinline__ float ema_step(float s_prev, float qbar, float a) {
  return add_rn(mul_rn(sub_rn(1.0f, a), s_prev), mul_rn(a, qbar));
}

// Workspace.  A header word holds the chunk length c the attention kernel
// used: the queue was cut into chunks [k*c, (k+1)*c), each run by one
// wavefront, which folded consecutive tasks of one (sequence, KV head) into a
// single partial stored at the position of the run's first task (a chunk
// start or a group's first task).  For capacity C tasks and G heads:
//   hdr [64]         int32, hdr[0] = c
//   o   [C][G][D]    float, unnormalised run partial (valid at run starts)
//   rm  [C][G]       float, run reference max (log2 domain); the raw page
//                    sums of the run's pages are relative to it as well
//   rl  [C][G]       float, run sum of exp2(score - rm)
struct WorkspaceView {
  int32_t* hdr;
  float* o;
  float* rm;
  float* rl;
};

constexpr int kWsHeaderWords = 64;

__host__ __device__ inline WorkspaceView ws_view(void* base, int64_t cap, int G, int D) {
  WorkspaceView w;
  w.hdr = reinterpret_cast<int32_t*>(base);
  w.o = reinterpret_cast<float*>(base) + kWsHeaderWords;
  w.rm = w.o + (size_t)cap * G * D;
  w.rl = w.rm + (size_t)cap * G;
  return w;
}

__host__ __device__ inline size_t ws_bytes(int64_t cap, int G, int D) {
  return (kWsHeaderWords + (size_t)cap * G * (D + 2)) * sizeof(float);
}

// Queue positions of the run partials of one (sequence, KV head) whose tasks
// are [lo, hi): lo, then lo + k for every k > 0 with (k + off) % c == 0,
// where c is the run length (chunk size of the attention kernel's schedule)
// and off the position of lo inside its chunk.
__host__ __device__ inline int run_count(int lo, int hi, int c, int off) {
  return hi <= lo ? 0 : 1 + (hi - lo - 1 + off) / c;
}
__host__ __device__ inline int run_slot(int lo, int i, int c, int off) {
  return i == 0 ? lo : lo + i * c - off;
}
// The run start that holds queue position t of a group beginning at lo.
__host__ __device__ inline int run_of(int lo, int t, int c, int off) {
  const int s = ((t - lo + off) / c) * c - off;
  return lo + (s > 0 ? s : 0);
}

}  // namespace kvpage
