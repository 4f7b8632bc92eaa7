// Compact work-queue builder and the page-table gather exporter.
//
// PersistentKV (aissential.tech summary, Summary and Method) schedules a
// compact workqueue that holds only non-empty (sequence, KV head, sequence
// split) tasks.  Here one workgroup per sequence computes its first task
// index from the lengths of the sequences before it (a deterministic prefix
// sum, no atomics) and writes its Hkv * ceil(ctx / S) tasks coalesced.
#include "kvpage_common.h"

namespace kvpage {

__device__ __forceinline__ int64_t splits_of(int32_t ctx, int32_t S) {
  return ctx > 0 ? ((int64_t)ctx + S - 1) / S : 0;
}

__device__ __forceinline__ int64_t wave_sum(int64_t v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// grid = B workgroups of one wave; workgroup b owns sequence b.
__global__ void __launch_bounds__(kWave) build_queue_kernel(
    const int32_t* __restrict__ ctx_lens, int32_t B, int32_t Hkv, int32_t S, int32_t max_pages,
    kvpage_task* __restrict__ tasks, int32_t capacity, int32_t* __restrict__ group_offsets,
    int32_t* __restrict__ n_tasks) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  int64_t before = 0;
  for (int i = lane; i < b; i += kWave) before += splits_of(clamp_ctx(ctx_lens[i], max_pages), S);
  before = wave_sum(before) * Hkv;
  const int32_t ctx = clamp_ctx(ctx_lens[b], max_pages);
  const int64_t n_b = splits_of(ctx, S);
  for (int g = lane; g < Hkv; g += kWave) {
    const int64_t off = before + g * n_b;
    group_offsets[(int64_t)b * Hkv + g] = (int32_t)(off < capacity ? off : capacity);
  }
  const int64_t mine = n_b * Hkv;
  // Tasks of (b, g) are contiguous: KV head outer, split inner, lanes over splits.
  for (int g = 0; g < Hkv; ++g) {
    const int64_t base = before + g * n_b;
    for (int j = lane; j < n_b; j += kWave) {
      const int64_t idx = base + j;
      if (idx >= capacity) break;
      kvpage_task t;
      t.seq = b;
      t.kv_head = g;
      t.tok_begin = j * S;
      t.tok_end = min(ctx, (j + 1) * S);
      tasks[idx] = t;
    }
  }
  if (b == B - 1 && lane == 0) {
    const int64_t total = before + mine;
    const int32_t clamped = (int32_t)(total < capacity ? total : capacity);
    group_offsets[(int64_t)B * Hkv] = clamped;
    n_tasks[0] = clamped;
  }
}

// Offsets inside a tile of the first element of token slot s that the
// attention kernel's lane maps read: K (chunk-major: s * 8) and V (row-major:
// s * d).  Each is -1 unless the pieces the K lanes (lane (s, r), every MFMA
// block) and the V lanes that land on slot s cover its d elements exactly
// once each, at the layout's places.
__device__ int2 lane_map_slot(int s, int d) {
  uint32_t kmask = 0, vmask = 0;
  bool kok = true, vok = true;
  for (int kb = 0; kb < d / 32; ++kb)
    for (int r = 0; r < 4; ++r) {   // K: lane (s, r) holds token s of every MFMA block
      const int el = (int)(k_piece_offset(kb, s, r, d) / 2) - s * 8;
      const int c = el / (kPage * 8);   // chunk
      kok = kok && el >= 0 && el % (kPage * 8) == 0 && c < d / 8;
      const uint32_t bit = 1u << (c & 31);
      kok = kok && !(kmask & bit);
      kmask |= bit;
    }
  for (int e = 0; e < 4; ++e)
    for (int r = 0; r < 4; ++r)
      for (int n = 0; n < 16; ++n) {   // V: every lane piece that lands in row s
        const int el = (int)(v_piece_offset(e, n, r, d) / 2);
        if (el / d != s) continue;
        const int col = el - s * d;
        vok = vok && col % (d / 16) == 0;
        const uint32_t bit = 1u << ((col / (d / 16)) & 31);
        vok = vok && !(vmask & bit);
        vmask |= bit;
      }
  const uint32_t full_k = (d / 8 >= 32) ? 0xffffffffu : ((1u << (d / 8)) - 1u);
  kok = kok && kmask == full_k;
  vok = vok && vmask == 0xffffu;
  return make_int2(kok ? s * 8 : -1, vok ? s * d : -1);
}

// One workgroup per queued task; lane j covers token slots j, j+64, ...  The
// offsets are built as the attention kernel builds its loads: the tile of
// the token's page and KV head (tile_offset), then the place its lane maps
// read for the token's slot.  Per token: [0] K, [1] V; -2 where the lane maps
// fail the check above, -1 past tok_end.
__global__ void __launch_bounds__(kWave) gather_offsets_kernel(
    const int32_t* __restrict__ block_tables, int32_t B, int32_t max_pages, int32_t Hkv, int32_t d,
    int32_t S, const kvpage_task* __restrict__ tasks, const int32_t* __restrict__ n_tasks,
    int32_t capacity, int64_t* __restrict__ offsets) {
  const int32_t n = min(n_tasks[0], capacity);
  for (int64_t i = blockIdx.x; i < n; i += gridDim.x) {
    kvpage_task t = tasks[i];
    t.seq = min(max(t.seq, 0), B - 1);
    t.tok_begin = clamp_ctx(t.tok_begin, max_pages);
    t.tok_end = min(clamp_ctx(t.tok_end, max_pages), t.tok_begin + S);
    const int32_t* bt_row = block_tables + (int64_t)t.seq * max_pages;
    for (int j = threadIdx.x; j < S; j += kWave) {
      const int32_t tok = t.tok_begin + j;
      int64_t ko = -1, vo = -1;
      if (tok < t.tok_end) {
        const int2 at = lane_map_slot(tok % kPage, d);
        const int64_t tile = tile_offset(bt_row[tok / kPage], t.kv_head, Hkv, d);
        ko = at.x < 0 ? -2 : tile + at.x;
        vo = at.y < 0 ? -2 : tile + at.y;
      }
      offsets[(i * S + j) * 2] = ko;
      offsets[(i * S + j) * 2 + 1] = vo;
    }
  }
}

hipError_t launch_build_queue(const kvpage_shape& s, const int32_t* ctx_lens, kvpage_task* tasks,
                              int32_t capacity, int32_t* group_offsets, int32_t* n_tasks,
                              hipStream_t stream) {
  hipLaunchKernelGGL(build_queue_kernel, dim3(s.B), dim3(kWave), 0, stream, ctx_lens, s.B, s.Hkv,
                     s.split_tokens, s.max_pages, tasks, capacity, group_offsets, n_tasks);
  return hipGetLastError();
}

hipError_t launch_gather_offsets(const kvpage_shape& s, const int32_t* block_tables,
                                 const kvpage_task* tasks, const int32_t* n_tasks,
                                 int32_t capacity, int64_t* offsets, hipStream_t stream) {
  const int grid = capacity < 65536 ? capacity : 65536;
  hipLaunchKernelGGL(gather_offsets_kernel, dim3(grid), dim3(kWave), 0, stream, block_tables,
                     s.B, s.max_pages, s.Hkv, s.d, s.split_tokens, tasks, n_tasks, capacity, offsets);
  return hipGetLastError();
}

}  // namespace kvpage
