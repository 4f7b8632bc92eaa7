// Split-KV paged GQA decode attention for gfx950.
//
// PersistentKV (aissential.tech summary, Summary and Method) maps decode
// work by KV-head group, reads K/V through native page tables and reuses each
// K/V tile across all query heads of the group.  Here one wavefront runs one
// queued (sequence, KV head, split) task at a time:
//
//   * a page is a 16-token tile, 16*d contiguous elements of K and of V;
//   * scores for the whole group come from 16x16x32 MFMAs with the K tile as
//     the 16-row operand (tokens) and the group's query rows as the 16
//     columns.  G <= 8 columns carry query heads; when budgeting, the next
//     columns carry the fast and slow query summaries split into 2 (f16) or
//     3 (bf16) pieces that sum to the float32 summary, so the summary-key dot
//     products (GrowPage: dual-timescale query summaries) cost no extra pass
//     over K;
//   * a task (at most PPT pages, PPT = 4, 8 or 16 by instance) runs in two
//     passes: all its scores first, kept in LDS, then the weights and P V;
//   * consecutive tasks of one (sequence, KV head) that a wavefront runs
//     share one partial whose reference max moves only when a task's max
//     exceeds it by more than 8 (log2 domain), so weights stay below 2^8;
//   * P V comes from 16x16x16 MFMAs whose P operand is the score tile's own
//     register layout, so no lane shuffles are needed between the two
//     contractions;
//   * K and V tiles stream through a ring of DEPTH register buffers, with
//     non-temporal loads (STREAM) when the caller says no page is shared.
//
// Outputs per run go to the workspace at the run's first queue position:
// m (log2 domain), l = sum exp2(y - m) and the unnormalised o = sum
// exp2(y - m) v for each query head of the group.
#include <float.h>
#include <math.h>

#include <atomic>
#include <type_traits>

#include <hip/hip_ext.h>

#include "kvpage_common.h"

namespace kvpage {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

template <bool BF>
struct Elem;

template <>
struct Elem<false> {  // float16
  static constexpr int kPieces = 2;
  static __device__ __forceinline__ f32x4 mfma_qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma_pv(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t bits(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
  }
  static __device__ __forceinline__ float value(uint32_t b16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b16);
  }
};

template <>
struct Elem<true> {  // bfloat16
  static constexpr int kPieces = 3;
  static __device__ __forceinline__ f32x4 mfma_qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma_pv(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                     __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t bits(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
  }
  static __device__ __forceinline__ float value(uint32_t b16) {
    return __builtin_bit_cast(float, (uint32_t)(b16 << 16));
  }
};

struct AttnParams {
  // What a wavefront needs first, kept together so that one batch of
  // kernel-argument loads brings it: lengths, page ids, query and summary
  // rows and the first tiles.
  const int32_t* ctx_lens;
  const int32_t* block_tables;
  const uint16_t* q;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const float* s_prev;
  int32_t split_tokens, B, Hq, Hkv, G, max_pages, num_pages, capacity;
  int32_t nwaves;   // wavefronts in the grid
  int32_t ncls;     // schedule classes (KV heads g % ncls), 1 or 8
  // Per sequence, leading logical pages that other sequences may share
  // (loads kLoadsPrefix only).
  const int32_t* shared_pages;
  // Division by split_tokens and by the number of wavefronts in the grid.
  DivMagic div_split, div_waves;
  const kvpage_task* tasks;
  const int32_t* n_tasks;
  // Fused queue build (one-call step): queue arrays out.
  kvpage_task* tasks_out;
  int32_t* group_offsets_out;
  int32_t* n_tasks_out;
  int32_t* ws_hdr;
  float* ws_o;
  float* ws_rm;
  float* ws_rl;
  float* page_mass;
  float* page_max;
  float alpha_fast, alpha_slow;
  float scale, c2, inv_g;
};

constexpr int kWavesPerGroup = 4;
constexpr int kMaxPagesPerTask = 16;   // pages of the longest split (256 tokens)
constexpr int kRunMax = 16;   // most pieces of work one wavefront takes in a row

// All-reduce over the four 16-lane rows of a wavefront (lanes n, n+16, n+32,
// n+48) with the gfx950 row-swap permutes: after a swap each lane holds its
// own value and its partner's, in some order.
__device__ __forceinline__ float rows_max(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float rows_sum(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Value of the lane `k` columns to the right inside the same 16-lane row.
template <int k>
__device__ __forceinline__ float from_right(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x100 + k, 0xf, 0xf, true));
}

// Two 16-bit halves (lo from a, hi from b), picking half `hi_half` of each word.
__device__ __forceinline__ uint32_t pick_pair(uint32_t a, uint32_t b, bool hi_half) {
  return hi_half ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
}

// One task = pages [0, npg) of one (sequence, KV head) split, npg <= PPT.
// Pass 1 streams the K tiles and keeps every score (PPT pages x 4 values per
// lane, in LDS), so the task's max is exact before any weight is formed;
// pass 2 streams the V tiles and applies exp2(score - run reference).  Tile
// loads form one stream (K pages 0..PPT-1, then V pages 0..PPT-1) fetched
// DEPTH tiles ahead; loads are issued for all 2 * PPT tiles whatever npg is
// (indices past npg - 1 repeat the last page) so the compiler can count
// outstanding loads exactly, while computation past npg is skipped.
// Task lookup for the fused queue build (at most 64 sequences): lane b holds
// sequence b's split count and the inclusive prefix of task counts, so the
// (sequence, KV head, split) of queue position t is one ballot away.  This is
// the same enumeration as the queue-build kernel.
// One tile load.  With STREAM the access is marked non-temporal, so the lines
// stream past the caches instead of displacing what is reused (page ids,
// query rows, partials).  Only right when no page is read twice in a call.
// Tile load policies of a kernel instance: all through the caches, all
// streaming, or streaming except the shared leading pages of each sequence
// (chosen per piece of work).
constexpr int kLoadsCached = 0;
constexpr int kLoadsStream = 1;
constexpr int kLoadsPrefix = 2;

// Run outputs (partials, page values) go past the L2 in the prefix-aware
// instances, where they would otherwise evict the shared prefix pages each
// XCD's L2 holds.  Measured on MI355X in alternating processes: B64 with a
// 128-page shared prefix 364.3 -> 357.6 us.  With streaming loads and no
// sharing they stay ordinary stores: B8 bimodal 132.0 -> 133.6 us with them
// streamed, B1 -0.2 us in one comparison and unchanged in another.
template <int LOADS>
struct OutPolicy {
  static constexpr bool kStream = LOADS == kLoadsPrefix;
};

template <bool STREAM, typename V>
__device__ __forceinline__ V tile_load(const char* addr) {
  if constexpr (STREAM) return __builtin_nontemporal_load(reinterpret_cast<const V*>(addr));
  else return *reinterpret_cast<const V*>(addr);
}

// A run output store: non-temporal with STREAM, so the value goes past the
// L2 instead of staying there dirty.
template <bool STREAM, typename T>
__device__ __forceinline__ void out_store(T* addr, T v) {
  if constexpr (STREAM) __builtin_nontemporal_store(v, addr);
  else *addr = v;
}

struct SeqScan {
  int ctx, ns, cnt, incl, total;
  float rns;   // 1 / ns (approximate)
};

// Lane b's length (lanes past B repeat the last one; the scan masks them).
// The load is unconditional (B >= 1 here): under a branch it came after two
// more rounds of kernel-argument loads; this way it leaves after the first
// (0.3 us earlier).
__device__ __forceinline__ int32_t load_length(const int32_t* ctx_lens, int B, int lane) {
  return ctx_lens[min(lane, B - 1)];
}

__device__ __forceinline__ SeqScan scan_lengths(int32_t raw, int B, int Hkv, int S,
                                                DivMagic div_s, int max_pages, int lane) {
  SeqScan q;
  q.ctx = clamp_ctx(raw & -(int32_t)(lane < B), max_pages);
  q.ns = (int)div_by((uint32_t)(q.ctx + S - 1), div_s);
  q.rns = __builtin_amdgcn_rcpf((float)q.ns);
  q.cnt = q.ns * Hkv;
  // Inclusive prefix over the lanes: within each row of 16 lanes by DPP row
  // shifts (a lane with no source reads 0), then the row totals added in.
  int v = q.cnt;
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15);
  const int r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  v += (lane >= 16 ? r0 : 0) + (lane >= 32 ? r1 : 0) + (lane >= 48 ? r2 : 0);
  q.incl = v;
  q.total = __builtin_amdgcn_readlane(v, kWave - 1);
  return q;
}

// The buffers of a wavefront's first dependent load (the lengths, or the
// caller's task count) and B come first, as arguments of their own: gfx950
// can preload leading scalar kernel arguments into SGPRs at wave launch, so
// that load does not wait for the kernel-argument block.
template <int D, bool BF, bool BUDGET, int DEPTH, bool FUSEDQ, int PPT, int LOADS>
__global__ void __launch_bounds__(kWave * kWavesPerGroup)
    split_attn_kernel(const int32_t* lead_lens, const int32_t* lead_ntasks, int32_t lead_B,
                      const AttnParams p) {
  using E = Elem<BF>;
  constexpr bool NTO = OutPolicy<LOADS>::kStream;   // run outputs past the L2
  constexpr int KB = D / 32;   // 16x16x32 MFMAs per page for the scores
  constexpr int VD = D / 16;   // output column blocks; V halves per lane per token
  constexpr int VW = VD / 2;   // V dwords per lane per token
  constexpr int TW = D / 8;    // dwords per lane per tile (K or V)
  constexpr int NPC = E::kPieces;
  // PPT: pages per piece this instance handles (a split of at most PPT
  // pages is one piece, a longer one several); every piece issues loads for
  // exactly PPT K and PPT V tiles.
  static_assert(PPT <= kMaxPagesPerTask, "at most 16 pages per task");
  constexpr int NT = 2 * PPT;
  // The next task's first tiles are fetched into the slots its first pages
  // are read from only if the ring length divides the tiles per task.
  static_assert(NT % DEPTH == 0, "prefetch depth must divide the tiles per task");
  // The next task is known only after this task's K pass, so the tiles the
  // ring fetches ahead of it during the V pass must all be K tiles.
  static_assert(DEPTH <= PPT, "prefetch depth must not exceed the K tiles of a task");
  constexpr int QCL = 8 * D / 8 / kWave;          // 16-byte query chunks per lane (8 rows max)
  // Staging words per wave: 16 operand rows of D halves (G query heads, then
  // the summary pieces), then the two float32 summary rows of s_prev.
  constexpr int kOpRows = 16;
  constexpr int kQStage = kOpRows * D / 2 + 2 * D;
  constexpr int DPL = D / kWave;                  // summary elements per lane
  constexpr int kMaxG = 8;                        // query heads per KV head, at most

  // Per-wave LDS: staged query / summary rows, and the scores of the task.
  __shared__ uint32_t lds_q[kWavesPerGroup * kQStage];
  __shared__ f32x4 lds_s[kWavesPerGroup][PPT][kWave];
  // Per-wave staging of a run's per-task outputs, written out once per run:
  // raw page sums per head, summary page maxima, the weight reference each
  // task used, and (fused queue build) the task records.
  __shared__ float lds_mass[kWavesPerGroup][BUDGET ? kRunMax : 1][8][kPage];
  __shared__ float lds_pmax[kWavesPerGroup][BUDGET ? kRunMax : 1][2][kPage];
  __shared__ float lds_tref[kWavesPerGroup][BUDGET ? kRunMax : 1][8];
  __shared__ kvpage_task lds_task[kWavesPerGroup][FUSEDQ ? kRunMax : 1];

  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane >> 4;       // row of 16 lanes
  const int n = lane & 15;       // column inside the row
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = p.nwaves;   // gridDim would add the 256-byte hidden argument block
  const int G = p.G;
  const bool is_head = n < G;
  const bool is_lead = BUDGET && (n == G || n == G + NPC);

  // Byte offsets of this lane's pieces inside one (page, head) tile.
  uint32_t koff[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) koff[kb] = k_piece_offset(kb, n, r, D);
  uint32_t voff[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) voff[e] = v_piece_offset(e, n, r, D);

  const char* kpool = reinterpret_cast<const char*>(p.k_pool);
  const char* vpool = reinterpret_cast<const char*>(p.v_pool);

  // A unit of work: piece `piece` (at most PPT pages) of queue entry t.
  // A split longer than PPT pages is run as consecutive pieces of one task;
  // tb0 / te are the task's token range, tok_begin / tok_end the piece's.
  struct Task {
    int t, b, g, tok_begin, tok_end, ntok, npg, lp0, piece, tb0, te;
    int sp;        // shared leading pages of sequence b (kLoadsPrefix)
    bool last;     // the task's last piece
    bool cached;   // loads through the caches (kLoadsPrefix: the piece starts on a shared page)
  };
  auto unit = [&](Task k, int pc) {
    k.piece = pc;
    k.tok_begin = k.tb0 + pc * (PPT * kPage);
    k.tok_end = min(k.te, k.tok_begin + PPT * kPage);
    k.ntok = k.tok_end - k.tok_begin;
    k.npg = (k.ntok + kPage - 1) / kPage;
    k.lp0 = k.tok_begin / kPage;
    k.last = k.tok_end >= k.te;
    k.cached = LOADS == kLoadsPrefix && k.lp0 < k.sp;
    return k;
  };
  SeqScan sq = {0, 0, 0, 0, 0};
  // Queue entry t: read from the queue, or (fused build) derived from the lengths.
  auto fetch = [&](int t) {
    kvpage_task tk;
    if constexpr (FUSEDQ) {
      const uint64_t past = __builtin_amdgcn_ballot_w64(sq.incl > t);
      const int bq = __builtin_ctzll(past);
      const int start = __builtin_amdgcn_readlane(sq.incl - sq.cnt, bq);
      const int ns = __builtin_amdgcn_readlane(sq.ns, bq);
      const int ctx = __builtin_amdgcn_readlane(sq.ctx, bq);
      const int k = t - start;
      // k / ns from the float reciprocal: the quotient is below Hkv, so the
      // estimate is off by at most one; corrected both ways.
      const float rns = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sq.rns), bq));
      int gq = (int)((float)k * rns);
      gq -= (uint32_t)gq * (uint32_t)ns > (uint32_t)k ? 1 : 0;
      gq += (uint32_t)(gq + 1) * (uint32_t)ns <= (uint32_t)k ? 1 : 0;
      const int j = k - gq * ns;
      tk.seq = bq;
      tk.kv_head = gq;
      tk.tok_begin = j * p.split_tokens;
      tk.tok_end = min(ctx, tk.tok_begin + p.split_tokens);
    } else {
      // A caller's queue entry is clamped into the shape: a bad entry gives
      // wrong values for its row, never an access outside the buffers.
      tk = p.tasks[t];
      tk.seq = min(max(tk.seq, 0), p.B - 1);
      tk.kv_head = min(max(tk.kv_head, 0), p.Hkv - 1);
      tk.tok_begin = clamp_ctx(tk.tok_begin, p.max_pages);
      tk.tok_end = min(max(tk.tok_end, tk.tok_begin),
                       min(tk.tok_begin + p.split_tokens, p.max_pages * kPage));
    }
    Task k;
    k.t = t;
    k.b = tk.seq;
    k.g = tk.kv_head;
    k.tb0 = tk.tok_begin;
    k.te = tk.tok_end;
    k.sp = 0;
    if constexpr (LOADS == kLoadsPrefix) k.sp = p.shared_pages[k.b];
    return unit(k, 0);
  };
  // Lane i < npg holds the physical id of the task's page i.
  auto load_page_ids = [&](const Task& k) -> int32_t {
    const int32_t* bt_row = p.block_tables + (int64_t)k.b * p.max_pages + k.lp0;
    return lane < k.npg ? bt_row[lane] : 0;
  };
  // The group's G query rows (contiguous G*D halves) and, when budgeting, its
  // two summary rows, as compact 16-byte chunks.
  struct Rows {
    u32x4 q[QCL];
    u32x4 s;
  };
  // Every lane loads (chunks past the group's rows repeat its last chunk), so
  // that no load is conditional and the wait counts stay exact.
  auto load_rows = [&](const Task& k) {
    Rows w;
    const uint16_t* qblk = p.q + ((int64_t)k.b * p.Hq + (int64_t)k.g * G) * D;
#pragma unroll
    for (int i = 0; i < QCL; ++i) {
      const int ch = min(lane + i * kWave, G * D / 8 - 1);
      w.q[i] = *reinterpret_cast<const u32x4*>(qblk + 8 * ch);
    }
    w.s = u32x4{0u, 0u, 0u, 0u};
    if constexpr (BUDGET) {
      const int ls = min(lane, D / 2 - 1);
      const int which = ls / (D / 4);
      const int ch = ls % (D / 4);
      w.s = *reinterpret_cast<const u32x4*>(
          p.s_prev + (((int64_t)which * p.B + k.b) * p.Hkv + k.g) * D + 4 * ch);
    }
    return w;
  };
  // Tile tau of a task: K page tau for tau < 16, V page tau - 16 after.  Pages
  // past npg - 1 repeat the last page (the load count never depends on npg).
  // sl: std::true_type for non-temporal (streaming) loads, false_type for
  // loads through the caches.
  auto load_tile = [&](auto sl, const Task& k, int32_t ids, int tau, uint32_t (&dst)[TW]) {
    constexpr bool SL = decltype(sl)::value;
    const bool is_v = tau >= PPT;
    const int pg = max(min(is_v ? tau - PPT : tau, k.npg - 1), 0);
    const int32_t pid = clamp_page(__builtin_amdgcn_readlane(ids, pg), p.num_pages);
    const int64_t off = tile_offset(pid, k.g, p.Hkv, D) * 2;
    if (!is_v) {
      const char* base = kpool + off;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const u32x4 w = tile_load<SL, u32x4>(base + koff[kb]);
#pragma unroll
        for (int x = 0; x < 4; ++x) dst[4 * kb + x] = w[x];
      }
    } else {
      const char* base = vpool + off;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (VW == 4) {
          const u32x4 w = tile_load<SL, u32x4>(base + voff[e]);
#pragma unroll
          for (int x = 0; x < 4; ++x) dst[VW * e + x] = w[x];
        } else {
          const u32x2 w = tile_load<SL, u32x2>(base + voff[e]);
#pragma unroll
          for (int x = 0; x < VW; ++x) dst[VW * e + x] = w[x];
        }
      }
    }
  };

  uint32_t* qs = lds_q + wave * kQStage;   // [16][D] halves, then [2][D] floats
  f32x4* S = lds_s[wave][0];               // page i at S[i * kWave + lane]
  uint16_t* qh = reinterpret_cast<uint16_t*>(qs);

  // Column operand from staged rows: query heads, then (budgeting) the
  // summary pieces, then zeros.  Each summary element is computed once, by
  // one lane: the group-mean query (heads added in head order), one EMA
  // step, then pieces in the storage type that sum back to the float32 value.
  auto build_operand = [&](const Rows& rows, u32x4 (&qop)[KB]) {
#pragma unroll
    for (int i = 0; i < QCL; ++i) *reinterpret_cast<u32x4*>(qs + 4 * (lane + i * kWave)) = rows.q[i];
    if constexpr (BUDGET) {
      if (lane < D / 2) *reinterpret_cast<u32x4*>(qs + kOpRows * D / 2 + 4 * lane) = rows.s;
    }
    __builtin_amdgcn_wave_barrier();
    if constexpr (BUDGET) {
      const float* sp = reinterpret_cast<const float*>(qs + kOpRows * D / 2);
      // Every read first, so that they share one LDS round trip: this lane's
      // elements of the first kMaxG staged rows (rows from G on are read and
      // not used) and of both summaries.
      float hv[kMaxG][DPL];
      float sv[2][DPL];
#pragma unroll
      for (int h = 0; h < kMaxG; ++h) {
        if constexpr (DPL == 2) {
          const uint32_t w = qs[h * D / 2 + lane];
          hv[h][0] = E::value(w & 0xffffu);
          hv[h][1] = E::value(w >> 16);
        } else {
#pragma unroll
          for (int x = 0; x < DPL; ++x) hv[h][x] = E::value(qh[h * D + DPL * lane + x]);
        }
      }
#pragma unroll
      for (int which = 0; which < 2; ++which)
#pragma unroll
        for (int x = 0; x < DPL; ++x) sv[which][x] = sp[which * D + DPL * lane + x];
      uint32_t pcs[2][NPC][DPL];
#pragma unroll
      for (int x = 0; x < DPL; ++x) {
        float acc = hv[0][x];
#pragma unroll
        for (int h = 1; h < kMaxG; ++h)
          if (h < G) acc = add_rn(acc, hv[h][x]);
        const float qbar = mul_rn(acc, p.inv_g);
#pragma unroll
        for (int which = 0; which < 2; ++which) {
          float rem = ema_step(sv[which][x], qbar, which ? p.alpha_slow : p.alpha_fast);
#pragma unroll
          for (int piece = 0; piece < NPC; ++piece) {
            pcs[which][piece][x] = E::bits(rem);
            rem = sub_rn(rem, E::value(pcs[which][piece][x]));
          }
        }
      }
#pragma unroll
      for (int which = 0; which < 2; ++which)
#pragma unroll
        for (int piece = 0; piece < NPC; ++piece) {
          const int row = G + which * NPC + piece;
          if constexpr (DPL == 2)
            qs[row * D / 2 + lane] = pcs[which][piece][0] | (pcs[which][piece][1] << 16);
          else
#pragma unroll
            for (int x = 0; x < DPL; ++x) qh[row * D + DPL * lane + x] = (uint16_t)pcs[which][piece][x];
        }
      __builtin_amdgcn_wave_barrier();
    }
    const bool has_row = n < G + (BUDGET ? 2 * NPC : 0);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int d0 = 8 * (4 * kb + r);
      qop[kb] = has_row ? *reinterpret_cast<const u32x4*>(qs + (n * D + d0) / 2)
                        : u32x4{0u, 0u, 0u, 0u};
    }
    __builtin_amdgcn_wave_barrier();
  };

  uint32_t buf[DEPTH][TW];
  u32x4 qop[KB];
  int ntask;
  if constexpr (FUSEDQ) {
    const int32_t raw_len = load_length(lead_lens, lead_B, lane);
    sq = scan_lengths(raw_len, p.B, p.Hkv, p.split_tokens, p.div_split, p.max_pages, lane);
    ntask = min(sq.total, p.capacity);
    if (blockIdx.x == 0 && wave == 0) {
      if (lane < p.B) {
        const int start = sq.incl - sq.cnt;
        for (int g = 0; g < p.Hkv; ++g)
          p.group_offsets_out[lane * p.Hkv + g] = min(start + g * sq.ns, p.capacity);
      }
      if (lane == 0) {
        p.group_offsets_out[p.B * p.Hkv] = ntask;
        p.n_tasks_out[0] = ntask;
      }
    }
  } else {
    ntask = min(lead_ntasks[0], p.capacity);
  }
  // Classes: with ncls > 1 the queue is taken as ncls classes, class x the
  // (sequence, KV head) groups with g % ncls == x in queue order, and class x
  // runs on the workgroups with blockIdx.x % ncls == x.  Workgroups go to the
  // 8 XCDs round robin, so all tasks of one KV head run on one XCD: a page
  // that several sequences share (a common prefix) is fetched into that
  // XCD's L2 once and served from there to the others.  It needs classes of
  // equal size (fused queue, Hkv % ncls == 0, nothing cut by capacity) and
  // a grid that is a multiple of ncls (checked on the host).
  int ncls = 1;
  if constexpr (FUSEDQ) ncls = (p.ncls > 1 && ntask == sq.total) ? p.ncls : 1;
  const int cls = (int)blockIdx.x % ncls;
  const int nwc = nwaves / ncls;                                        // wavefronts of the class
  const int wc = ((int)blockIdx.x / ncls) * kWavesPerGroup + wave;   // this one's rank in it
  const int T = ntask / ncls;                                           // positions of the class
  // Class position j -> queue position: j falls in sequence b when b's
  // class positions, [start_b, end_b) / ncls, hold it; inside b it is task
  // s of the class's gi-th KV head, g = cls + ncls * gi.
  auto pos_of = [&](int j) -> int {
    if constexpr (FUSEDQ) {
      if (ncls > 1) {
        const uint64_t past = __builtin_amdgcn_ballot_w64(sq.incl > ncls * j);
        const int bq = __builtin_ctzll(past);
        const int start = __builtin_amdgcn_readlane(sq.incl - sq.cnt, bq);
        const int ns = __builtin_amdgcn_readlane(sq.ns, bq);
        const int rr = j - start / ncls;
        const int gi = rr / ns;
        return start + (cls + ncls * gi) * ns + (rr - gi * ns);
      }
    }
    return j;
  };
  // The class is cut into chunks of c consecutive positions (c pieces of
  // work at most kRunMax, sized so every wavefront gets nearly the same
  // number of chunks); wavefront wc runs chunks wc, wc + nwc, ...  Run
  // partials start at a group's first task and at the first task of every
  // chunk.
  const int pieces = (p.split_tokens + PPT * kPage - 1) / (PPT * kPage);   // per task
  const int cmax = kRunMax / pieces;
  int c;
  if (T <= nwc * cmax) {   // one round
    c = max(1, ncls == 1 ? (int)div_by((uint32_t)(T + nwc - 1), p.div_waves) : (T + nwc - 1) / nwc);
  } else {
    const int rounds = (T + nwc * cmax - 1) / (nwc * cmax);
    c = (T + nwc * rounds - 1) / (nwc * rounds);
  }
  if (blockIdx.x == 0 && wave == 0 && lane == 0) {
    p.ws_hdr[0] = c;
    p.ws_hdr[1] = ncls;
  }
  int chunk = wc;
  if (chunk * c >= T) return;   // chunk past the last one
  int chunk_end = min((chunk + 1) * c, T);   // exclusive
  int cj = chunk * c;                        // class position of the current task

  // Runs f with the load policy of task k: one uniform branch per task, so
  // that no tile load sits under a branch of its own.
  auto with_policy = [&](const Task& k, auto f) __attribute__((always_inline)) {
    if constexpr (LOADS == kLoadsPrefix) {
      if (k.cached) return f(std::false_type{});
      return f(std::true_type{});
    } else {
      return f(std::integral_constant<bool, LOADS == kLoadsStream>{});
    }
  };

  Task cur = fetch(pos_of(cj));
  // Query rows first: they arrive with the page ids, so the operand is built
  // while the first tiles are in flight.
  const Rows rows = load_rows(cur);
  int32_t ids = load_page_ids(cur);
  with_policy(cur, [&](auto sl) __attribute__((always_inline)) {
#pragma unroll
    for (int tau = 0; tau < DEPTH; ++tau) load_tile(sl, cur, ids, tau, buf[tau]);
  });
  build_operand(rows, qop);

  // Run state: the running partial of consecutive tasks of one (b, g).
  int run_start = cur.t;
  int run_lp0 = cur.lp0;
  int run_pages = 0;
  int run_units = 0;   // pieces of the run done so far
  // A run is consecutive pieces of consecutive tasks of one (sequence, KV
  // head); all but its last are whole pieces of upg pages, so page pp of the
  // run is page pp % upg of its piece pp / upg.
  const int upg = min(p.split_tokens / kPage, PPT);
  float mrun = is_head ? -INFINITY : INFINITY;   // log2-domain reference; non-head lanes weigh 0
  float l = 0.f;
  f32x4 O[VD];
#pragma unroll
  for (int j = 0; j < VD; ++j) O[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One piece of work: pass 1, pass 2, staging and (at a run boundary) the
  // partial.  Returns false after the wavefront's last piece.
  auto step = [&](auto sl) __attribute__((always_inline)) -> bool {
    constexpr bool SL = decltype(sl)::value;
    const int b = cur.b, g = cur.g, ntok = cur.ntok, npg = cur.npg;

    // ---- pass 1: scores of every page; page max (budget) and task max ----
    float keep[4] = {0.f, 0.f, 0.f, 0.f};  // per-page outputs, page 4*r + u
    float mloc = -INFINITY;                 // in-lane max of this lane's scores
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int slot = i % DEPTH;
      // The tile's operands are taken first and the slot refilled at once, so
      // the next request does not wait behind this tile's MFMAs.
      u32x4 a[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int x = 0; x < 4; ++x) a[kb][x] = buf[slot][4 * kb + x];
      if (i + DEPTH < NT) load_tile(sl, cur, ids, i + DEPTH, buf[slot]);
      if (i < npg) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) acc = E::mfma_qk(a[kb], qop[kb], acc);
        if constexpr (BUDGET) {
          // Summary pieces sit in adjacent columns: add them into the lead column.
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float sum = add_rn(acc[e], from_right<1>(acc[e]));
            if constexpr (NPC == 3) sum = add_rn(sum, from_right<2>(acc[e]));
            acc[e] = is_head ? acc[e] : sum;
          }
        }
        const int nvalid = ntok - kPage * i;
        if (nvalid < kPage) {  // last page is partial: drop slots past the context
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * r + e >= nvalid) acc[e] = -INFINITY;
        }
        S[i * kWave + lane] = acc;
        const float pm = fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3]));
        if constexpr (BUDGET) {
          const float pmr = rows_max(pm);
          mloc = fmaxf(mloc, pmr);
          if (r == (i >> 2)) keep[i & 3] = pmr * p.scale;  // used by summary lead lanes
        } else {
          mloc = fmaxf(mloc, pm);
        }
      }
    }
    // The run's reference moves only when a task's max exceeds it by more
    // than 8 (log2 domain), so weights stay below 2^8 and rescales are rare.
    const float ymax = (BUDGET ? mloc : rows_max(mloc)) * p.c2;
    const bool need = is_head && ymax > mrun + 8.0f;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float alpha = need ? (mrun == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrun - ymax)) : 1.f;
      mrun = need ? ymax : mrun;
      l *= alpha;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ae = __shfl(alpha, 4 * r + e, kWave);
#pragma unroll
        for (int j = 0; j < VD; ++j) O[j][e] *= ae;
      }
    }

    // ---- the next piece of this wave (or this one again at the end) ----
    const bool more = !cur.last;   // another piece of this task
    const bool in_chunk = more || cj + 1 < chunk_end;
    const bool next_chunk = !in_chunk && (chunk + nwc) * c < T;
    const bool has_next = in_chunk || next_chunk;
    const int jn = more ? cj
                        : (cj + 1 < chunk_end ? cj + 1 : (next_chunk ? (chunk + nwc) * c : cj));
    const Task nxt = more ? unit(cur, cur.piece + 1) : fetch(pos_of(jn));
    const int32_t ids_n = load_page_ids(nxt);
    const Rows rows_n = load_rows(nxt);

    // ---- pass 2: weights, page sums, P V into the run's accumulators ----
    // Each V tile is first packed into its MFMA operands; its registers are
    // then free, so the next tile is requested before this tile's MFMAs and
    // the request does not wait behind them (with the request after the
    // MFMAs, a wavefront's two-tile stream stalled on every V tile: ~15% of
    // the B1 kernel time).
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int tau = PPT + i;
      const int slot = tau % DEPTH;
      const int nvalid = ntok - kPage * i;
      if (i < npg && nvalid < kPage) {  // zero V rows past the context (they may hold NaN)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * r + e >= nvalid) {
#pragma unroll
            for (int w = 0; w < VW; ++w) buf[slot][VW * e + w] = 0u;
          }
      }
      // Pages past the task's last one (the load count is fixed) contribute
      // nothing: their operands are zero (their rows may hold anything), so
      // the MFMAs below run unconditionally.  With them under a branch the
      // accumulators were copied at the join after every tile, which waited
      // for the MFMAs to finish and stalled the stream.
      const bool used = i < npg;
      u32x2 vop[VD];
#pragma unroll
      for (int j = 0; j < VD; ++j) {
        const bool hi = j & 1;
        const int w = j >> 1;
        vop[j][0] = used ? pick_pair(buf[slot][w], buf[slot][VW + w], hi) : 0u;
        vop[j][1] = used ? pick_pair(buf[slot][2 * VW + w], buf[slot][3 * VW + w], hi) : 0u;
      }
      if (tau + DEPTH < NT) {
        load_tile(sl, cur, ids, tau + DEPTH, buf[slot]);
      } else {
        // The next task's first K tiles; with no next task, the same number of
        // loads re-read this task's last V tile (just fetched, so cached).
        const int pg = max(has_next ? min(tau + DEPTH - NT, nxt.npg - 1) : npg - 1, 0);
        const int32_t pid = clamp_page(__builtin_amdgcn_readlane(has_next ? ids_n : ids, pg), p.num_pages);
        const char* base = (has_next ? kpool : vpool) + tile_offset(pid, has_next ? nxt.g : g, p.Hkv, D) * 2;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const u32x4 w = tile_load<SL, u32x4>(base + koff[kb]);
#pragma unroll
          for (int x = 0; x < 4; ++x) buf[slot][4 * kb + x] = w[x];
        }
      }
      {
        const f32x4 sc = S[i * kWave + lane];
        float pe[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pe[e] = used ? __builtin_amdgcn_exp2f(fmaf(sc[e], p.c2, -mrun)) : 0.f;
        const float psum = (pe[0] + pe[1]) + (pe[2] + pe[3]);
        l += psum;
        if constexpr (BUDGET) {
          const float page_sum = rows_sum(psum);
          if (used && is_head && r == (i >> 2)) keep[i & 3] = page_sum;
        }
        uint32_t pb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pb[e] = E::bits(pe[e]);
        u32x2 pop;
        pop[0] = pb[0] | (pb[1] << 16);
        pop[1] = pb[2] | (pb[3] << 16);
        // bfloat16 keeps 8 significant bits of a weight: the rounding
        // remainder goes in as a second bfloat16 term, so P V sees ~16 bits.
        // With one rounding, a few dominant weights on an output that cancels
        // to a small value exceeded the output tolerance (1 to 3 entries in
        // 10^5 in random bf16 cases).  float16 rounds 4x finer and needs no
        // second term.
        u32x2 pop_lo = {0u, 0u};
        if constexpr (BF) {
          uint32_t rb[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) rb[e] = E::bits(sub_rn(pe[e], E::value(pb[e])));
          pop_lo[0] = rb[0] | (rb[1] << 16);
          pop_lo[1] = rb[2] | (rb[3] << 16);
        }
#pragma unroll
        for (int j = 0; j < VD; ++j) {
          O[j] = E::mfma_pv(pop, vop[j], O[j]);
          if constexpr (BF) O[j] = E::mfma_pv(pop_lo, vop[j], O[j]);
        }
      }
    }

    // ---- per piece: stage the queue entry and budgeting values in LDS ----
    const int kin = run_units;            // piece position inside the run, < kRunMax
    const int ktask = cur.t - run_start;  // task position inside the run
    if constexpr (FUSEDQ) {
      if (lane == 0 && cur.piece == 0) {
        kvpage_task out_t;
        out_t.seq = b;
        out_t.kv_head = g;
        out_t.tok_begin = cur.tb0;
        out_t.tok_end = cur.te;
        lds_task[wave][ktask] = out_t;
      }
    }
    if constexpr (BUDGET) {
      const f32x4 kv4 = {keep[0], keep[1], keep[2], keep[3]};
      if (is_head) *reinterpret_cast<f32x4*>(&lds_mass[wave][kin][n][4 * r]) = kv4;
      if (is_lead) *reinterpret_cast<f32x4*>(&lds_pmax[wave][kin][n == G ? 0 : 1][4 * r]) = kv4;
      if (r == 0 && is_head) lds_tref[wave][kin][n] = mrun;
    }
    run_pages += npg;
    ++run_units;

    // ---- run boundary: write the run's partial (m, l, o) per head ----
    const bool new_group = nxt.b != b || nxt.g != g;
    if (!in_chunk || new_group) {
      // The run's stores wait for issue slots behind the tile loads of the
      // compute unit's other wavefronts; raised priority lets them go first
      // (B1 0.3-0.6% faster, B8 unchanged, interleaved).
      __builtin_amdgcn_s_setprio(3);
      const float ltot = rows_sum(l);
      if (r == 0 && is_head) {
        out_store<NTO>(&p.ws_rm[(int64_t)run_start * G + n], mrun);
        out_store<NTO>(&p.ws_rl[(int64_t)run_start * G + n], ltot);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int h = 4 * r + e;
        if (h < G) {
          float* dst = p.ws_o + ((int64_t)run_start * G + h) * D + n * VD;
#pragma unroll
          for (int j = 0; j < VD; ++j) out_store<NTO>(&dst[j], O[j][e]);
        }
      }
      const int nk = ktask + 1;
      if constexpr (FUSEDQ) {
        __builtin_amdgcn_wave_barrier();
        if (lane < nk) p.tasks_out[run_start + lane] = lds_task[wave][lane];
      }
      if (BUDGET && kin == 0) {
        // A run of one task: its reference is the run's, so the staged page
        // values are final.  Lane (h, pg) = (lane / 16, lane % 16) stores page
        // pg of head h (of summary h for the page maxima): one store per four
        // heads instead of one per page and column.
        __builtin_amdgcn_wave_barrier();
        const int pg = lane & 15;
        const int hl = lane >> 4;
#pragma unroll
        for (int hb = 0; hb < kMaxG; hb += 4) {
          const int h = hb + hl;
          if (hb < G && h < G && pg < npg)
            out_store<NTO>(
                &p.page_mass[((int64_t)b * p.Hq + (int64_t)g * G + h) * p.max_pages + run_lp0 + pg],
                lds_mass[wave][0][h][pg]);
        }
        if (hl < 2 && pg < npg)
          out_store<NTO>(
              &p.page_max[(((int64_t)hl * p.B + b) * p.Hkv + g) * p.max_pages + run_lp0 + pg],
              lds_pmax[wave][0][hl][pg]);
      } else if constexpr (BUDGET) {
        // Raw page sums move to the run's final reference, the one its
        // partial carries; pages of a run are consecutive in the sequence.
        __builtin_amdgcn_wave_barrier();
        const int rp = min(run_pages, p.max_pages - run_lp0);
        for (int h = 0; h < G; ++h) {
          const float mh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mrun), h));
          float* row = p.page_mass + ((int64_t)b * p.Hq + (int64_t)g * G + h) * p.max_pages + run_lp0;
          for (int pp = lane; pp < rp; pp += kWave) {
            const int kk = pp / upg;   // piece of the run holding page pp
            out_store<NTO>(&row[pp], lds_mass[wave][kk][h][pp - kk * upg] *
                                         __builtin_amdgcn_exp2f(lds_tref[wave][kk][h] - mh));
          }
        }
        for (int which = 0; which < 2; ++which) {
          float* row = p.page_max + (((int64_t)which * p.B + b) * p.Hkv + g) * p.max_pages + run_lp0;
          for (int pp = lane; pp < rp; pp += kWave) {
            const int kk = pp / upg;
            out_store<NTO>(&row[pp], lds_pmax[wave][kk][which][pp - kk * upg]);
          }
        }
      }
      __builtin_amdgcn_s_setprio(0);
      if (!has_next) return false;
      if (next_chunk) {
        chunk += nwc;
        chunk_end = min((chunk + 1) * c, T);
      }
      run_start = nxt.t;
      run_lp0 = nxt.lp0;
      run_pages = 0;
      run_units = 0;
      mrun = is_head ? -INFINITY : INFINITY;
      l = 0.f;
#pragma unroll
      for (int j = 0; j < VD; ++j) O[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      build_operand(rows_n, qop);
    }
    cur = nxt;
    cj = jn;
    ids = ids_n;
    return true;
  };
  while (with_policy(cur, step)) {
  }
}

template <int D, bool BF, bool BUDGET, int DEPTH, bool FUSEDQ, int PPT, int LOADS>
static hipError_t launch_one(const AttnParams& p, int capacity, hipStream_t stream,
                             hipEvent_t ev_start, hipEvent_t ev_stop, int max_wg) {
  auto kern = split_attn_kernel<D, BF, BUDGET, DEPTH, FUSEDQ, PPT, LOADS>;
  // The grid is one workgroup per compute unit, whatever else would fit:
  // the grid, and with it the schedule, the runs and the rounding of every
  // result, is then the same for every instance (the load policies give the
  // same bits); a second resident workgroup measured no faster.  Compute
  // units per device, found once; concurrent first calls store the same
  // value.
  static std::atomic<int> resident_wg[64];
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  std::atomic<int>& cached = resident_wg[dev & 63];
  int resident_n = cached.load(std::memory_order_relaxed);
  if (resident_n == 0) {
    int cus = 0;
    err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    resident_n = cus > 0 ? cus : 1;
    cached.store(resident_n, std::memory_order_relaxed);
  }
  const int64_t want = ((int64_t)capacity + kWavesPerGroup - 1) / kWavesPerGroup;
  const int64_t resident = resident_n;
  int64_t grid64 = want < resident ? want : resident;
  if (max_wg > 0 && grid64 > max_wg) grid64 = max_wg;
  const int grid = (int)grid64;
  if (grid <= 0) return hipSuccess;
  AttnParams a = p;
  a.nwaves = grid * kWavesPerGroup;
  // One class per XCD when the fused queue splits evenly over them and there
  // is more than one sequence (only then can a page be shared).  Measured on
  // MI355X: B64 with a shared prefix 3.4% faster, B8 workloads 1.3-2.1%; one
  // 32K-token sequence 2.5% slower, hence not for B = 1.
  a.ncls = (FUSEDQ && p.B >= 2 && p.Hkv % 8 == 0 && grid % 8 == 0) ? 8 : 1;
  a.div_waves = div_magic((uint32_t)grid * kWavesPerGroup);
  if (ev_start || ev_stop) {
    // Timestamps taken by the dispatch itself: start and end of this kernel.
    hipExtLaunchKernelGGL(kern, dim3(grid), dim3(kWave * kWavesPerGroup), 0, stream, ev_start,
                          ev_stop, 0, a.ctx_lens, a.n_tasks, a.B, a);
  } else {
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kWave * kWavesPerGroup), 0, stream, a.ctx_lens,
                       a.n_tasks, a.B, a);
  }
  return hipGetLastError();
}

// Tiles (4 KiB at d = 128) each wave keeps in flight.  Two is fastest on
// MI355X for every workload measured: with 1024 wavefronts, 8 tiles each put
// 32 MiB in flight, as much as all XCDs' L2 together, and ran 3-8% slower;
// one tile each cannot cover the memory latency.
#ifndef KVPAGE_ATTN_DEPTH
#define KVPAGE_ATTN_DEPTH 2
#endif

template <bool FUSEDQ, int PPT, int LOADS>
static hipError_t dispatch_ppt(const kvpage_shape& s, const AttnParams& p, int capacity, bool bud,
                               hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop,
                               int max_wg) {
  constexpr int DP = KVPAGE_ATTN_DEPTH < PPT ? KVPAGE_ATTN_DEPTH : PPT;
  const bool bf = s.dtype == KVPAGE_BF16;
  if (s.d == 128) {
    if (bf) return bud ? launch_one<128, true, true, DP, FUSEDQ, PPT, LOADS>(p, capacity, stream, ev_start, ev_stop, max_wg)
                       : launch_one<128, true, false, DP, FUSEDQ, PPT, LOADS>(p, capacity, stream, ev_start, ev_stop, max_wg);
    return bud ? launch_one<128, false, true, DP, FUSEDQ, PPT, LOADS>(p, capacity, stream, ev_start, ev_stop, max_wg)
               : launch_one<128, false, false, DP, FUSEDQ, PPT, LOADS>(p, capacity, stream, ev_start, ev_stop, max_wg);
  }
  if (bf) return bud ? launch_one<64, true, true, DP, FUSEDQ, PPT, LOADS>(p, capacity, stream, ev_start, ev_stop, max_wg)
                     : launch_one<64, true, false, DP, FUSEDQ, PPT, LOADS>(p, capacity, stream, ev_start, ev_stop, max_wg);
  return bud ? launch_one<64, false, true, DP, FUSEDQ, PPT, LOADS>(p, capacity, stream, ev_start, ev_stop, max_wg)
             : launch_one<64, false, false, DP, FUSEDQ, PPT, LOADS>(p, capacity, stream, ev_start, ev_stop, max_wg);
}

// The instance with the fewest pages per task that holds one split: a task
// issues loads for all of its instance's pages, so a short split run by the
// 16-page instance would spend most of its loads on repeats.  Splits longer
// than 16 pages run on the 16-page instance as consecutive pieces.
template <bool FUSEDQ, int LOADS>
static hipError_t dispatch(const kvpage_shape& s, const AttnParams& p, int capacity, bool bud,
                           hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop,
                           int max_wg) {
  const int pages = s.split_tokens / kPage;
  if (pages <= 4) return dispatch_ppt<FUSEDQ, 4, LOADS>(s, p, capacity, bud, stream, ev_start, ev_stop, max_wg);
  if (pages <= 8) return dispatch_ppt<FUSEDQ, 8, LOADS>(s, p, capacity, bud, stream, ev_start, ev_stop, max_wg);
  return dispatch_ppt<FUSEDQ, 16, LOADS>(s, p, capacity, bud, stream, ev_start, ev_stop, max_wg);
}

// Wavefronts of one resident round per compute unit (one workgroup per CU).
int split_attn_waves_per_cu() { return kWavesPerGroup; }

// Most queue positions in one chunk of the schedule at this split.
int split_attn_chunk_max(int split_tokens) {
  return kRunMax / ((split_tokens + 16 * kPage - 1) / (16 * kPage));
}

// Fused queue build: B <= 64 sequences (one lane each in the task lookup).
bool split_attn_can_fuse_queue(const kvpage_shape& s) { return s.B >= 1 && s.B <= kWave; }

hipError_t launch_split_attn(const kvpage_shape& s, const void* q, const void* k_pool,
                             const void* v_pool, const int32_t* block_tables,
                             const kvpage_task* tasks, const int32_t* n_tasks, int32_t capacity,
                             void* workspace, const kvpage_budget* budget, hipStream_t stream,
                             hipEvent_t ev_start, hipEvent_t ev_stop, const int32_t* ctx_lens,
                             kvpage_task* tasks_out, int32_t* group_offsets_out,
                             int32_t* n_tasks_out, int32_t max_wg,
                             const int32_t* shared_pages) {
  const int G = s.Hq / s.Hkv;
  const WorkspaceView ws = ws_view(workspace, capacity, G, s.d);
  AttnParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k_pool = static_cast<const uint16_t*>(k_pool);
  p.v_pool = static_cast<const uint16_t*>(v_pool);
  p.block_tables = block_tables;
  p.tasks = tasks;
  p.n_tasks = n_tasks;
  p.ctx_lens = ctx_lens;
  p.tasks_out = tasks_out;
  p.group_offsets_out = group_offsets_out;
  p.n_tasks_out = n_tasks_out;
  p.split_tokens = s.split_tokens;
  p.ws_hdr = ws.hdr;
  p.ws_o = ws.o;
  p.ws_rm = ws.rm;
  p.ws_rl = ws.rl;
  p.page_mass = budget ? budget->page_mass : nullptr;
  p.s_prev = budget ? budget->s_prev : nullptr;
  p.page_max = budget ? budget->page_max : nullptr;
  p.alpha_fast = budget ? budget->alpha_fast : 0.f;
  p.alpha_slow = budget ? budget->alpha_slow : 0.f;
  p.B = s.B;
  p.Hq = s.Hq;
  p.Hkv = s.Hkv;
  p.G = G;
  p.max_pages = s.max_pages;
  p.num_pages = s.num_pages;
  p.capacity = capacity;
  p.scale = s.scale;
  p.c2 = s.scale * 1.4426950408889634f;
  p.inv_g = 1.0f / (float)G;
  p.nwaves = 0;
  p.div_split = div_magic((uint32_t)s.split_tokens);
  p.div_waves = div_magic(1);
  const bool fused = tasks_out != nullptr;
  const bool bud = budget != nullptr;
  const bool stream_kv = (s.flags & KVPAGE_FLAG_STREAM_KV) != 0;
  p.shared_pages = shared_pages;
  const int loads = !stream_kv ? kLoadsCached : (shared_pages ? kLoadsPrefix : kLoadsStream);
#define KV_DISPATCH(F, L) dispatch<F, L>(s, p, capacity, bud, stream, ev_start, ev_stop, max_wg)
  if (fused) {
    if (loads == kLoadsPrefix) return KV_DISPATCH(true, kLoadsPrefix);
    return loads == kLoadsStream ? KV_DISPATCH(true, kLoadsStream) : KV_DISPATCH(true, kLoadsCached);
  }
  if (loads == kLoadsPrefix) return KV_DISPATCH(false, kLoadsPrefix);
  return loads == kLoadsStream ? KV_DISPATCH(false, kLoadsStream) : KV_DISPATCH(false, kLoadsCached);
#undef KV_DISPATCH
}

}  // namespace kvpage
