// Log-sum-exp merge of split partials, and the page-mass / summary finish.
//
// The run partials of one (sequence, query head) are combined in a fixed
// order (per-thread sums, then butterflies, so the bits do not depend on
// timing): with M = max_j m_j and w_j = 2^(m_j - M), out = sum_j w_j o_j /
// sum_j w_j l_j and lse = ln 2 * (M + log2 sum_j w_j l_j).  Page mass is the
// softmax weight of each logical page (GrowPage, Abstract: page-level KV
// budgeting), finished here from the per-task page sums that the attention
// kernel left relative to its own max.  The finish kernel also writes the
// fast/slow query-summary state of every (sequence, KV head).
#include <math.h>

#include "kvpage_common.h"

namespace kvpage {

constexpr int kMergeThreads = 256;
constexpr int kPagesPerThread = 4;
constexpr int kPagesPerBlock = kMergeThreads * kPagesPerThread;
constexpr int kMaxGroup = 8;   // query heads per KV head supported
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kLog2e = 1.4426950408889634f;

struct FinishParams {
  float* page_mass;
  float* page_max;
  const float* s_prev;
  float* s_next;
  float alpha_fast, alpha_slow;
  const uint16_t* q;
  const int32_t* ctx_lens;
  int32_t max_pages, pages_per_split;
  float inv_g;
};

struct MergeParams {
  const int32_t* group_offsets;
  const int32_t* ws_hdr;
  const float* ws_o;
  const float* ws_rm;
  const float* ws_rl;
  uint16_t* out;
  float* lse;
  int32_t B, Hq, Hkv, G, capacity;
  FinishParams fin;
};

// Two (max, sum) statistics in the log2 domain combine as m = max(m1, m2),
// l = l1 2^(m1 - m) + l2 2^(m2 - m); a -inf max carries no mass.
__device__ __forceinline__ void ml_combine(float& m, float& l, float m2, float l2) {
  const float nm = fmaxf(m, m2);
  l = (m == -INFINITY ? 0.f : l * __builtin_amdgcn_exp2f(m - nm)) +
      (m2 == -INFINITY ? 0.f : l2 * __builtin_amdgcn_exp2f(m2 - nm));
  m = nm;
}

// Workgroup-wide combine of every thread's (m, l): the maximum M, then the
// sum of l 2^(m - M), each a butterfly per wavefront (a + b == b + a bit for
// bit, so every lane ends with the same value) followed by the wavefronts'
// results in wavefront order; every thread returns the same bits.  Called
// once per kernel (scratch, 2 floats per wavefront, is not reused).  Two
// plain reductions measured faster than one butterfly over (m, l) pairs,
// which needs two exponentials per step.
__device__ __forceinline__ void block_ml(float& m, float& l, float* scratch) {
  constexpr int NW = kMergeThreads / kWave;
  const int w = threadIdx.x / kWave;
  const bool lead = (threadIdx.x & (kWave - 1)) == 0;
  float v = m;
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  if (lead) scratch[w] = v;
  __syncthreads();
  float M = scratch[0];
  for (int i = 1; i < NW; ++i) M = fmaxf(M, scratch[i]);
  float u = m == -INFINITY ? 0.f : l * __builtin_amdgcn_exp2f(m - M);
  for (int off = 32; off > 0; off >>= 1) u += __shfl_xor(u, off, kWave);
  if (lead) scratch[NW + w] = u;
  __syncthreads();
  float L = scratch[NW];
  for (int i = 1; i < NW; ++i) L += scratch[NW + i];
  m = M;
  l = L;
}

template <bool BF>
__device__ __forceinline__ uint16_t to_bits(float x) {
  if constexpr (BF) return __builtin_bit_cast(uint16_t, (__bf16)x);
  else return __builtin_bit_cast(uint16_t, (_Float16)x);
}

template <bool BF>
__device__ __forceinline__ float bits_value(uint32_t b16) {
  if constexpr (BF) return __builtin_bit_cast(float, b16 << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)b16);
}

__device__ __forceinline__ int pages_of(int32_t ctx) {
  return ctx > 0 ? (ctx + kPage - 1) / kPage : 0;
}

// One (sequence, query head) row: its KV head, its head inside the group, and
// the run partials of the group's task range [lo, lo + n).  All of a
// workgroup's row metadata is requested at once.
struct Row {
  int b, h, g, hh, lo, n, runlen, off, nrun, npg;
};

// The buffers of the row metadata loads and the shape fields their addresses
// need.  The merge and finish kernels take these as leading kernel arguments
// of their own (KV_ROW_LEAD_ARGS): gfx950 can preload leading scalar kernel
// arguments into SGPRs at wave launch, so a workgroup's first loads do not
// wait for the kernel-argument block.
struct RowLead {
  const int32_t* group_offsets;
  const int32_t* ws_hdr;
  const int32_t* ctx_lens;
  int32_t B, Hq, Hkv, G;
};
#define KV_ROW_LEAD_ARGS                                                               \
  const int32_t *lead_go, const int32_t *lead_hdr, const int32_t *lead_ctx, int32_t lead_b, \
      int32_t lead_hq, int32_t lead_hkv, int32_t lead_g
#define KV_ROW_LEAD RowLead{lead_go, lead_hdr, lead_ctx, lead_b, lead_hq, lead_hkv, lead_g}
#define KV_ROW_LEAD_OF(p) \
  (p).group_offsets, (p).ws_hdr, (p).fin.ctx_lens, (p).B, (p).Hq, (p).Hkv, (p).G

__device__ __forceinline__ Row row_of(const MergeParams& p, const RowLead& ld, int bh,
                                      bool need_pages) {
  Row r;
  r.b = bh / ld.Hq;
  r.h = bh % ld.Hq;
  r.g = r.h / ld.G;
  r.hh = r.h % ld.G;
  const int lo = ld.group_offsets[r.b * ld.Hkv + r.g];
  const int hi = ld.group_offsets[r.b * ld.Hkv + r.g + 1];
  const int runlen = ld.ws_hdr[0];
  const int ncls = ld.ws_hdr[1];
  const int seq_lo = ld.group_offsets[r.b * ld.Hkv];
  const int seq_lo1 = ld.group_offsets[r.b * ld.Hkv + 1];
  const int ctx = need_pages ? clamp_ctx(ld.ctx_lens[r.b], p.fin.max_pages) : 0;
  r.lo = min(max(lo, 0), p.capacity);
  r.n = max(min(hi, p.capacity) - r.lo, 0);
  r.runlen = max(1, runlen);
  // Where the group's first task sits inside its chunk of the schedule.  With
  // the queue taken as ncls classes (KV heads g % ncls), class-local position
  // of the group's first task: start / ncls + (g / ncls) * ns for the
  // sequence's first queue position `start` and ns tasks per KV head.
  if (ncls > 1 && ld.Hkv % ncls == 0) {
    const int start = max(seq_lo, 0);
    const int ns = max(seq_lo1 - start, 0);
    r.off = (start / ncls + (r.g / ncls) * ns) % r.runlen;
  } else {
    r.off = r.lo % r.runlen;
  }
  r.nrun = run_count(r.lo, r.lo + r.n, r.runlen, r.off);
  r.npg = pages_of(ctx);
  return r;
}

// Index into [capacity][G] arrays of run j of the row, clamped into the
// arrays so that a load for a missing run (j >= nrun) stays in bounds.
__device__ __forceinline__ int64_t run_index(const MergeParams& p, const Row& r, int j) {
  const int jj = min(j, max(r.nrun - 1, 0));
  const int slot = min(run_slot(r.lo, jj, r.runlen, r.off), p.capacity - 1);
  return (int64_t)slot * p.G + r.hh;
}

// Run statistics (m_j, l_j) of run j = thread, requested with the other
// loads of the row.  The loads are unconditional (a missing run re-reads the
// last one and is dropped afterwards): a load under a branch would make the
// compiler wait for everything in flight before the next use.
struct StatLoads {
  float m, l;
  __device__ __forceinline__ void issue(const MergeParams& p, const Row& r) {
    const int64_t i = run_index(p, r, threadIdx.x);
    m = p.ws_rm[i];
    l = p.ws_rl[i];
  }
};

// Log-sum-exp statistics of a row over its run partials: M = max_j m_j and
// L = sum_j 2^(m_j - M) l_j (log2 domain), in a fixed order, so that every
// workgroup that needs them gets the same bits.  Returns the natural-log lse
// exactly as it is stored (-inf for an empty row).
__device__ float row_lse(const MergeParams& p, const Row& r, const StatLoads& first,
                         float* scratch, float* L_out, float* M_out) {
  float tm = (int)threadIdx.x < r.nrun ? first.m : -INFINITY;
  float tl = (int)threadIdx.x < r.nrun ? first.l : 0.f;
  for (int j = threadIdx.x + kMergeThreads; j < r.nrun; j += kMergeThreads) {
    const int64_t i = run_index(p, r, j);
    ml_combine(tm, tl, p.ws_rm[i], p.ws_rl[i]);
  }
  block_ml(tm, tl, scratch);
  *M_out = tm;
  *L_out = tl;
  return r.n > 0 ? (tm + log2f(tl)) * kLn2 : -INFINITY;
}

// A 32-bit buffer view of `bytes` bytes at `base`: loads past the end read 0
// and stores past the end are dropped by the hardware, so masked stores need
// no branch (a masked lane stores to an offset past the end).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_view(void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, 0x00020000);
}
constexpr int kDropOffset = 0x7ffffff0;

__device__ __forceinline__ void buffer_store_f32(float v, __amdgpu_buffer_rsrc_t rs, int byte_off) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rs, byte_off, 0, 0);
}

// Output row of (b, h): out = sum_j 2^(m_j - M) o_j / L over the row's run
// partials.  The D columns are split into CG groups, one per workgroup of the
// row.  Thread (rr, c) owns float4 column c of its group and the runs rr,
// rr + R, ..., kMergeBatch at a time; the R thread sums are added by a
// butterfly inside each wavefront and then across wavefronts in a fixed
// order.  The first batch is requested before the row statistics.
constexpr int kMergeBatch = 4;

template <int D, int CG>
struct MergeLoads {
  static constexpr int C4 = D / 4 / CG;   // float4 columns per workgroup
  static constexpr int R = kMergeThreads / C4;
  float4 v[kMergeBatch];
  float m[kMergeBatch];

  __device__ __forceinline__ void issue(const MergeParams& p, const Row& r, int j0, int col0) {
    const int c = threadIdx.x % C4;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int j = j0 + u * R;
      const int64_t i = run_index(p, r, j);
      v[u] = *reinterpret_cast<const float4*>(p.ws_o + i * D + col0 + 4 * c);
      m[u] = p.ws_rm[i];
    }
  }

  // Runs j0 + u*R at or past nrun (re-reads of the last run) weigh 0.
  __device__ __forceinline__ void add_to(float4& acc, float M, int j0, int nrun) const {
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const bool live = j0 + u * R < nrun && m[u] != -INFINITY;
      const float w = live ? __builtin_amdgcn_exp2f(m[u] - M) : 0.f;
      acc.x = fmaf(w, v[u].x, acc.x);
      acc.y = fmaf(w, v[u].y, acc.y);
      acc.z = fmaf(w, v[u].z, acc.z);
      acc.w = fmaf(w, v[u].w, acc.w);
    }
  }
};

template <int D, bool BF, int CG>
__device__ void merge_cols(const MergeParams& p, const Row& r, int bh, int col0,
                           const MergeLoads<D, CG>& first, float M, float L) {
  using ML = MergeLoads<D, CG>;
  static_assert(ML::C4 <= kWave, "a wavefront holds every column of its group");
  constexpr int NW = kMergeThreads / kWave;
  __shared__ float4 part[NW][ML::C4];
  const int tid = threadIdx.x;
  const int c = tid % ML::C4, rr = tid / ML::C4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  first.add_to(acc, M, rr, r.nrun);
  for (int j0 = rr + ML::R * kMergeBatch; j0 < r.nrun; j0 += ML::R * kMergeBatch) {
    ML more;
    more.issue(p, r, j0, col0);
    more.add_to(acc, M, j0, r.nrun);
  }
  // Lanes c, c + C4, ... of a wavefront hold column c.
#pragma unroll
  for (int off = ML::C4; off < kWave; off <<= 1) {
    acc.x += __shfl_xor(acc.x, off, kWave);
    acc.y += __shfl_xor(acc.y, off, kWave);
    acc.z += __shfl_xor(acc.z, off, kWave);
    acc.w += __shfl_xor(acc.w, off, kWave);
  }
  if ((tid & (kWave - 1)) < ML::C4) part[tid / kWave][c] = acc;
  __syncthreads();
  if (rr == 0) {
    float4 t = part[0][c];
    for (int i = 1; i < NW; ++i) {
      t.x += part[i][c].x;
      t.y += part[i][c].y;
      t.z += part[i][c].z;
      t.w += part[i][c].w;
    }
    uint32_t w0 = 0, w1 = 0;
    if (r.n > 0) {
      const float inv = 1.0f / L;
      w0 = to_bits<BF>(t.x * inv) | ((uint32_t)to_bits<BF>(t.y * inv) << 16);
      w1 = to_bits<BF>(t.z * inv) | ((uint32_t)to_bits<BF>(t.w * inv) << 16);
    }
    *reinterpret_cast<uint2*>(p.out + (int64_t)bh * D + col0 + 4 * c) = make_uint2(w0, w1);
  }
}

// Budgeting finish of one slice of kPagesPerBlock logical pages of row (b, h)
// (GrowPage, Abstract: page-level KV budgeting).  Page pg of the sequence
// lies in split pg / pages_per_split of the group's task range; the attention
// kernel left its raw sum relative to the reference max of the run holding
// that task, so its softmax weight is raw * 2^(m_run - lse / ln 2).  Pages
// past the sequence get mass 0; for the group's first head the slice also
// sets the page-max tails to -inf.
struct PageLoads {
  float raw[kPagesPerThread], m[kPagesPerThread];

  __device__ __forceinline__ void issue(const MergeParams& p, const Row& r, int bh, int slice) {
    const FinishParams& f = p.fin;
    const float* mrow = f.page_mass + (int64_t)bh * f.max_pages;
    const int last = max(r.npg - 1, 0);
#pragma unroll
    for (int k = 0; k < kPagesPerThread; ++k) {
      const int pg = min(slice * kPagesPerBlock + k * kMergeThreads + (int)threadIdx.x, last);
      raw[k] = mrow[pg];
      const int run = run_of(r.lo, r.lo + pg / f.pages_per_split, r.runlen, r.off);
      m[k] = p.ws_rm[(int64_t)min(run, p.capacity - 1) * p.G + r.hh];
    }
  }
};

template <bool BF>
__device__ void finish_slice(const MergeParams& p, const Row& r, int bh, int slice, int D,
                             const PageLoads& pl, float lse_nat) {
  const FinishParams& f = p.fin;
  const float lse2 = lse_nat * kLog2e;
  const auto mass = buffer_view(f.page_mass + (int64_t)bh * f.max_pages, f.max_pages * 4);
#pragma unroll
  for (int k = 0; k < kPagesPerThread; ++k) {
    const int pg = slice * kPagesPerBlock + k * kMergeThreads + (int)threadIdx.x;
    const float v = pg < r.npg ? pl.raw[k] * __builtin_amdgcn_exp2f(pl.m[k] - lse2) : 0.f;
    buffer_store_f32(v, mass, pg * 4);
  }
  if (r.hh != 0) return;
  for (int which = 0; which < 2; ++which) {
    const auto pmax = buffer_view(
        f.page_max + (((int64_t)which * p.B + r.b) * p.Hkv + r.g) * f.max_pages, f.max_pages * 4);
#pragma unroll
    for (int k = 0; k < kPagesPerThread; ++k) {
      const int pg = slice * kPagesPerBlock + k * kMergeThreads + (int)threadIdx.x;
      buffer_store_f32(-INFINITY, pmax, pg >= r.npg ? pg * 4 : kDropOffset);
    }
  }
}

// Next query-summary state of (b, g), elements d and d + 1 of both
// summaries: the group-mean query (heads added in head order, then scaled by
// 1/G, the attention kernel's expression) and one EMA step of the fast and
// the slow summary (GrowPage, Technical Details).  It needs only q and
// s_prev; each query load brings both elements of a head.
template <bool BF>
struct SummaryStep {
  uint32_t qb[kMaxGroup];   // bits of q[b, g*G + head, d .. d+1]
  float sp[2][2];           // s_prev[which][b, g, d .. d+1]
  int64_t si[2];            // index of (which, b, g, d)

  __device__ __forceinline__ void issue(const MergeParams& p, int b, int g, int d, int D) {
    const FinishParams& f = p.fin;
    const int64_t q0 = ((int64_t)b * p.Hq + (int64_t)g * p.G) * D + d;
#pragma unroll
    for (int hq = 0; hq < kMaxGroup; ++hq)
      qb[hq] = *reinterpret_cast<const uint32_t*>(f.q + q0 + (int64_t)min(hq, p.G - 1) * D);
    si[0] = ((int64_t)b * p.Hkv + g) * D + d;
    si[1] = si[0] + (int64_t)p.B * p.Hkv * D;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      sp[w][0] = f.s_prev[si[w]];
      sp[w][1] = f.s_prev[si[w] + 1];
    }
  }

  __device__ __forceinline__ void store(const MergeParams& p) const {
    const FinishParams& f = p.fin;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      float acc = bits_value<BF>((qb[0] >> (16 * e)) & 0xffffu);
#pragma unroll
      for (int hq = 1; hq < kMaxGroup; ++hq)
        if (hq < p.G) acc = add_rn(acc, bits_value<BF>((qb[hq] >> (16 * e)) & 0xffffu));
      const float qbar = mul_rn(acc, f.inv_g);
      f.s_next[si[0] + e] = ema_step(sp[0][e], qbar, f.alpha_fast);
      f.s_next[si[1] + e] = ema_step(sp[1][e], qbar, f.alpha_slow);
    }
  }
};

// Each row has nsub = max(CG, nslice) workgroups: workgroup k merges column
// group k (k < CG) and, with FINISH, finishes page slice k (k < nslice).
// Once the row's metadata is in, every load of the workgroup goes out at
// once and unconditionally (a workgroup with no column group or no slice
// loads its neighbour's, which stay in cache), so the data arrives in one
// memory round trip and the compiler's wait counts stay exact.
template <int D, bool BF, bool FINISH, int CG>
__global__ void __launch_bounds__(kMergeThreads) merge_kernel(KV_ROW_LEAD_ARGS, int nslice,
                                                              int nsub, const MergeParams p) {
  __shared__ float scratch[2 * kMergeThreads / kWave];
  const int bh = blockIdx.x / nsub, sub = blockIdx.x % nsub;
  const Row r = row_of(p, KV_ROW_LEAD, bh, FINISH);
  const bool do_cols = sub < CG;
  const bool do_pages = FINISH && sub < nslice;
  const int col0 = min(sub, CG - 1) * (D / CG);
  MergeLoads<D, CG> ml;
  ml.issue(p, r, threadIdx.x / MergeLoads<D, CG>::C4, col0);
  PageLoads pl;
  if constexpr (FINISH) pl.issue(p, r, bh, min(sub, nslice - 1));
  StatLoads st;
  st.issue(p, r);
  float M, L;
  const float lse_nat = row_lse(p, r, st, scratch, &L, &M);
  if (do_cols) merge_cols<D, BF, CG>(p, r, bh, col0, ml, M, L);
  if (sub == 0 && threadIdx.x == 0) p.lse[bh] = lse_nat;
  if (do_pages) finish_slice<BF>(p, r, bh, sub, D, pl, lse_nat);
  // The group's first head, first workgroup, also steps the summaries.  (The
  // same loads requested at kernel start measured slower in every merge
  // kernel: they delay that workgroup's metadata round trip.)
  if (FINISH && sub == 0 && r.hh == 0 && (int)threadIdx.x < D / 2) {
    SummaryStep<BF> ss;
    ss.issue(p, r.b, r.g, 2 * threadIdx.x, D);
    ss.store(p);
  }
}

// ---- Many rows: one wavefront per (row, page slice) ----------------------
//
// With hundreds of rows each has few runs, and the cost is the chain of
// dependent round trips per workgroup and how many are resident.  Here a
// wavefront owns one (row, slice of kPagesPerBlock pages): it requests the
// row's run statistics, (slice 0) the run partials of its 64 x D/64 output
// columns, and its slice's raw page sums and run maxima at once, then reduces
// with cross-lane shuffles only (no LDS, no barrier).  The butterfly gives
// every lane, and every wavefront of the row, the same bits.
constexpr int kWavePagesPerLane = kPagesPerBlock / kWave;   // 16
constexpr int kWaveRunBatch = 4;

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

template <int D, bool BF, bool FINISH>
__global__ void __launch_bounds__(kMergeThreads) merge_wave_kernel(KV_ROW_LEAD_ARGS, int nslice,
                                                                   const MergeParams p) {
  constexpr int CPL = D / kWave;   // output columns per lane (1 or 2)
  const int lane = threadIdx.x & (kWave - 1);
  const int item = blockIdx.x * (kMergeThreads / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (item >= lead_b * lead_hq * nslice) return;
  const int bh = item / nslice, slice = item % nslice;
  const Row r = row_of(p, KV_ROW_LEAD, bh, FINISH);
  const bool do_out = slice == 0;

  // Run partials of this lane's columns, first batch.
  float ov[kWaveRunBatch][CPL], om[kWaveRunBatch];
  auto issue_runs = [&](int j0) {
#pragma unroll
    for (int u = 0; u < kWaveRunBatch; ++u) {
      const int64_t i = run_index(p, r, j0 + u);
      const float* src = p.ws_o + i * D + CPL * lane;
#pragma unroll
      for (int x = 0; x < CPL; ++x) ov[u][x] = src[x];
      om[u] = p.ws_rm[i];
    }
  };
  // Every load goes out unconditionally (slices past 0 load the partials
  // too, and missing runs re-read the last one), so all arrive in one round
  // trip and the compiler's wait counts stay exact.
  issue_runs(0);
  // Raw page sums of the slice and the run maxima they are relative to.
  float raw[kWavePagesPerLane], rmx[kWavePagesPerLane];
  if constexpr (FINISH) {
    const FinishParams& f = p.fin;
    const float* mrow = f.page_mass + (int64_t)bh * f.max_pages;
    const int last = max(r.npg - 1, 0);
#pragma unroll
    for (int k = 0; k < kWavePagesPerLane; ++k) {
      const int pg = min(slice * kPagesPerBlock + k * kWave + lane, last);
      raw[k] = mrow[pg];
      const int run = run_of(r.lo, r.lo + pg / f.pages_per_split, r.runlen, r.off);
      rmx[k] = p.ws_rm[(int64_t)min(run, p.capacity - 1) * p.G + r.hh];
    }
  }
  // Row statistics over all runs, lanes strided over the runs.
  const int64_t i0 = run_index(p, r, lane);
  const float m0 = p.ws_rm[i0], l0 = p.ws_rl[i0];
  float tm = lane < r.nrun ? m0 : -INFINITY;
  float tl = lane < r.nrun ? l0 : 0.f;
  for (int j = lane + kWave; j < r.nrun; j += kWave) {
    const int64_t i = run_index(p, r, j);
    ml_combine(tm, tl, p.ws_rm[i], p.ws_rl[i]);
  }
  const float M = wave_max(tm);
  const float L = wave_sum(tm == -INFINITY ? 0.f : tl * __builtin_amdgcn_exp2f(tm - M));
  const float lse_nat = r.n > 0 ? (M + log2f(L)) * kLn2 : -INFINITY;

  if (do_out) {
    float acc[CPL];
#pragma unroll
    for (int x = 0; x < CPL; ++x) acc[x] = 0.f;
    for (int j0 = 0;;) {
#pragma unroll
      for (int u = 0; u < kWaveRunBatch; ++u) {
        const bool live = j0 + u < r.nrun && om[u] != -INFINITY;
        const float w = live ? __builtin_amdgcn_exp2f(om[u] - M) : 0.f;
#pragma unroll
        for (int x = 0; x < CPL; ++x) acc[x] = fmaf(w, ov[u][x], acc[x]);
      }
      j0 += kWaveRunBatch;
      if (j0 >= r.nrun) break;
      issue_runs(j0);
    }
    const float inv = r.n > 0 ? 1.0f / L : 0.f;
    uint16_t* orow = p.out + (int64_t)bh * D + CPL * lane;
#pragma unroll
    for (int x = 0; x < CPL; ++x) orow[x] = r.n > 0 ? to_bits<BF>(acc[x] * inv) : (uint16_t)0;
    if (lane == 0) p.lse[bh] = lse_nat;
  }
  if constexpr (FINISH) {
    const FinishParams& f = p.fin;
    const float lse2 = lse_nat * kLog2e;
    const auto mass = buffer_view(f.page_mass + (int64_t)bh * f.max_pages, f.max_pages * 4);
#pragma unroll
    for (int k = 0; k < kWavePagesPerLane; ++k) {
      const int pg = slice * kPagesPerBlock + k * kWave + lane;
      const float v = pg < r.npg ? raw[k] * __builtin_amdgcn_exp2f(rmx[k] - lse2) : 0.f;
      buffer_store_f32(v, mass, pg * 4);
    }
    if (r.hh != 0) return;
    for (int which = 0; which < 2; ++which) {
      const auto pmax = buffer_view(
          f.page_max + (((int64_t)which * p.B + r.b) * p.Hkv + r.g) * f.max_pages, f.max_pages * 4);
#pragma unroll
      for (int k = 0; k < kWavePagesPerLane; ++k) {
        const int pg = slice * kPagesPerBlock + k * kWave + lane;
        buffer_store_f32(-INFINITY, pmax, pg >= r.npg ? pg * 4 : kDropOffset);
      }
    }
    // The group's first head, slice 0, also steps the summaries (elements
    // 2*lane and 2*lane + 1).
    if (slice == 0 && 2 * lane < D) {
      SummaryStep<BF> ss;
      ss.issue(p, r.b, r.g, 2 * lane, D);
      ss.store(p);
    }
  }
}

// Standalone finish after a merge that already wrote lse: one workgroup per
// slice of pages of one row.
template <bool BF>
__global__ void __launch_bounds__(kMergeThreads) finish_kernel(KV_ROW_LEAD_ARGS, int nslice,
                                                               const MergeParams p, int D) {
  const int bh = blockIdx.x / nslice, slice = blockIdx.x % nslice;
  const Row r = row_of(p, KV_ROW_LEAD, bh, true);
  PageLoads pl;
  pl.issue(p, r, bh, slice);
  finish_slice<BF>(p, r, bh, slice, D, pl, p.lse[bh]);
  if (slice == 0 && r.hh == 0 && (int)threadIdx.x < D / 2) {
    SummaryStep<BF> ss;
    ss.issue(p, r.b, r.g, 2 * threadIdx.x, D);
    ss.store(p);
  }
}

static MergeParams merge_params(const kvpage_shape& s, const int32_t* group_offsets,
                                int32_t capacity, const void* workspace, void* out, float* lse,
                                const kvpage_budget* bud, const void* q, const int32_t* ctx_lens) {
  const int G = s.Hq / s.Hkv;
  const WorkspaceView ws = ws_view(const_cast<void*>(workspace), capacity, G, s.d);
  MergeParams p;
  p.group_offsets = group_offsets;
  p.ws_hdr = ws.hdr;
  p.ws_o = ws.o;
  p.ws_rm = ws.rm;
  p.ws_rl = ws.rl;
  p.out = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.B = s.B;
  p.Hq = s.Hq;
  p.Hkv = s.Hkv;
  p.G = G;
  p.capacity = capacity;
  p.fin.page_mass = bud ? bud->page_mass : nullptr;
  p.fin.page_max = bud ? bud->page_max : nullptr;
  p.fin.s_prev = bud ? bud->s_prev : nullptr;
  p.fin.s_next = bud ? bud->s_next : nullptr;
  p.fin.alpha_fast = bud ? bud->alpha_fast : 0.f;
  p.fin.alpha_slow = bud ? bud->alpha_slow : 0.f;
  p.fin.q = static_cast<const uint16_t*>(q);
  p.fin.ctx_lens = ctx_lens;
  p.fin.max_pages = s.max_pages;
  p.fin.pages_per_split = s.split_tokens / s.page_size;
  p.fin.inv_g = 1.0f / (float)G;
  return p;
}

static int page_slices(const kvpage_shape& s) {
  return (s.max_pages + kPagesPerBlock - 1) / kPagesPerBlock;
}

// Few rows: each row's output is merged by 4 workgroups (a quarter of the
// columns each), so the partials are read by 4x as many compute units.  Many
// rows: one wavefront per (row, page slice).
constexpr int kWaveMergeMinRows = 512;

template <int D, bool BF, bool FINISH>
static void launch_merge_d(int rows, int nslice, const MergeParams& p, hipStream_t stream) {
  if (rows < kWaveMergeMinRows) {
    const int nsub = nslice > 4 ? nslice : 4;
    hipLaunchKernelGGL((merge_kernel<D, BF, FINISH, 4>), dim3(rows * nsub), dim3(kMergeThreads), 0,
                       stream, KV_ROW_LEAD_OF(p), nslice, nsub, p);
  } else {
    const int waves_per_block = kMergeThreads / kWave;
    const int grid = (rows * nslice + waves_per_block - 1) / waves_per_block;
    hipLaunchKernelGGL((merge_wave_kernel<D, BF, FINISH>), dim3(grid), dim3(kMergeThreads), 0,
                       stream, KV_ROW_LEAD_OF(p), nslice, p);
  }
}

template <bool FINISH>
static void launch_merge_variant(const kvpage_shape& s, const MergeParams& p, hipStream_t stream) {
  const int rows = s.B * s.Hq;
  const int nslice = FINISH ? page_slices(s) : 1;
  const bool bf = s.dtype == KVPAGE_BF16;
  if (s.d == 128) {
    if (bf) launch_merge_d<128, true, FINISH>(rows, nslice, p, stream);
    else launch_merge_d<128, false, FINISH>(rows, nslice, p, stream);
  } else {
    if (bf) launch_merge_d<64, true, FINISH>(rows, nslice, p, stream);
    else launch_merge_d<64, false, FINISH>(rows, nslice, p, stream);
  }
}

hipError_t launch_merge(const kvpage_shape& s, const int32_t* group_offsets, int32_t capacity,
                        const void* workspace, void* out, float* lse, hipStream_t stream) {
  if (s.B * s.Hq <= 0) return hipSuccess;
  const MergeParams p = merge_params(s, group_offsets, capacity, workspace, out, lse, nullptr,
                                     nullptr, nullptr);
  launch_merge_variant<false>(s, p, stream);
  return hipGetLastError();
}

hipError_t launch_merge_finish(const kvpage_shape& s, const kvpage_budget& bud, const void* q,
                               const int32_t* ctx_lens, const int32_t* group_offsets,
                               int32_t capacity, const void* workspace, void* out, float* lse,
                               hipStream_t stream) {
  if (s.B * s.Hq <= 0) return hipSuccess;
  const MergeParams p = merge_params(s, group_offsets, capacity, workspace, out, lse, &bud, q,
                                     ctx_lens);
  launch_merge_variant<true>(s, p, stream);
  return hipGetLastError();
}

hipError_t launch_page_mass(const kvpage_shape& s, const kvpage_budget& bud, const void* q,
                            const float* lse, const int32_t* ctx_lens,
                            const int32_t* group_offsets, int32_t capacity, const void* workspace,
                            hipStream_t stream) {
  if (s.B * s.Hq <= 0) return hipSuccess;
  const MergeParams p = merge_params(s, group_offsets, capacity, workspace, nullptr,
                                     const_cast<float*>(lse), &bud, q, ctx_lens);
  const int nslice = page_slices(s);
  const int grid = s.B * s.Hq * nslice;
  if (s.dtype == KVPAGE_BF16)
    hipLaunchKernelGGL(finish_kernel<true>, dim3(grid), dim3(kMergeThreads), 0, stream,
                       KV_ROW_LEAD_OF(p), nslice, p, s.d);
  else
    hipLaunchKernelGGL(finish_kernel<false>, dim3(grid), dim3(kMergeThreads), 0, stream,
                       KV_ROW_LEAD_OF(p), nslice, p, s.d);
  return hipGetLastError();
}

}  // namespace kvpage
