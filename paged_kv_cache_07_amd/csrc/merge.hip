// Log-sum-exp merge of split partials, and the page-mass / summary finish.
//
// The split partials of one (sequence, query head) are combined in split
// order: with M = max_j m_j and w_j = 2^(m_j - M), out = sum_j w_j o_j /
// sum_j w_j l_j and lse = ln 2 * (M + log2 sum_j w_j l_j).  Page mass is the
// softmax weight of each logical page (GrowPage, Abstract: page-level KV
// budgeting), finished here from the per-task page sums that the attention
// kernel left relative to its own max.  The finish kernel also writes the
// fast/slow query-summary state of every (sequence, KV head).
#include <math.h>

#include "kvpage_common.h"

namespace kvpage {

constexpr int kMergeThreads = 256;
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

__device__ __forceinline__ float block_reduce(float v, bool is_max, float* scratch) {
  for (int off = 32; off > 0; off >>= 1) {
    const float o = __shfl_xor(v, off, kWave);
    v = is_max ? fmaxf(v, o) : v + o;
  }
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[w] = v;
  __syncthreads();
  float r = scratch[0];
  for (int i = 1; i < kMergeThreads / kWave; ++i) r = is_max ? fmaxf(r, scratch[i]) : r + scratch[i];
  return r;
}

template <bool BF>
__device__ __forceinline__ uint16_t to_bits(float x) {
  if constexpr (BF) return __builtin_bit_cast(uint16_t, (__bf16)x);
  else return __builtin_bit_cast(uint16_t, (_Float16)x);
}

template <bool BF>
__device__ __forceinline__ float q_value(const uint16_t* q, int64_t idx) {
  const uint32_t b16 = q[idx];
  if constexpr (BF) return __builtin_bit_cast(float, b16 << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)b16);
}

__device__ __forceinline__ int pages_of(int32_t ctx) {
  return ctx > 0 ? (ctx + kPage - 1) / kPage : 0;
}

// Budgeting finish for query head h of sequence b, given its merged lse
// (natural log, as stored).  Page p of the sequence lies in split
// p / pages_per_split of the (b, g) task range starting at `lo`; its raw sum
// (relative to that task's m) becomes the softmax weight of the page.  The
// workgroup of the group's first head also writes the page-max tails and the
// next query-summary state of (b, g).
template <bool BF>
__device__ void finish_head(const FinishParams& f, const float* ws_rm, int runlen, int b, int h,
                            int g, int hh, int B, int Hq, int Hkv, int G, int D, int lo,
                            float lse_nat) {
  const int npg = pages_of(f.ctx_lens[b]);
  const float lse2 = lse_nat * kLog2e;
  float* mrow = f.page_mass + ((int64_t)b * Hq + h) * f.max_pages;
  for (int pg = threadIdx.x; pg < f.max_pages; pg += kMergeThreads) {
    float v = 0.f;
    if (pg < npg) {
      const int run = run_of(lo, lo + pg / f.pages_per_split, runlen);
      v = mrow[pg] * __builtin_amdgcn_exp2f(ws_rm[(int64_t)run * G + hh] - lse2);
    }
    mrow[pg] = v;
  }
  if (hh != 0) return;
  for (int k = 0; k < 2; ++k) {
    float* prow = f.page_max + (((int64_t)k * B + b) * Hkv + g) * f.max_pages;
    for (int pg = npg + threadIdx.x; pg < f.max_pages; pg += kMergeThreads) prow[pg] = -INFINITY;
  }
  const int64_t q0 = ((int64_t)b * Hq + (int64_t)g * G) * D;
  for (int x = threadIdx.x; x < 2 * D; x += kMergeThreads) {
    const int which = x >= D;
    const int d = x - which * D;
    float acc = q_value<BF>(f.q, q0 + d);
    for (int hq = 1; hq < G; ++hq) acc = __fadd_rn(acc, q_value<BF>(f.q, q0 + (int64_t)hq * D + d));
    const int64_t si = (((int64_t)which * B + b) * Hkv + g) * D + d;
    f.s_next[si] = ema_step(f.s_prev[si], __fmul_rn(acc, f.inv_g), which ? f.alpha_slow : f.alpha_fast);
  }
}

// One workgroup per (sequence, query head).  With FINISH the budgeting
// outputs of that head are finished in the same pass.  Thread (r, c) owns
// output columns 4c..4c+3 and the splits j = r, r + R, ...; it loads U of
// them at a time (partial row, m and l together, so one memory latency per
// batch), keeps its own running max, and the threads are combined at the end
// with the same log-sum-exp rule in a fixed order.
template <int D, bool BF, bool FINISH>
__global__ void __launch_bounds__(kMergeThreads) merge_kernel(const MergeParams p) {
  constexpr int C4 = D / 4;                // float4 columns of one output row
  constexpr int R = kMergeThreads / C4;    // partial rows read side by side
  constexpr int U = 16;                    // splits per thread per batch
  constexpr int NW = kMergeThreads / kWave;
  __shared__ float scratch[NW];
  __shared__ float4 part[R][C4];
  __shared__ float part_m[R], part_l[R];

  const int bh = blockIdx.x;
  const int b = bh / p.Hq, h = bh % p.Hq;
  const int g = h / p.G, hh = h % p.G;
  const int lo = min(p.group_offsets[b * p.Hkv + g], p.capacity);
  const int hi = min(p.group_offsets[b * p.Hkv + g + 1], p.capacity);
  const int n = hi - lo;
  const int tid = threadIdx.x;
  uint16_t* orow = p.out + (int64_t)bh * D;
  if (n <= 0) {
    for (int d = tid; d < D; d += kMergeThreads) orow[d] = 0;
    if (tid == 0) p.lse[bh] = -INFINITY;
    if constexpr (FINISH)
      finish_head<BF>(p.fin, p.ws_rm, max(1, p.ws_hdr[0]), b, h, g, hh, p.B, p.Hq, p.Hkv, p.G, D, lo, -INFINITY);
    return;
  }
  const int c = tid % C4, r = tid / C4;
  // Run partials of this (b, g): queue positions lo, then multiples of the run length.
  const int runlen = max(1, p.ws_hdr[0]);
  const int nrun = run_count(lo, hi, runlen);

  float tm = -INFINITY, tl = 0.f;               // this thread's running max / sum
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = r; j0 < nrun; j0 += R * U) {
    float4 v[U];
    float mv[U], lv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * R;
      if (j < nrun) {
        const int64_t slot = run_slot(lo, j, runlen);
        v[u] = *reinterpret_cast<const float4*>(p.ws_o + (slot * p.G + hh) * D + 4 * c);
        mv[u] = p.ws_rm[slot * p.G + hh];
        lv[u] = p.ws_rl[slot * p.G + hh];
      } else {
        v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        mv[u] = -INFINITY;
        lv[u] = 0.f;
      }
    }
    float bm = mv[0];
#pragma unroll
    for (int u = 1; u < U; ++u) bm = fmaxf(bm, mv[u]);
    const float nm = fmaxf(tm, bm);
    const float sc = tm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(tm - nm);
    acc.x *= sc;
    acc.y *= sc;
    acc.z *= sc;
    acc.w *= sc;
    tl *= sc;
    tm = nm;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float wu = mv[u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mv[u] - nm);
      acc.x = fmaf(wu, v[u].x, acc.x);
      acc.y = fmaf(wu, v[u].y, acc.y);
      acc.z = fmaf(wu, v[u].z, acc.z);
      acc.w = fmaf(wu, v[u].w, acc.w);
      tl = fmaf(wu, lv[u], tl);
    }
  }
  const float M = block_reduce(tm, true, scratch);
  const float sc = tm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(tm - M);
  part[r][c] = make_float4(acc.x * sc, acc.y * sc, acc.z * sc, acc.w * sc);
  if (c == 0) {
    part_m[r] = tm;
    part_l[r] = tl * sc;
  }
  __syncthreads();
  float L = 0.f;
  for (int i = 0; i < R; ++i) L += part_l[i];
  if (r == 0) {
    float4 t = part[0][c];
    for (int i = 1; i < R; ++i) {
      t.x += part[i][c].x;
      t.y += part[i][c].y;
      t.z += part[i][c].z;
      t.w += part[i][c].w;
    }
    const float inv = 1.0f / L;
    const uint32_t w0 = to_bits<BF>(t.x * inv) | ((uint32_t)to_bits<BF>(t.y * inv) << 16);
    const uint32_t w1 = to_bits<BF>(t.z * inv) | ((uint32_t)to_bits<BF>(t.w * inv) << 16);
    *reinterpret_cast<uint2*>(orow + 4 * c) = make_uint2(w0, w1);
  }
  const float lse_nat = (M + log2f(L)) * kLn2;
  if (tid == 0) p.lse[bh] = lse_nat;
  if constexpr (FINISH)
    finish_head<BF>(p.fin, p.ws_rm, max(1, p.ws_hdr[0]), b, h, g, hh, p.B, p.Hq, p.Hkv, p.G, D, lo, lse_nat);
}

// Standalone finish (after a merge already wrote lse): one workgroup per
// (sequence, query head).
template <bool BF>
__global__ void __launch_bounds__(kMergeThreads) finish_kernel(const MergeParams p, int D) {
  const int bh = blockIdx.x;
  const int b = bh / p.Hq, h = bh % p.Hq;
  const int g = h / p.G, hh = h % p.G;
  const int lo = min(p.group_offsets[b * p.Hkv + g], p.capacity);
  finish_head<BF>(p.fin, p.ws_rm, max(1, p.ws_hdr[0]), b, h, g, hh, p.B, p.Hq, p.Hkv, p.G, D, lo, p.lse[bh]);
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

template <bool FINISH>
static void launch_merge_variant(const kvpage_shape& s, const MergeParams& p, hipStream_t stream) {
  const int grid = s.B * s.Hq;
  const bool bf = s.dtype == KVPAGE_BF16;
  if (s.d == 128) {
    if (bf) hipLaunchKernelGGL((merge_kernel<128, true, FINISH>), dim3(grid), dim3(kMergeThreads), 0, stream, p);
    else hipLaunchKernelGGL((merge_kernel<128, false, FINISH>), dim3(grid), dim3(kMergeThreads), 0, stream, p);
  } else {
    if (bf) hipLaunchKernelGGL((merge_kernel<64, true, FINISH>), dim3(grid), dim3(kMergeThreads), 0, stream, p);
    else hipLaunchKernelGGL((merge_kernel<64, false, FINISH>), dim3(grid), dim3(kMergeThreads), 0, stream, p);
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
  const int grid = s.B * s.Hq;
  if (s.dtype == KVPAGE_BF16)
    hipLaunchKernelGGL(finish_kernel<true>, dim3(grid), dim3(kMergeThreads), 0, stream, p, s.d);
  else
    hipLaunchKernelGGL(finish_kernel<false>, dim3(grid), dim3(kMergeThreads), 0, stream, p, s.d);
  return hipGetLastError();
}

}  // namespace kvpage
