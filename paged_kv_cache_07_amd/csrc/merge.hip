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

struct MergeParams {
  const int32_t* group_offsets;
  const float* ws_o;
  const float* ws_m;
  const float* ws_l;
  uint16_t* out;
  float* lse;
  int32_t Hq, Hkv, G, capacity;
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

// One workgroup per (sequence, query head).
template <int D, bool BF>
__global__ void __launch_bounds__(kMergeThreads) merge_kernel(const MergeParams p) {
  constexpr int DP = D / 2;                  // float2 columns
  constexpr int SUB = kMergeThreads / DP;    // splits handled in parallel
  __shared__ float scratch[kMergeThreads / kWave];
  __shared__ float2 part[SUB][DP];

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
    return;
  }
  const float* m = p.ws_m + (int64_t)lo * p.G + hh;
  const float* l = p.ws_l + (int64_t)lo * p.G + hh;
  float mx = -INFINITY;
  for (int j = tid; j < n; j += kMergeThreads) mx = fmaxf(mx, m[(int64_t)j * p.G]);
  const float M = block_reduce(mx, true, scratch);
  float sl = 0.f;
  for (int j = tid; j < n; j += kMergeThreads)
    sl += __builtin_amdgcn_exp2f(m[(int64_t)j * p.G] - M) * l[(int64_t)j * p.G];
  const float L = block_reduce(sl, false, scratch);

  const int dp = tid % DP, s = tid / DP;
  float2 acc = make_float2(0.f, 0.f);
  const float* o = p.ws_o + ((int64_t)lo * p.G + hh) * D + 2 * dp;
  for (int j = s; j < n; j += SUB) {
    const float w = __builtin_amdgcn_exp2f(m[(int64_t)j * p.G] - M);
    const float2 v = *reinterpret_cast<const float2*>(o + (int64_t)j * p.G * D);
    acc.x = fmaf(w, v.x, acc.x);
    acc.y = fmaf(w, v.y, acc.y);
  }
  part[s][dp] = acc;
  __syncthreads();
  if (s == 0) {
    float2 t = part[0][dp];
    for (int i = 1; i < SUB; ++i) {
      t.x += part[i][dp].x;
      t.y += part[i][dp].y;
    }
    const float inv = 1.0f / L;
    orow[2 * dp] = to_bits<BF>(t.x * inv);
    orow[2 * dp + 1] = to_bits<BF>(t.y * inv);
  }
  if (tid == 0) p.lse[bh] = (M + log2f(L)) * 0.69314718055994531f;
}

struct MassParams {
  float* page_mass;
  float* page_max;
  const float* s_prev;
  float* s_next;
  float alpha_fast, alpha_slow;
  const uint16_t* q;
  const float* lse;
  const int32_t* ctx_lens;
  const int32_t* group_offsets;
  const float* ws_m;
  int32_t B, Hq, Hkv, G, D, max_pages, pages_per_split, capacity;
  float inv_g;
  int64_t n_mass, n_pmax, n_state;
  bool bf;
};

__device__ __forceinline__ float q_value(const MassParams& p, int64_t idx) {
  const uint32_t b16 = p.q[idx];
  if (p.bf) return __builtin_bit_cast(float, b16 << 16);
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b16);
}

__device__ __forceinline__ int pages_of(int32_t ctx) {
  return ctx > 0 ? (ctx + kPage - 1) / kPage : 0;
}

__global__ void __launch_bounds__(256) page_mass_kernel(const MassParams p) {
  const int64_t total = p.n_mass + p.n_pmax + p.n_state;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    if (idx < p.n_mass) {
      const int64_t bh = idx / p.max_pages;
      const int pg = (int)(idx % p.max_pages);
      const int b = (int)(bh / p.Hq), h = (int)(bh % p.Hq);
      const int g = h / p.G, hh = h % p.G;
      if (pg < pages_of(p.ctx_lens[b])) {
        const int64_t task = (int64_t)p.group_offsets[b * p.Hkv + g] + pg / p.pages_per_split;
        float v = 0.f;
        if (task < p.capacity) {
          const float e = p.ws_m[task * p.G + hh] - p.lse[bh] * 1.4426950408889634f;
          v = p.page_mass[idx] * __builtin_amdgcn_exp2f(e);
        }
        p.page_mass[idx] = v;
      } else {
        p.page_mass[idx] = 0.f;
      }
    } else if (idx < p.n_mass + p.n_pmax) {
      const int64_t k = idx - p.n_mass;
      const int pg = (int)(k % p.max_pages);
      const int64_t kbg = k / p.max_pages;
      const int b = (int)((kbg / p.Hkv) % p.B);
      if (pg >= pages_of(p.ctx_lens[b])) p.page_max[k] = -INFINITY;
    } else {
      const int64_t k = idx - p.n_mass - p.n_pmax;
      const int d = (int)(k % p.D);
      const int64_t kbg = k / p.D;
      const int g = (int)(kbg % p.Hkv);
      const int b = (int)((kbg / p.Hkv) % p.B);
      const int which = (int)(kbg / ((int64_t)p.Hkv * p.B));
      const int64_t q0 = ((int64_t)b * p.Hq + (int64_t)g * p.G) * p.D + d;
      float acc = q_value(p, q0);
      for (int h = 1; h < p.G; ++h) acc = __fadd_rn(acc, q_value(p, q0 + (int64_t)h * p.D));
      const float a = which ? p.alpha_slow : p.alpha_fast;
      p.s_next[k] = ema_step(p.s_prev[k], __fmul_rn(acc, p.inv_g), a);
    }
  }
}

hipError_t launch_merge(const kvpage_shape& s, const int32_t* group_offsets, int32_t capacity,
                        const void* workspace, void* out, float* lse, hipStream_t stream) {
  const int G = s.Hq / s.Hkv;
  const WorkspaceView ws = ws_view(const_cast<void*>(workspace), capacity, G, s.d);
  MergeParams p;
  p.group_offsets = group_offsets;
  p.ws_o = ws.o;
  p.ws_m = ws.m;
  p.ws_l = ws.l;
  p.out = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.Hq = s.Hq;
  p.Hkv = s.Hkv;
  p.G = G;
  p.capacity = capacity;
  const int grid = s.B * s.Hq;
  if (grid <= 0) return hipSuccess;
  const bool bf = s.dtype == KVPAGE_BF16;
  if (s.d == 128) {
    if (bf) hipLaunchKernelGGL((merge_kernel<128, true>), dim3(grid), dim3(kMergeThreads), 0, stream, p);
    else hipLaunchKernelGGL((merge_kernel<128, false>), dim3(grid), dim3(kMergeThreads), 0, stream, p);
  } else {
    if (bf) hipLaunchKernelGGL((merge_kernel<64, true>), dim3(grid), dim3(kMergeThreads), 0, stream, p);
    else hipLaunchKernelGGL((merge_kernel<64, false>), dim3(grid), dim3(kMergeThreads), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_page_mass(const kvpage_shape& s, const kvpage_budget& bud, const void* q,
                            const float* lse, const int32_t* ctx_lens,
                            const int32_t* group_offsets, int32_t capacity, const void* workspace,
                            hipStream_t stream) {
  const int G = s.Hq / s.Hkv;
  const WorkspaceView ws = ws_view(const_cast<void*>(workspace), capacity, G, s.d);
  MassParams p;
  p.page_mass = bud.page_mass;
  p.page_max = bud.page_max;
  p.s_prev = bud.s_prev;
  p.s_next = bud.s_next;
  p.alpha_fast = bud.alpha_fast;
  p.alpha_slow = bud.alpha_slow;
  p.q = static_cast<const uint16_t*>(q);
  p.lse = lse;
  p.ctx_lens = ctx_lens;
  p.group_offsets = group_offsets;
  p.ws_m = ws.m;
  p.B = s.B;
  p.Hq = s.Hq;
  p.Hkv = s.Hkv;
  p.G = G;
  p.D = s.d;
  p.max_pages = s.max_pages;
  p.pages_per_split = s.split_tokens / s.page_size;
  p.capacity = capacity;
  p.inv_g = 1.0f / (float)G;
  p.n_mass = (int64_t)s.B * s.Hq * s.max_pages;
  p.n_pmax = 2LL * s.B * s.Hkv * s.max_pages;
  p.n_state = 2LL * s.B * s.Hkv * s.d;
  p.bf = s.dtype == KVPAGE_BF16;
  const int64_t total = p.n_mass + p.n_pmax + p.n_state;
  if (total <= 0) return hipSuccess;
  int64_t grid = (total + 255) / 256;
  if (grid > 8192) grid = 8192;
  hipLaunchKernelGGL(page_mass_kernel, dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kvpage
