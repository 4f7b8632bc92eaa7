// GrowPage's compress-or-acquire decision from the step's summary page maxima.
//
// GrowPage (mlsanity.com entry, Abstract; aitrending.vip article, Technical
// Details, on-demand page allocation) keeps a fast and a slow query summary,
// compares their attention working sets, and at each capacity boundary
// either compresses within the current allocation or acquires a physical
// page.  Read here as:
//   * working set of (summary, sequence, KV head): the softmax of the
//     summary's page scores (its page maxima) over the sequence's pages
//     weighs each page; the set is every page scoring at or above the
//     highest score level whose at-or-above pages hold >= tau of the weight
//     (the smallest top set covering tau, equal scores entering together);
//   * F and S: the unions over KV heads of the fast and slow sets (a physical
//     page carries every KV head of its tokens);
//   * a sequence whose last page is full (ctx > 0, ctx % 16 == 0) acquires
//     when |F| > |S| (recent demand broader than long-term demand) or no page
//     lies outside F and S; otherwise it compresses, and the victim is the
//     page outside both whose largest slow score over the KV heads is lowest
//     (ties: the lowest page).
//
// ws_select_kernel finds each working set's closing level by a radix select
// over order-preserving score keys with 40-bit fixed-point weights, so every
// sum is an exact integer whatever order threads add it in; decide_kernel
// tests every page against the levels and takes the decision.
#include <math.h>

#include "kvpage_common.h"

namespace kvpage {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / kWave;
constexpr int kDigitBits = 11;              // radix digit of the working-set select
constexpr int kBins = 1 << kDigitBits;
constexpr int kMaxDecidePages = 1 << 23;   // 2^23 pages x 2^40 per weight fits 64 bits
constexpr int kStagePages = 8192;           // keys and weights of one set held in LDS (96 KiB)
constexpr int kStagePagesSmall = 2048;      // the same for rows up to 2048 pages (24 KiB)
constexpr int kDecideThreads = 1024;        // decide_kernel: one workgroup per sequence

struct DecideParams {
  const float* page_max;    // [2, B, Hkv, max_pages]
  const int32_t* ctx_lens;  // [B]
  int32_t* ws_size;         // [2, B, Hkv]
  float* ws_level;          // [2, B, Hkv]
  int32_t* ws_union;        // [2, B]
  int32_t* decision;        // [B]
  int32_t* victim;          // [B]
  int32_t B, Hkv, max_pages;
  float tau;
};

// Order-preserving 32-bit key of a score (-0 taken as +0, so equal scores
// have equal keys), and back.
__device__ __forceinline__ uint32_t score_key(float x) {
  const uint32_t u = __float_as_uint(x == 0.0f ? 0.0f : x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Softmax weight relative to the largest score M, in units of 2^-40: at most
// 2^40 (the top page weighs exactly that), truncated.  All -inf: all weigh 1.
__device__ __forceinline__ uint64_t fixed_weight(float x, float M) {
  const float w = x == M ? 1.0f : __builtin_amdgcn_exp2f((x - M) * 1.4426950408889634f);
  return (uint64_t)(w * 1099511627776.0f);
}

__device__ __forceinline__ int pages_in(int32_t ctx) { return (ctx + kPage - 1) / kPage; }

// Inclusive prefix scans over a wavefront with DPP moves (gfx9 wave64): row
// shifts by 1, 2, 4 and 8 scan each row of 16 lanes, then lane 15 of rows 0
// and 2 goes to rows 1 and 3, and lane 31 to rows 2 and 3.  Lane i gets the
// combination of lanes 0..i, lane 63 that of the whole wavefront.  Lanes a
// move does not reach read 0, the identity of unsigned add and max.  Each
// step is a register move between lanes, where a shuffle is an LDS
// crossbar round trip.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_move(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, true);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp_move(uint64_t v) {
  return ((uint64_t)dpp_move<CTRL, ROWS>((uint32_t)(v >> 32)) << 32) |
         dpp_move<CTRL, ROWS>((uint32_t)v);
}
template <typename T, typename Op>
__device__ __forceinline__ T wave_scan(T x, Op op) {
  x = op(x, dpp_move<0x111, 0xF>(x));   // row_shr:1
  x = op(x, dpp_move<0x112, 0xF>(x));   // row_shr:2
  x = op(x, dpp_move<0x114, 0xF>(x));   // row_shr:4
  x = op(x, dpp_move<0x118, 0xF>(x));   // row_shr:8
  x = op(x, dpp_move<0x142, 0xA>(x));   // row_bcast:15 into rows 1 and 3
  x = op(x, dpp_move<0x143, 0xC>(x));   // row_bcast:31 into rows 2 and 3
  return x;
}
struct AddOp {
  template <typename T>
  __device__ T operator()(T a, T b) const { return a + b; }
};
struct MaxOp {
  template <typename T>
  __device__ T operator()(T a, T b) const { return a > b ? a : b; }
};
constexpr int kLastLane = kWave - 1;

// Workgroup sum (every thread gets it); `red` holds one slot per wavefront
// and is reused, so the call ends with a barrier.
__device__ __forceinline__ uint64_t block_sum_u64(uint64_t v, uint64_t* red) {
  v = wave_scan(v, AddOp{});
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == kLastLane) red[threadIdx.x / kWave] = v;
  __syncthreads();
  uint64_t r = 0;
  for (int i = 0; i < kDecWaves; ++i) r += red[i];
  return r;
}
// One workgroup per (summary k, sequence b, KV head g), blockIdx.x =
// (k * B + b) * Hkv + g, the row of page_max it reads.
//
// Each page's key and fixed-point weight are computed once and kept in LDS
// when every row fits (instances for rows up to 2048 and 8192 pages); the
// instance for longer rows recomputes them from global memory in every pass.  The radix digits are 11 bits of the key relative to the
// smallest key, top bit of the range first (at most three passes): scores of
// one set usually share their sign and exponent, so digits of the raw key's
// top bits would put every page in a few bins, and the LDS atomics of one
// bin run one lane at a time.
template <int STAGE>
__global__ void __launch_bounds__(kDecThreads) ws_select_kernel(const DecideParams p) {
  __shared__ uint32_t skey[STAGE > 0 ? STAGE : 1];
  __shared__ uint64_t swt[STAGE > 0 ? STAGE : 1];
  __shared__ uint64_t hm[kBins];   // weight per digit bin
  __shared__ uint64_t redu[kDecWaves];
  __shared__ uint64_t wsum[kDecWaves];   // wavefront totals of the bin search
  __shared__ uint32_t pick_bin;
  __shared__ uint64_t pick_above;
  const int item = blockIdx.x;
  const int b = (item / p.Hkv) % p.B;
  const int tid = threadIdx.x;
  const int npg = pages_in(clamp_ctx(p.ctx_lens[b], p.max_pages));
  if (npg == 0) {
    if (tid == 0) {
      p.ws_size[item] = 0;
      p.ws_level[item] = INFINITY;
    }
    return;
  }
  const float* xg = p.page_max + (int64_t)item * p.max_pages;
  constexpr bool staged = STAGE > 0;   // the launch picks STAGE >= max_pages

  // Keys, and the smallest and largest of them.
  uint32_t tmax = 0, tmin = 0xffffffffu;
#pragma unroll 8
  for (int i = tid; i < npg; i += kDecThreads) {
    const uint32_t key = score_key(xg[i]);
    if (staged) skey[i] = key;
    tmax = max(tmax, key);
    tmin = min(tmin, key);
  }
  // Largest key, and the smallest as the largest complement.
  tmax = wave_scan(tmax, MaxOp{});
  tmin = ~wave_scan(~tmin, MaxOp{});
  if ((tid & (kWave - 1)) == kLastLane) redu[tid / kWave] = ((uint64_t)tmax << 32) | tmin;
  __syncthreads();   // also: keys staged
  uint32_t kmax = 0, kmin = 0xffffffffu;
  for (int i = 0; i < kDecWaves; ++i) {
    kmax = max(kmax, (uint32_t)(redu[i] >> 32));
    kmin = min(kmin, (uint32_t)redu[i]);
  }
  __syncthreads();   // redu is reused below
  const float M = key_score(kmax);
  auto key_of = [&](int i) { return staged ? skey[i] : score_key(xg[i]); };
  auto wt_of = [&](int i) { return staged ? swt[i] : fixed_weight(key_score(score_key(xg[i])), M); };

  uint32_t level_key = kmin;   // every page ties when the range is one key
  if (kmax != kmin) {
    const int L = 32 - __clz(kmax - kmin);   // bits of the relative keys
    // Digits of kDigitBits bits aligned to bit 0; the first holds the top bits.
    int shift = L > kDigitBits ? (L - 1) / kDigitBits * kDigitBits : 0;
    for (int i = tid; i < kBins; i += kDecThreads) hm[i] = 0;
    __syncthreads();
    // Weights, their total and the first digit's histogram.
    uint64_t z = 0;
#pragma unroll 8
    for (int i = tid; i < npg; i += kDecThreads) {
      const uint32_t key = key_of(i);
      const uint64_t u = fixed_weight(key_score(key), M);
      if (staged) swt[i] = u;
      z += u;
      atomicAdd(reinterpret_cast<unsigned long long*>(&hm[(key - kmin) >> shift]),
                (unsigned long long)u);
    }
    const uint64_t Z = block_sum_u64(z, redu);   // ends with a barrier: histogram complete
    // Target mass: the smallest integer >= tau * Z, within [1, Z].
    uint64_t T = (uint64_t)ceil((double)p.tau * (double)Z);
    T = T < 1 ? 1 : (T > Z ? Z : T);

    // Radix select, highest digit first: keep the bin where the mass of the
    // pages above it plus its own first reaches T.  Invariant: `above` (mass
    // of the pages whose relative key lies above the current prefix range)
    // < T <= above + mass of the range.
    uint32_t prefix = 0;
    uint64_t above = 0;
    for (bool first = true;; first = false) {
      if (!first) {
        for (int i = tid; i < kBins; i += kDecThreads) hm[i] = 0;
        __syncthreads();
        const int hi = shift + kDigitBits;
#pragma unroll 8
        for (int i = tid; i < npg; i += kDecThreads) {
          const uint32_t rel = key_of(i) - kmin;
          if ((rel >> hi) == (prefix >> hi)) {
            const uint32_t d = (rel >> shift) & (kBins - 1);
            atomicAdd(reinterpret_cast<unsigned long long*>(&hm[d]),
                      (unsigned long long)wt_of(i));
          }
        }
        __syncthreads();
      }
      {
        // Thread t holds the kPer bins from kBins - kPer*(t+1) up, so the
        // threads before it hold every bin above its own: their mass is a
        // prefix sum, inside each wavefront by DPP moves, then over the
        // totals of the wavefronts before.  The one thread whose bins cross
        // T scans them, highest first.
        constexpr int kPer = kBins / kDecThreads;
        const int bin0 = kBins - kPer * (tid + 1);
        uint64_t bins[kPer];
        uint64_t sm = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          bins[j] = hm[bin0 + j];
          sm += bins[j];
        }
        const int lane = tid & (kWave - 1), w = tid / kWave;
        const uint64_t im = wave_scan(sm, AddOp{});   // this thread's and those before it
        if (lane == kLastLane) wsum[w] = im;
        __syncthreads();
        uint64_t run = above + (im - sm);
        for (int v = 0; v < w; ++v) run += wsum[v];
        if (run < T && run + sm >= T) {   // exactly one thread holds the bin
#pragma unroll
          for (int j = kPer - 1; j >= 0; --j) {
            if (run < T && run + bins[j] >= T) {
              pick_bin = bin0 + j;
              pick_above = run;
            }
            run += bins[j];
          }
        }
      }
      __syncthreads();
      const uint32_t d = pick_bin & (kBins - 1);   // one lane always picks
      prefix |= d << shift;
      above = pick_above;
      if (shift == 0) break;
      __syncthreads();   // every thread has read the pick before the next pass
      shift -= kDigitBits;
    }
    level_key = kmin + prefix;
  }
  // Size: the pages at or above the closing level.
  uint32_t cnt = 0;
#pragma unroll 8
  for (int i = tid; i < npg; i += kDecThreads) cnt += key_of(i) >= level_key;
  cnt = wave_scan(cnt, AddOp{});
  if ((tid & (kWave - 1)) == kLastLane) wsum[tid / kWave] = cnt;
  __syncthreads();
  uint32_t size = 0;
  for (int i = 0; i < kDecWaves; ++i) size += (uint32_t)wsum[i];
  if (tid == 0) {
    p.ws_size[item] = (int32_t)size;
    p.ws_level[item] = key_score(level_key);
  }
}

// One workgroup per sequence: membership of every page in F and S, their
// sizes, the lowest (slow score, page) outside both, and the decision.
// Dynamic LDS: the 2 * Hkv closing levels.  A thread takes pages tid, tid +
// 1024, ...; the 2 * Hkv scores of a page are requested together, eight
// KV heads at a time, so a page costs one memory round trip per eight heads.
__global__ void __launch_bounds__(kDecideThreads) decide_kernel(const DecideParams p) {
  constexpr int NW = kDecideThreads / kWave;
  extern __shared__ float levels[];   // [2][Hkv]
  __shared__ uint64_t red[NW];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t ctx = clamp_ctx(p.ctx_lens[b], p.max_pages);
  const int npg = pages_in(ctx);
  for (int i = tid; i < 2 * p.Hkv; i += kDecideThreads) {
    const int k = i / p.Hkv, g = i % p.Hkv;
    levels[i] = p.ws_level[((int64_t)k * p.B + b) * p.Hkv + g];
  }
  __syncthreads();
  const float* fast = p.page_max + (int64_t)b * p.Hkv * p.max_pages;
  const float* slow = p.page_max + ((int64_t)p.B + b) * p.Hkv * p.max_pages;
  uint32_t nf = 0, ns = 0;
  uint64_t best = ~0ull;
  for (int pg = tid; pg < npg; pg += kDecideThreads) {
    bool in_f = false, in_s = false;
    float sig = -INFINITY;
    for (int g0 = 0; g0 < p.Hkv; g0 += 8) {
      float xf[8], xs[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {   // heads past Hkv re-read the last one
        const int g = min(g0 + j, p.Hkv - 1);
        xf[j] = fast[(int64_t)g * p.max_pages + pg];
        xs[j] = slow[(int64_t)g * p.max_pages + pg];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int g = min(g0 + j, p.Hkv - 1);
        in_f = in_f || xf[j] >= levels[g];
        in_s = in_s || xs[j] >= levels[p.Hkv + g];
        sig = fmaxf(sig, xs[j]);
      }
    }
    nf += in_f;
    ns += in_s;
    if (!in_f && !in_s) {
      const uint64_t cand = ((uint64_t)score_key(sig) << 32) | (uint32_t)pg;
      best = cand < best ? cand : best;
    }
  }
  // Workgroup sums of the two counts (packed) and minimum candidate.
  // (Lane 63 holds each wavefront's; the minimum as the largest complement.)
  uint64_t counts = wave_scan(((uint64_t)nf << 32) | ns, AddOp{});
  best = ~wave_scan(~best, MaxOp{});
  if ((tid & (kWave - 1)) == kLastLane) red[tid / kWave] = counts;
  __syncthreads();
  if (tid == 0) {
    counts = 0;
    for (int i = 0; i < NW; ++i) counts += red[i];
  }
  __syncthreads();
  if ((tid & (kWave - 1)) == kLastLane) red[tid / kWave] = best;
  __syncthreads();
  if (tid == 0) {
    for (int i = 0; i < NW; ++i) best = red[i] < best ? red[i] : best;
    const uint32_t F = (uint32_t)(counts >> 32), S = (uint32_t)counts;
    p.ws_union[b] = (int32_t)F;
    p.ws_union[p.B + b] = (int32_t)S;
    int32_t dec = KVPAGE_DECIDE_NONE, vic = -1;
    if (ctx > 0 && ctx % kPage == 0) {
      if (F > S || best == ~0ull) {
        dec = KVPAGE_DECIDE_ACQUIRE;
      } else {
        dec = KVPAGE_DECIDE_COMPRESS;
        vic = (int32_t)(best & 0xffffffffu);
      }
    }
    p.decision[b] = dec;
    p.victim[b] = vic;
  }
}

int decide_max_pages() { return kMaxDecidePages; }

hipError_t launch_budget_decide(const kvpage_shape& s, const float* page_max,
                                const int32_t* ctx_lens, float tau, int32_t* ws_size,
                                float* ws_level, int32_t* ws_union, int32_t* decision,
                                int32_t* victim, hipStream_t stream) {
  DecideParams p;
  p.page_max = page_max;
  p.ctx_lens = ctx_lens;
  p.ws_size = ws_size;
  p.ws_level = ws_level;
  p.ws_union = ws_union;
  p.decision = decision;
  p.victim = victim;
  p.B = s.B;
  p.Hkv = s.Hkv;
  p.max_pages = s.max_pages;
  p.tau = tau;
  // The smallest LDS stage that holds a row: less LDS, more resident workgroups.
  const dim3 grid(2 * s.B * s.Hkv), block(kDecThreads);
  if (s.max_pages <= kStagePagesSmall)
    hipLaunchKernelGGL(ws_select_kernel<kStagePagesSmall>, grid, block, 0, stream, p);
  else if (s.max_pages <= kStagePages)
    hipLaunchKernelGGL(ws_select_kernel<kStagePages>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(ws_select_kernel<0>, grid, block, 0, stream, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(decide_kernel, dim3(s.B), dim3(kDecideThreads), 2 * s.Hkv * sizeof(float),
                     stream, p);
  return hipGetLastError();
}

}  // namespace kvpage
