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
//   * online softmax keeps, per head, a reference max m in the log2 domain,
//     moved only when a page's max exceeds it by more than 8 (weights stay
//     below 2^8 in between);
//   * P V comes from 16x16x16 MFMAs whose P operand is the score tile's own
//     register layout, so no lane shuffles are needed between the two
//     contractions;
//   * K/V pages are prefetched DEPTH pages ahead into registers.
//
// Outputs per task go to the workspace: m (log2 domain), l = sum exp2(y - m)
// and the unnormalised o = sum exp2(y - m) v for each query head of the group.
#include <float.h>
#include <math.h>

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
  const uint16_t* q;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* block_tables;
  const kvpage_task* tasks;
  const int32_t* n_tasks;
  float* ws_o;
  float* ws_m;
  float* ws_l;
  float* page_mass;
  const float* s_prev;
  float* page_max;
  float alpha_fast, alpha_slow;
  int32_t B, Hq, Hkv, G, max_pages, capacity;
  float scale, c2, inv_g;
};

constexpr int kWavesPerGroup = 4;
constexpr int kMaxPagesPerTask = 16;
constexpr float kRescaleLog2 = 8.0f;

__device__ __forceinline__ float row_allreduce_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, kWave));
  return fmaxf(v, __shfl_xor(v, 32, kWave));
}

__device__ __forceinline__ float row_allreduce_sum(float v) {
  v += __shfl_xor(v, 16, kWave);
  return v + __shfl_xor(v, 32, kWave);
}

// Two 16-bit halves (lo from a, hi from b), picking half `hi_half` of each word.
__device__ __forceinline__ uint32_t pick_pair(uint32_t a, uint32_t b, bool hi_half) {
  return hi_half ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
}

template <int D, bool BF, bool BUDGET, int DEPTH>
__global__ void __launch_bounds__(kWave * kWavesPerGroup)
    split_attn_kernel(const AttnParams p) {
  using E = Elem<BF>;
  constexpr int KB = D / 32;   // 16x16x32 MFMAs per page for Q K^T
  constexpr int VD = D / 16;   // output column blocks; V halves per lane per token
  constexpr int VW = VD / 2;   // V dwords per lane per token
  constexpr int NPC = E::kPieces;

  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane >> 4;       // row of 16 lanes
  const int n = lane & 15;       // column inside the row
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int first = blockIdx.x * kWavesPerGroup + wave;
  const int stride = gridDim.x * kWavesPerGroup;
  const int ntask = min(p.n_tasks[0], p.capacity);
  const int G = p.G;
  const bool is_head = n < G;
  const bool is_sum = BUDGET && n >= G && n < G + 2 * NPC;
  const bool is_lead = BUDGET && (n == G || n == G + NPC);

  // Byte offsets of this lane's pieces inside one (page, head) tile.
  uint32_t koff[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) koff[kb] = (uint32_t)(n * D + 8 * (4 * kb + r)) * 2u;
  uint32_t voff[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) voff[e] = (uint32_t)((4 * r + e) * D + n * VD) * 2u;

  const char* kpool = reinterpret_cast<const char*>(p.k_pool);
  const char* vpool = reinterpret_cast<const char*>(p.v_pool);

  for (int t = first; t < ntask; t += stride) {
    const kvpage_task tk = p.tasks[t];
    const int b = tk.seq, g = tk.kv_head;
    const int ntok = tk.tok_end - tk.tok_begin;
    const int npg = (ntok + kPage - 1) / kPage;
    const int lp0 = tk.tok_begin / kPage;
    const int32_t* bt_row = p.block_tables + (int64_t)b * p.max_pages + lp0;
    const int32_t page_ids = lane < npg ? bt_row[lane] : 0;

    u32x4 kbuf[DEPTH][KB];
    uint32_t vbuf[DEPTH][4][VW];

    auto load_k = [&](int i, int slot) {
      const int32_t pid = __builtin_amdgcn_readlane(page_ids, i);
      const char* base = kpool + tile_offset(pid, g, p.Hkv, D) * 2;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        kbuf[slot][kb] = *reinterpret_cast<const u32x4*>(base + koff[kb]);
    };
    auto load_v = [&](int i, int slot) {
      const int32_t pid = __builtin_amdgcn_readlane(page_ids, i);
      const char* base = vpool + tile_offset(pid, g, p.Hkv, D) * 2;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (VW == 4) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(base + voff[e]);
#pragma unroll
          for (int x = 0; x < 4; ++x) vbuf[slot][e][x] = w[x];
        } else {
          const u32x2 w = *reinterpret_cast<const u32x2*>(base + voff[e]);
#pragma unroll
          for (int x = 0; x < VW; ++x) vbuf[slot][e][x] = w[x];
        }
      }
    };

#pragma unroll
    for (int i = 0; i < DEPTH; ++i) {
      if (i < npg) {
        load_k(i, i);
        load_v(i, i);
      }
    }

    // Column operand: query heads, then summary pieces, then zeros.
    u32x4 qop[KB];
    const uint16_t* qrow0 = p.q + ((int64_t)b * p.Hq + (int64_t)g * G) * D;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int d0 = 8 * (4 * kb + r);
      u32x4 v = {0u, 0u, 0u, 0u};
      if (is_head) {
        v = *reinterpret_cast<const u32x4*>(qrow0 + (int64_t)n * D + d0);
      } else if (is_sum) {
        const int which = (n - G) / NPC;
        const int piece = (n - G) % NPC;
        const float a = which ? p.alpha_slow : p.alpha_fast;
        float acc[8];
#pragma unroll
        for (int h = 0; h < 8; ++h) {
          if (h < G) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(qrow0 + (int64_t)h * D + d0);
#pragma unroll
            for (int x = 0; x < 8; ++x) {
              const float qv = E::value((w[x >> 1] >> (16 * (x & 1))) & 0xffffu);
              acc[x] = h == 0 ? qv : __fadd_rn(acc[x], qv);
            }
          }
        }
        const float* sp = p.s_prev + (((int64_t)which * p.B + b) * p.Hkv + g) * D + d0;
        uint32_t hv[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const float s = ema_step(sp[x], __fmul_rn(acc[x], p.inv_g), a);
          float rem = s;
          uint32_t pc = E::bits(rem);
          for (int k = 0; k < piece; ++k) {
            rem = __fsub_rn(rem, E::value(pc));
            pc = E::bits(rem);
          }
          hv[x] = pc;
        }
#pragma unroll
        for (int x = 0; x < 4; ++x) v[x] = hv[2 * x] | (hv[2 * x + 1] << 16);
      }
      qop[kb] = v;
    }

    f32x4 O[VD];
#pragma unroll
    for (int j = 0; j < VD; ++j) O[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float mref = is_head ? -INFINITY : INFINITY;  // non-head lanes get zero weights
    float l = 0.f;
    float keep[4] = {0.f, 0.f, 0.f, 0.f};         // per-page outputs, page 4*r + u

#pragma unroll
    for (int i = 0; i < kMaxPagesPerTask; ++i) {
      if (i < npg) {
        const int slot = i % DEPTH;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) acc = E::mfma_qk(kbuf[slot][kb], qop[kb], acc);
        if (i + DEPTH < npg) load_k(i + DEPTH, slot);

        // acc[e] = dot(column n, key of token 4r+e).  Summary pieces sit in
        // adjacent columns: add them into the lead column.
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float c = acc[e];
          if constexpr (BUDGET) {
            float sum = __fadd_rn(acc[e], __shfl_down(acc[e], 1, 16));
            if constexpr (NPC == 3) sum = __fadd_rn(sum, __shfl_down(acc[e], 2, 16));
            c = is_head ? acc[e] : sum;
          }
          x[e] = c;
        }
        const int nvalid = ntok - kPage * i;
        if (nvalid < kPage) {  // last page is partial: drop slots past the context
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (4 * r + e >= nvalid) {
              x[e] = -INFINITY;
#pragma unroll
              for (int w = 0; w < VW; ++w) vbuf[slot][e][w] = 0u;
            }
          }
        }
        const float pm = row_allreduce_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
        const float ymax = pm * p.c2;
        const bool need = is_head && (ymax > mref + kRescaleLog2);
        if (__builtin_amdgcn_ballot_w64(need)) {
          const float mnew = need ? ymax : mref;
          const float alpha = need ? (mref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mref - mnew)) : 1.f;
          mref = mnew;
          l *= alpha;
          if constexpr (BUDGET) {
#pragma unroll
            for (int u = 0; u < 4; ++u) keep[u] *= alpha;
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float ae = __shfl(alpha, 4 * r + e, kWave);
#pragma unroll
            for (int j = 0; j < VD; ++j) O[j][e] *= ae;
          }
        }
        float pe[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pe[e] = __builtin_amdgcn_exp2f(fmaf(x[e], p.c2, -mref));
        const float psum = (pe[0] + pe[1]) + (pe[2] + pe[3]);
        l += psum;
        if constexpr (BUDGET) {
          const float page_sum = row_allreduce_sum(psum);
          if (r == (i >> 2)) keep[i & 3] = is_head ? page_sum : pm * p.scale;
        }
        u32x2 pop;
        pop[0] = E::bits(pe[0]) | (E::bits(pe[1]) << 16);
        pop[1] = E::bits(pe[2]) | (E::bits(pe[3]) << 16);
#pragma unroll
        for (int j = 0; j < VD; ++j) {
          const bool hi = j & 1;
          const int w = j >> 1;
          u32x2 vop;
          vop[0] = pick_pair(vbuf[slot][0][w], vbuf[slot][1][w], hi);
          vop[1] = pick_pair(vbuf[slot][2][w], vbuf[slot][3][w], hi);
          O[j] = E::mfma_pv(pop, vop, O[j]);
        }
        if (i + DEPTH < npg) load_v(i + DEPTH, slot);
      }
    }

    // Task epilogue: partial (m, l, o) per head; per-page budgeting values.
    const float ltot = row_allreduce_sum(l);
    if (r == 0 && is_head) {
      p.ws_m[(int64_t)t * G + n] = mref;
      p.ws_l[(int64_t)t * G + n] = ltot;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int h = 4 * r + e;
      if (h < G) {
        float* dst = p.ws_o + ((int64_t)t * G + h) * D + n * VD;
#pragma unroll
        for (int j = 0; j < VD; ++j) dst[j] = O[j][e];
      }
    }
    if constexpr (BUDGET) {
      float* dst = nullptr;
      if (is_head) {
        dst = p.page_mass + ((int64_t)b * p.Hq + (int64_t)g * G + n) * p.max_pages + lp0;
      } else if (is_lead) {
        const int which = n == G ? 0 : 1;
        dst = p.page_max + (((int64_t)which * p.B + b) * p.Hkv + g) * p.max_pages + lp0;
      }
      if (dst) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (4 * r + u < npg) dst[4 * r + u] = keep[u];
      }
    }
  }
}

template <int D, bool BF, bool BUDGET, int DEPTH>
static hipError_t launch_one(const AttnParams& p, int capacity, hipStream_t stream) {
  auto kern = split_attn_kernel<D, BF, BUDGET, DEPTH>;
  static int blocks_per_cu[64] = {0};
  static int num_cus[64] = {0};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  const int slot = dev & 63;
  if (blocks_per_cu[slot] == 0) {
    int cus = 0;
    err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    int per = 0;
    err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kern, kWave * kWavesPerGroup, 0);
    if (err != hipSuccess) return err;
    num_cus[slot] = cus;
    blocks_per_cu[slot] = per > 0 ? per : 1;
  }
  const int64_t want = ((int64_t)capacity + kWavesPerGroup - 1) / kWavesPerGroup;
  const int64_t resident = (int64_t)blocks_per_cu[slot] * num_cus[slot];
  const int grid = (int)(want < resident ? want : resident);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kWave * kWavesPerGroup), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_split_attn(const kvpage_shape& s, const void* q, const void* k_pool,
                             const void* v_pool, const int32_t* block_tables,
                             const kvpage_task* tasks, const int32_t* n_tasks, int32_t capacity,
                             void* workspace, const kvpage_budget* budget, hipStream_t stream) {
  const int G = s.Hq / s.Hkv;
  const WorkspaceView ws = ws_view(workspace, capacity, G, s.d);
  AttnParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k_pool = static_cast<const uint16_t*>(k_pool);
  p.v_pool = static_cast<const uint16_t*>(v_pool);
  p.block_tables = block_tables;
  p.tasks = tasks;
  p.n_tasks = n_tasks;
  p.ws_o = ws.o;
  p.ws_m = ws.m;
  p.ws_l = ws.l;
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
  p.capacity = capacity;
  p.scale = s.scale;
  p.c2 = s.scale * 1.4426950408889634f;
  p.inv_g = 1.0f / (float)G;
  const bool bf = s.dtype == KVPAGE_BF16;
  const bool bud = budget != nullptr;
  constexpr int DP = 4;
  if (s.d == 128) {
    if (bf) return bud ? launch_one<128, true, true, DP>(p, capacity, stream)
                       : launch_one<128, true, false, DP>(p, capacity, stream);
    return bud ? launch_one<128, false, true, DP>(p, capacity, stream)
               : launch_one<128, false, false, DP>(p, capacity, stream);
  }
  if (bf) return bud ? launch_one<64, true, true, DP>(p, capacity, stream)
                     : launch_one<64, true, false, DP>(p, capacity, stream);
  return bud ? launch_one<64, false, true, DP>(p, capacity, stream)
             : launch_one<64, false, false, DP>(p, capacity, stream);
}

}  // namespace kvpage
