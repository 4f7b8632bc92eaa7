// Standalone check of the C ABI: plain host code, hipMalloc'd buffers, no
// Python and no torch.  One decode step (queue, split attention, merge and
// budgeting finish in kvpage_decode_step) on inputs whose results have a
// closed form: with q = 0 every score is 0, so attention is a plain mean over
// each sequence's tokens, lse = ln(ctx), the mass of a page is its share of
// the tokens, and with s_prev = 0 the summaries stay 0 and every valid page
// maximum is 0.  V holds (g + 1) / 4 for KV head g, so out = (g + 1) / 4.
// Exit status 0 and "c abi check ok" on success.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "kvpage.h"

#define CHECK(cond, ...)                                \
  do {                                                  \
    if (!(cond)) {                                      \
      std::fprintf(stderr, "c abi check failed: ");     \
      std::fprintf(stderr, __VA_ARGS__);                \
      std::fprintf(stderr, "\n");                       \
      std::exit(1);                                     \
    }                                                   \
  } while (0)

#define HIP_OK(call) CHECK((call) == hipSuccess, "%s", #call)

template <typename T>
static T* dev_copy(const std::vector<T>& h) {
  void* d = nullptr;
  HIP_OK(hipMalloc(&d, h.size() * sizeof(T) + 256));
  HIP_OK(hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice));
  return static_cast<T*>(d);
}

template <typename T>
static std::vector<T> host_copy(const T* d, size_t n) {
  std::vector<T> h(n);
  HIP_OK(hipMemcpy(h.data(), d, n * sizeof(T), hipMemcpyDeviceToHost));
  return h;
}

// f16 bits of the few exact values used here.
static uint16_t half_bits(float v) {
  if (v == 0.0f) return 0x0000;
  if (v == 0.25f) return 0x3400;
  if (v == 0.5f) return 0x3800;
  if (v == 1.0f) return 0x3c00;
  std::fprintf(stderr, "no f16 encoding for %f here\n", v);
  std::exit(1);
}

static float half_value(uint16_t b) {
  const int e = (b >> 10) & 31, m = b & 1023;
  const float s = (b & 0x8000) ? -1.0f : 1.0f;
  if (e == 0) return s * std::ldexp((float)m, -24);
  return s * std::ldexp(1.0f + m / 1024.0f, e - 15);
}

int main() {
  const int B = 3, Hq = 8, Hkv = 2, d = 128, P = 16, S = 64, G = Hq / Hkv;
  const std::vector<int32_t> ctx = {37, 300, 0};
  const int max_pages = 19, num_pages = 64;

  kvpage_shape shape = {B, Hq, Hkv, d, P, S, max_pages, num_pages, KVPAGE_F16, 1.0f / std::sqrt((float)d), 0};
  const int32_t cap = kvpage_queue_capacity(&shape);
  CHECK(cap == B * Hkv * ((max_pages * P + S - 1) / S), "capacity %d", cap);
  const int64_t ws_bytes = kvpage_workspace_bytes(&shape, cap);
  CHECK(ws_bytes > 0, "workspace bytes %lld", (long long)ws_bytes);

  // Pools: K = 1 everywhere, V = (g + 1) / 4 for KV head g.
  const size_t tile = (size_t)P * d;
  std::vector<uint16_t> k((size_t)num_pages * Hkv * tile, half_bits(1.0f));
  std::vector<uint16_t> v(k.size());
  for (int pg = 0; pg < num_pages; ++pg)
    for (int g = 0; g < Hkv; ++g)
      for (size_t i = 0; i < tile; ++i) v[((size_t)pg * Hkv + g) * tile + i] = half_bits(0.25f * (g + 1));
  // Sequence b owns pages 20b, 20b + 1, ... (table rows padded with page 0).
  std::vector<int32_t> bt((size_t)B * max_pages, 0);
  for (int b = 0; b < B; ++b)
    for (int j = 0; j < (ctx[b] + P - 1) / P; ++j) bt[(size_t)b * max_pages + j] = 20 * b + j;
  std::vector<uint16_t> q((size_t)B * Hq * d, half_bits(0.0f));
  std::vector<float> s_prev((size_t)2 * B * Hkv * d, 0.0f);

  uint16_t* d_q = dev_copy(q);
  uint16_t* d_k = dev_copy(k);
  uint16_t* d_v = dev_copy(v);
  int32_t* d_bt = dev_copy(bt);
  int32_t* d_ctx = dev_copy(ctx);
  float* d_sprev = dev_copy(s_prev);
  void *d_tasks, *d_offs, *d_n, *d_ws, *d_out, *d_lse, *d_mass, *d_snext, *d_pmax;
  HIP_OK(hipMalloc(&d_tasks, (size_t)cap * sizeof(kvpage_task)));
  HIP_OK(hipMalloc(&d_offs, (B * Hkv + 1) * sizeof(int32_t)));
  HIP_OK(hipMalloc(&d_n, sizeof(int32_t)));
  HIP_OK(hipMalloc(&d_ws, (size_t)ws_bytes));
  HIP_OK(hipMalloc(&d_out, (size_t)B * Hq * d * 2));
  HIP_OK(hipMalloc(&d_lse, (size_t)B * Hq * sizeof(float)));
  HIP_OK(hipMalloc(&d_mass, (size_t)B * Hq * max_pages * sizeof(float)));
  HIP_OK(hipMalloc(&d_snext, s_prev.size() * sizeof(float)));
  HIP_OK(hipMalloc(&d_pmax, (size_t)2 * B * Hkv * max_pages * sizeof(float)));

  kvpage_budget bud = {static_cast<float*>(d_mass), d_sprev, static_cast<float*>(d_snext),
                       0.5f, 0.05f, static_cast<float*>(d_pmax)};

  // An invalid call is refused before anything is enqueued.
  int rc = kvpage_decode_step(&shape, nullptr, d_k, d_v, d_bt, d_ctx, static_cast<kvpage_task*>(d_tasks),
                              static_cast<int32_t*>(d_offs), static_cast<int32_t*>(d_n), cap, d_ws, &bud,
                              d_out, static_cast<float*>(d_lse), nullptr, nullptr);
  CHECK(rc == KVPAGE_ERR_INVALID_ARG, "null q gave %d", rc);
  CHECK(kvpage_status_string(rc) != nullptr, "no status string");

  rc = kvpage_decode_step(&shape, d_q, d_k, d_v, d_bt, d_ctx, static_cast<kvpage_task*>(d_tasks),
                          static_cast<int32_t*>(d_offs), static_cast<int32_t*>(d_n), cap, d_ws, &bud, d_out,
                          static_cast<float*>(d_lse), nullptr, nullptr);
  CHECK(rc == KVPAGE_OK, "decode step: %s", kvpage_status_string(rc));
  HIP_OK(hipDeviceSynchronize());

  const int32_t n = host_copy(static_cast<int32_t*>(d_n), 1)[0];
  int want_n = 0;
  for (int b = 0; b < B; ++b) want_n += Hkv * ((ctx[b] + S - 1) / S);
  CHECK(n == want_n, "n_tasks %d, want %d", n, want_n);
  const auto tasks = host_copy(static_cast<kvpage_task*>(d_tasks), (size_t)n);
  int t = 0;
  for (int b = 0; b < B; ++b)
    for (int g = 0; g < Hkv; ++g)
      for (int j = 0; j * S < ctx[b]; ++j, ++t) {
        const kvpage_task& x = tasks[t];
        CHECK(x.seq == b && x.kv_head == g && x.tok_begin == j * S &&
                  x.tok_end == (ctx[b] < (j + 1) * S ? ctx[b] : (j + 1) * S),
              "task %d", t);
      }

  const auto out = host_copy(static_cast<uint16_t*>(d_out), (size_t)B * Hq * d);
  const auto lse = host_copy(static_cast<float*>(d_lse), (size_t)B * Hq);
  const auto mass = host_copy(static_cast<float*>(d_mass), (size_t)B * Hq * max_pages);
  const auto pmax = host_copy(static_cast<float*>(d_pmax), (size_t)2 * B * Hkv * max_pages);
  const auto snext = host_copy(static_cast<float*>(d_snext), s_prev.size());
  for (int b = 0; b < B; ++b) {
    const int npg = (ctx[b] + P - 1) / P;
    for (int h = 0; h < Hq; ++h) {
      const int g = h / G;
      const float want_out = ctx[b] > 0 ? 0.25f * (g + 1) : 0.0f;
      for (int i = 0; i < d; ++i) {
        const float o = half_value(out[((size_t)b * Hq + h) * d + i]);
        CHECK(std::fabs(o - want_out) <= 2e-3f + 1e-2f * want_out, "out[%d,%d,%d] = %f, want %f", b, h, i, o,
              want_out);
      }
      const float l = lse[(size_t)b * Hq + h];
      if (ctx[b] > 0)
        CHECK(std::fabs(l - std::log((float)ctx[b])) <= 1e-3f + 1e-4f * std::log((float)ctx[b]),
              "lse[%d,%d] = %f", b, h, l);
      else
        CHECK(std::isinf(l) && l < 0, "lse of an empty sequence is %f", l);
      for (int p = 0; p < max_pages; ++p) {
        const int valid = p < npg ? ((p + 1) * P <= ctx[b] ? P : ctx[b] - p * P) : 0;
        const float want = ctx[b] > 0 ? (float)valid / ctx[b] : 0.0f;
        const float got = mass[((size_t)b * Hq + h) * max_pages + p];
        CHECK(std::fabs(got - want) <= 1e-4f, "mass[%d,%d,%d] = %f, want %f", b, h, p, got, want);
      }
    }
    for (int w = 0; w < 2; ++w)
      for (int g = 0; g < Hkv; ++g)
        for (int p = 0; p < max_pages; ++p) {
          const float got = pmax[(((size_t)w * B + b) * Hkv + g) * max_pages + p];
          if (p < npg)
            CHECK(got == 0.0f, "page_max[%d,%d,%d,%d] = %f, want 0", w, b, g, p, got);
          else
            CHECK(std::isinf(got) && got < 0, "page_max past the end is %f", got);
        }
  }
  for (float x : snext) CHECK(x == 0.0f, "s_next %f, want 0", x);

  for (void* p : {(void*)d_q, (void*)d_k, (void*)d_v, (void*)d_bt, (void*)d_ctx, (void*)d_sprev, d_tasks,
                  d_offs, d_n, d_ws, d_out, d_lse, d_mass, d_snext, d_pmax})
    HIP_OK(hipFree(p));
  std::printf("c abi check ok: %d tasks, closed-form outputs match\n", n);
  return 0;
}
