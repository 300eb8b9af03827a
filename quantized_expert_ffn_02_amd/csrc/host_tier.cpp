// Host miss tier: the SwiGLU FFN of the selected experts that a GPU expert cache
// does not hold, computed on the CPU from a host copy of every expert (pages and
// format: host_tier.h).  Plain C++ (built once, no instruction-set flags); the row
// dots come from host_ffn.cpp's AVX-512 or AVX2 build, chosen at run time.
//
// Work of one call, entries r = t*k + i of the miss list:
//   1. group the entries by expert (ascending expert id, entries ascending within);
//   2. reorder each token's activations for the row dot (act_pos order);
//   3. gate/up: per (expert, 8 rows of I), a = Wg x and b = Wu x for every token of
//      the group, h = SiLU(a) * b;
//   4. down: per (expert, 32 rows of H), z_r = Wd h_r for every entry of the group;
//   5. y[t] = sum over t's entries in ascending r of gate[r] * z_r (zero if none).
// Each output is computed by one thread in a fixed order, so the result does not
// depend on the thread count.
#include <stdint.h>
#include <string.h>

#include <immintrin.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <condition_variable>
#include <functional>
#include <memory>
#include <mutex>
#include <thread>
#include <vector>

#include "host_tier.h"
#include "moe.h"

namespace moe_host {
namespace {

enum Isa { kNone = 0, kAvx2 = 1, kAvx512 = 2 };

int detect_isa() {
  __builtin_cpu_init();
  const bool avx2 = __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma");
  const bool avx512 = avx2 && __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
                      __builtin_cpu_supports("avx512vl") && __builtin_cpu_supports("avx512dq");
  return avx512 ? kAvx512 : avx2 ? kAvx2 : kNone;
}

int isa() {
  static const int v = detect_isa();
  return v;
}

struct Kernels {
  void (*prep)(const uint16_t*, int, float*);
  void (*dot)(const HostMat&, int, int, const float* const*, int, float*, int);
};

Kernels kernels() {
  if (isa() == kAvx512) return {avx512::prep_act_bf16, avx512::rows_dot};
  return {avx2::prep_act_bf16, avx2::rows_dot};
}

// Persistent workers; run(units, fn) calls fn(u) for every u < units across the
// workers and the calling thread (dynamic assignment) and returns when all are done.
// Idle workers poll for new work for up to kSpinMicros before they sleep, so the
// barriers between the phases of a call, and calls that follow each other closely
// (one per layer), do not pay a sleeping thread's wake-up.
class Pool {
 public:
  static constexpr int kSpinMicros = 50;
  explicit Pool(int n) : n_(n) {
    for (int i = 1; i < n; ++i) th_.emplace_back([this] { worker(); });
  }
  ~Pool() {
    {
      std::lock_guard<std::mutex> g(mu_);
      stop_.store(true);
    }
    cv_.notify_all();
    for (auto& t : th_) t.join();
  }
  int size() const { return n_; }
  void run(int units, const std::function<void(int)>& fn) {
    if (units <= 0) return;
    if (th_.empty() || units == 1) {
      for (int u = 0; u < units; ++u) fn(u);
      return;
    }
    fn_ = &fn;
    units_ = units;
    next_.store(0, std::memory_order_relaxed);
    busy_.store((int)th_.size(), std::memory_order_relaxed);
    {
      std::lock_guard<std::mutex> g(mu_);   // a worker checks gen_ under the lock before it sleeps
      gen_.fetch_add(1, std::memory_order_release);
    }
    cv_.notify_all();
    drain();
    while (busy_.load(std::memory_order_acquire) != 0) _mm_pause();
    fn_ = nullptr;
  }

 private:
  void drain() {
    for (;;) {
      const int u = next_.fetch_add(1, std::memory_order_relaxed);
      if (u >= units_) return;
      (*fn_)(u);
    }
  }
  // Returns false when the pool is being destroyed.
  bool wait_for_work(uint64_t seen) {
    const auto until = std::chrono::steady_clock::now() + std::chrono::microseconds(kSpinMicros);
    for (int i = 0;; ++i) {
      if (gen_.load(std::memory_order_acquire) != seen) return true;
      if (stop_.load(std::memory_order_relaxed)) return false;
      _mm_pause();
      if ((i & 63) == 63 && std::chrono::steady_clock::now() > until) break;
    }
    std::unique_lock<std::mutex> lk(mu_);
    cv_.wait(lk, [&] { return stop_.load() || gen_.load(std::memory_order_acquire) != seen; });
    return !stop_.load();
  }
  void worker() {
    uint64_t seen = 0;
    for (;;) {
      if (!wait_for_work(seen)) return;
      seen = gen_.load(std::memory_order_acquire);
      drain();
      busy_.fetch_sub(1, std::memory_order_release);
    }
  }
  const int n_;
  std::vector<std::thread> th_;
  std::mutex mu_;
  std::condition_variable cv_;
  const std::function<void(int)>* fn_ = nullptr;
  int units_ = 0;
  std::atomic<uint64_t> gen_{0};
  std::atomic<int> busy_{0};
  std::atomic<int> next_{0};
  std::atomic<bool> stop_{false};
};

// One call at a time: the pool and the scratch buffers are shared.
std::mutex g_call;
std::unique_ptr<Pool> g_pool;
std::vector<float> g_xp, g_hp, g_z;

// Three quarters of the hardware threads, at most 12: the HIP runtime's own threads
// and the caller's GPU work need cores too (with 16 threads on a 16-thread share the
// tiered layer ran no faster than with 12).
int default_threads() {
  const unsigned hw = std::thread::hardware_concurrency();
  return (int)std::max(1u, std::min(16u, hw ? hw : 1u) * 3 / 4);
}

HostMat expert_mat(const moe_bank_t& b, bool w13, int e) {
  const size_t n = (size_t)2 * b.inter * b.hidden, m = (size_t)b.hidden * b.inter;
  const size_t w = w13 ? n : m;
  HostMat h;
  h.lo = (const uint8_t*)(w13 ? b.w13 : b.w2) + (size_t)e * (w / 4);
  h.hi = b.fmt == MOE_FMT_Q3 ? (const uint8_t*)(w13 ? b.w13_hi : b.w2_hi) + (size_t)e * (w / 8) : nullptr;
  h.scale = (w13 ? b.w13_scale : b.w2_scale) + (size_t)e * (w / 32);
  h.N = w13 ? 2 * b.inter : b.hidden;
  h.K = w13 ? b.hidden : b.inter;
  return h;
}

float silu(float a) { return a / (1.0f + std::exp(-a)); }

constexpr int kGateRows = 8;    // rows of I per gate/up unit
constexpr int kDownRows = 32;   // rows of H per down unit
constexpr int kSumCols = 256;   // columns of H per final-sum unit

}  // namespace

int cpu_isa() { return isa(); }

int cpu_expert_ffn(const moe_bank_t& bank, const uint16_t* x, int T, int k, const int32_t* ids,
                   const float* gates, const int32_t* rows, int n_rows, float* y, int n_threads) {
  const int H = bank.hidden, I = bank.inter;
  std::lock_guard<std::mutex> call(g_call);
  const int want = n_threads > 0 ? n_threads : default_threads();
  if (!g_pool || g_pool->size() != want) {
    g_pool.reset();
    g_pool.reset(new Pool(want));
  }
  Pool& pool = *g_pool;
  const Kernels kn = kernels();

  // 1. entries grouped by expert
  std::vector<int> order(n_rows);   // indices into rows[]
  for (int p = 0; p < n_rows; ++p) order[p] = p;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return ids[rows[a]] < ids[rows[b]]; });
  std::vector<int> pos_of(n_rows);   // rows[] index -> position in order
  for (int p = 0; p < n_rows; ++p) pos_of[order[p]] = p;
  std::vector<int> gstart;
  for (int p = 0; p < n_rows; ++p)
    if (p == 0 || ids[rows[order[p]]] != ids[rows[order[p - 1]]]) gstart.push_back(p);
  const int n_groups = (int)gstart.size();
  gstart.push_back(n_rows);

  // tokens with at least one entry, and each token's entries in rows[] (contiguous: rows ascend)
  std::vector<int> tok_first(T + 1, 0);
  for (int p = 0; p < n_rows; ++p) tok_first[rows[p] / k + 1]++;
  for (int t = 0; t < T; ++t) tok_first[t + 1] += tok_first[t];
  std::vector<int> toks;
  for (int t = 0; t < T; ++t)
    if (tok_first[t + 1] > tok_first[t]) toks.push_back(t);

  g_xp.resize((size_t)T * H);
  g_hp.resize((size_t)n_rows * I);
  g_z.resize((size_t)n_rows * H);
  float* xp = g_xp.data();
  float* hp = g_hp.data();
  float* z = g_z.data();

  // 2. activations in act_pos order
  pool.run((int)toks.size(), [&](int u) {
    const int t = toks[u];
    kn.prep(x + (size_t)t * H, H, xp + (size_t)t * H);
  });

  // 3. gate/up and SwiGLU: h of entry at position p is hp[p * I + act_pos(j)]
  const int gu_chunks = I / kGateRows;
  pool.run(n_groups * gu_chunks, [&](int u) {
    const int g = u / gu_chunks, j0 = (u % gu_chunks) * kGateRows;
    const int p0 = gstart[g], nt = gstart[g + 1] - p0;
    const int e = ids[rows[order[p0]]];
    std::vector<const float*> xs(nt);
    for (int j = 0; j < nt; ++j) xs[j] = xp + (size_t)(rows[order[p0 + j]] / k) * H;
    std::vector<float> a((size_t)kGateRows * nt), b((size_t)kGateRows * nt);
    const HostMat w13 = expert_mat(bank, true, e);
    kn.dot(w13, j0, kGateRows, xs.data(), nt, a.data(), nt);
    kn.dot(w13, I + j0, kGateRows, xs.data(), nt, b.data(), nt);
    for (int r = 0; r < kGateRows; ++r)
      for (int j = 0; j < nt; ++j)
        hp[(size_t)(p0 + j) * I + act_pos(j0 + r)] = silu(a[(size_t)r * nt + j]) * b[(size_t)r * nt + j];
  });

  // 4. down: z of entry at position p is z[p * H + n]
  const int dn_chunks = H / kDownRows;
  pool.run(n_groups * dn_chunks, [&](int u) {
    const int g = u / dn_chunks, n0 = (u % dn_chunks) * kDownRows;
    const int p0 = gstart[g], nt = gstart[g + 1] - p0;
    const int e = ids[rows[order[p0]]];
    std::vector<const float*> hs(nt);
    for (int j = 0; j < nt; ++j) hs[j] = hp + (size_t)(p0 + j) * I;
    std::vector<float> o((size_t)kDownRows * nt);
    kn.dot(expert_mat(bank, false, e), n0, kDownRows, hs.data(), nt, o.data(), nt);
    for (int r = 0; r < kDownRows; ++r)
      for (int j = 0; j < nt; ++j) z[(size_t)(p0 + j) * H + n0 + r] = o[(size_t)r * nt + j];
  });

  // 5. gate-weighted sum per token in ascending entry order
  const int sum_chunks = (H + kSumCols - 1) / kSumCols;
  pool.run(T * sum_chunks, [&](int u) {
    const int t = u / sum_chunks, c0 = (u % sum_chunks) * kSumCols, c1 = std::min(H, c0 + kSumCols);
    float* yt = y + (size_t)t * H;
    for (int c = c0; c < c1; ++c) yt[c] = 0.0f;
    for (int q = tok_first[t]; q < tok_first[t + 1]; ++q) {
      const float g = gates[rows[q]];
      const float* zr = z + (size_t)pos_of[q] * H;
      for (int c = c0; c < c1; ++c) yt[c] += g * zr[c];
    }
  });
  return MOE_OK;
}

}  // namespace moe_host

extern "C" {

int moe_cpu_isa(void) { return moe_host::cpu_isa(); }

int moe_cpu_expert_ffn(const moe_bank_t* bank, const uint16_t* x, int32_t T, int32_t k, const int32_t* ids,
                       const float* gates, const int32_t* rows, int32_t n_rows, float* y, int32_t n_threads) {
  if (!bank || !x || !ids || !gates || !y || T <= 0 || T > MOE_MAX_TOKENS || k <= 0 || n_rows < 0 || n_threads < 0)
    return MOE_EINVAL;
  if (n_rows > 0 && !rows) return MOE_EINVAL;
  if ((int64_t)n_rows > (int64_t)T * k) return MOE_EINVAL;
  const moe_bank_t& b = *bank;
  if (b.fmt != MOE_FMT_Q2 && b.fmt != MOE_FMT_Q3) return MOE_EUNSUPPORTED;
  if (b.n_experts <= 0 || b.hidden <= 0 || b.inter <= 0) return MOE_EINVAL;
  if (b.hidden % 128 || b.inter % 128) return MOE_EINVAL;
  if (!b.w13 || !b.w13_scale || !b.w2 || !b.w2_scale) return MOE_EINVAL;
  if (b.fmt == MOE_FMT_Q3 && (!b.w13_hi || !b.w2_hi)) return MOE_EINVAL;
  for (int32_t p = 0; p < n_rows; ++p) {
    const int32_t r = rows[p];
    if (r < 0 || r >= T * k || (p > 0 && r <= rows[p - 1])) return MOE_EINVAL;
    if (ids[r] < 0 || ids[r] >= b.n_experts) return MOE_EINVAL;
  }
  if (moe_host::cpu_isa() == 0) return MOE_EUNSUPPORTED;
  return moe_host::cpu_expert_ffn(b, x, T, k, ids, gates, rows, n_rows, y, n_threads);
}

}  // extern "C"
