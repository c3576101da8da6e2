// Host executor of the expert FFN: the CPU side of CPU-GPU co-execution.
//
// On a cache miss the expert can either cross PCIe into VRAM or be computed
// where it already is, on the host cores that can read it from system RAM
// ("FreeToken Inference Engine: 3x Speed Boost for MoE Models", section
// "Q* Strategy: Intelligently Choosing Where to Compute"; the fork README
// names the CPU dot product as the part that needs AVX2/AVX-512).  This
// file computes h = silu(Wg x) * (Wu x), y = Wd h for a few tokens straight
// from the pinned host pool, in the same slot layout the GPU reads: rows of
// 256-weight groups, each group the quant bytes of 8 ggml blocks followed
// by their fifth bits, scales and offsets (for the types that have them).  x and y are fp32; every dot product accumulates
// in fp32.
//
// The rows of one call are split over a small pool of worker threads; the
// inner loops use AVX-512 when the CPU has it (checked at run time) and
// plain C++ otherwise.
#include <immintrin.h>

#include <atomic>
#include <cmath>
#include <condition_variable>
#include <cstring>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

#include "moe_internal.h"

namespace moe {
namespace {

float half_to_float(uint16_t h) {
  const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  const uint32_t ex = (h >> 10) & 0x1Fu, man = h & 0x3FFu;
  uint32_t bits;
  if (ex == 0) {
    if (man == 0) {
      bits = sign;
    } else {  // subnormal: normalise
      int e = -1;
      uint32_t m = man;
      do {
        m <<= 1;
        ++e;
      } while (!(m & 0x400u));
      bits = sign | ((uint32_t)(127 - 15 - e) << 23) | ((m & 0x3FFu) << 13);
    }
  } else if (ex == 31) {
    bits = sign | 0x7F800000u | (man << 13);
  } else {
    bits = sign | ((ex - 15 + 127) << 23) | (man << 13);
  }
  float f;
  std::memcpy(&f, &bits, 4);
  return f;
}

__attribute__((target("avx2"))) inline float _mm256_reduce_add_ps_(__m256 v) {
  const __m128 s = _mm_add_ps(_mm256_castps256_ps128(v), _mm256_extractf128_ps(v, 1));
  const __m128 t = _mm_add_ps(s, _mm_movehl_ps(s, s));
  return _mm_cvtss_f32(_mm_add_ss(t, _mm_shuffle_ps(t, t, 1)));
}

// ---------------------------------------------------------------- row dots
// sum_k w_k x_k over one row of `cols` weights (cols % 256 == 0); xs holds
// the sum of x over each 32-element block (used by the types with an offset
// m: w = d*u + m).
inline uint16_t load_u16(const uint8_t* p) {
  uint16_t v;
  std::memcpy(&v, p, 2);
  return v;
}
inline uint32_t load_u32(const uint8_t* p) {
  uint32_t v;
  std::memcpy(&v, p, 4);
  return v;
}

// K-quants: the 8 sub-blocks' scales d * scale_j and offsets -dmin * min_j
// of a group (exact in fp32), from the super-block's fp16 d, dmin and the
// 6-bit codes in its 12 packed bytes.
template <int QT>
inline void k_group_scales(const uint8_t* grp, float (&d)[8], float (&m)[8]) {
  const uint8_t* sc = grp + group_ksc_off(QT);
  const float dd = half_to_float(load_u16(grp + group_d_off(QT)));
  const float dm = half_to_float(load_u16(grp + group_m_off(QT)));
  for (int j = 0; j < 8; ++j) {
    const int s = j < 4 ? (sc[j] & 63) : ((sc[j + 4] & 15) | ((sc[j - 4] >> 6) << 4));
    const int n = j < 4 ? (sc[j + 4] & 63) : ((sc[j + 4] >> 4) | ((sc[j] >> 6) << 4));
    d[j] = dd * (float)s;
    m[j] = -(dm * (float)n);
  }
}

template <int QT>
float row_dot_scalar(const uint8_t* row, const float* x, const float* xs, int cols) {
  constexpr int qb = quant_bytes_per_block(QT);
  constexpr int off = (int)qtype_code_off(QT);
  float acc = 0.0f;
  for (int g = 0; g < cols / kGroupWeights; ++g) {
    const uint8_t* grp = row + (size_t)g * group_bytes(QT);
    float kd[8], km[8];
    if constexpr (qtype_is_k(QT)) k_group_scales<QT>(grp, kd, km);
    for (int b = 0; b < kGroupBlocks; ++b) {
      const float d = qtype_is_k(QT) ? kd[b] : half_to_float(load_u16(grp + group_d_off(QT) + 2 * b));
      const uint8_t* q = grp + b * qb;
      const float* xb = x + g * kGroupWeights + b * kQK;
      float s = 0.0f;
      if constexpr (QT == MOE_QTYPE_Q8_0) {
        for (int j = 0; j < 32; ++j) s += (float)(int8_t)q[j] * xb[j];
      } else {
        const uint32_t qh = qtype_has_qh(QT) ? load_u32(grp + group_qh_off(QT) + 4 * b) : 0u;
        for (int j = 0; j < 16; ++j) {
          const int u0 = (q[j] & 0x0F) | (int)(((qh >> j) & 1u) << 4);
          const int u1 = (q[j] >> 4) | (int)(((qh >> (j + 16)) & 1u) << 4);
          s += (float)(u0 - off) * xb[j];
          s += (float)(u1 - off) * xb[j + 16];
        }
      }
      acc += d * s;
      if constexpr (qtype_is_k(QT))
        acc += km[b] * xs[g * kGroupBlocks + b];
      else if constexpr (qtype_has_min(QT))
        acc += half_to_float(load_u16(grp + group_m_off(QT) + 2 * b)) * xs[g * kGroupBlocks + b];
    }
  }
  return acc;
}

template <int QT>
__attribute__((target("avx512f,avx512bw,avx512vl,f16c"))) float row_dot_avx512(const uint8_t* row, const float* x,
                                                                               const float* xs, int cols) {
  constexpr int qb = quant_bytes_per_block(QT);
  __m512 acc = _mm512_setzero_ps();
  float macc = 0.0f;
  const __m512i iota = _mm512_setr_epi32(0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
  for (int g = 0; g < cols / kGroupWeights; ++g) {
    const uint8_t* grp = row + (size_t)g * group_bytes(QT);
    alignas(32) float d[8];
    if constexpr (qtype_is_k(QT)) {
      float km[8];
      k_group_scales<QT>(grp, d, km);
      macc += _mm256_reduce_add_ps_(_mm256_mul_ps(_mm256_loadu_ps(km), _mm256_loadu_ps(xs + g * kGroupBlocks)));
    } else {
      const __m256 d8 = _mm256_cvtph_ps(_mm_loadu_si128(reinterpret_cast<const __m128i*>(grp + group_d_off(QT))));
      _mm256_store_ps(d, d8);
    }
    if constexpr (qtype_has_min(QT) && !qtype_is_k(QT)) {
      const __m256 m8 = _mm256_cvtph_ps(_mm_loadu_si128(reinterpret_cast<const __m128i*>(grp + group_m_off(QT))));
      macc += _mm256_reduce_add_ps_(_mm256_mul_ps(m8, _mm256_loadu_ps(xs + g * kGroupBlocks)));
    }
    const float* xg = x + g * kGroupWeights;
#pragma unroll
    for (int b = 0; b < kGroupBlocks; ++b) {
      const uint8_t* q = grp + b * qb;
      const float* xb = xg + b * kQK;
      __m512 lo, hi;
      if constexpr (QT == MOE_QTYPE_Q8_0) {
        lo = _mm512_cvtepi32_ps(_mm512_cvtepi8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(q))));
        hi = _mm512_cvtepi32_ps(_mm512_cvtepi8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(q + 16))));
      } else {
        const __m512i u = _mm512_cvtepu8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(q)));
        __m512i ul = _mm512_and_si512(u, _mm512_set1_epi32(0x0F)), uh = _mm512_srli_epi32(u, 4);
        if constexpr (qtype_has_qh(QT)) {
          const uint32_t qh = load_u32(grp + group_qh_off(QT) + 4 * b);
          const __m512i one = _mm512_set1_epi32(1);
          ul = _mm512_or_si512(ul, _mm512_slli_epi32(_mm512_and_si512(_mm512_srlv_epi32(_mm512_set1_epi32((int)qh), iota), one), 4));
          uh = _mm512_or_si512(uh, _mm512_slli_epi32(
                                       _mm512_and_si512(_mm512_srlv_epi32(_mm512_set1_epi32((int)(qh >> 16)), iota), one), 4));
        }
        if constexpr (!qtype_has_min(QT)) {
          const __m512i off = _mm512_set1_epi32((int)qtype_code_off(QT));
          ul = _mm512_sub_epi32(ul, off);
          uh = _mm512_sub_epi32(uh, off);
        }
        lo = _mm512_cvtepi32_ps(ul);
        hi = _mm512_cvtepi32_ps(uh);
      }
      __m512 s = _mm512_mul_ps(lo, _mm512_loadu_ps(xb));
      s = _mm512_fmadd_ps(hi, _mm512_loadu_ps(xb + 16), s);
      acc = _mm512_fmadd_ps(_mm512_set1_ps(d[b]), s, acc);
    }
  }
  return _mm512_reduce_add_ps(acc) + macc;
}

using RowDot = float (*)(const uint8_t*, const float*, const float*, int);

bool has_avx512() {
  static const bool ok = __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
                         __builtin_cpu_supports("avx512vl") && __builtin_cpu_supports("f16c");
  return ok;
}

RowDot row_dot_for(int qtype, bool vector) {
  switch (qtype) {
    case MOE_QTYPE_Q8_0: return vector ? row_dot_avx512<MOE_QTYPE_Q8_0> : row_dot_scalar<MOE_QTYPE_Q8_0>;
    case MOE_QTYPE_Q4_1: return vector ? row_dot_avx512<MOE_QTYPE_Q4_1> : row_dot_scalar<MOE_QTYPE_Q4_1>;
    case MOE_QTYPE_Q5_0: return vector ? row_dot_avx512<MOE_QTYPE_Q5_0> : row_dot_scalar<MOE_QTYPE_Q5_0>;
    case MOE_QTYPE_Q5_1: return vector ? row_dot_avx512<MOE_QTYPE_Q5_1> : row_dot_scalar<MOE_QTYPE_Q5_1>;
    case MOE_QTYPE_Q4_K: return vector ? row_dot_avx512<MOE_QTYPE_Q4_K> : row_dot_scalar<MOE_QTYPE_Q4_K>;
    case MOE_QTYPE_Q5_K: return vector ? row_dot_avx512<MOE_QTYPE_Q5_K> : row_dot_scalar<MOE_QTYPE_Q5_K>;
    default: return vector ? row_dot_avx512<MOE_QTYPE_Q4_0> : row_dot_scalar<MOE_QTYPE_Q4_0>;
  }
}

// Sums of v over each 32-element block.
void block_sums(const float* v, int n, float* out) {
  for (int b = 0; b < n / kQK; ++b) {
    float s = 0.0f;
    for (int j = 0; j < kQK; ++j) s += v[b * kQK + j];
    out[b] = s;
  }
}

// ---------------------------------------------------------------- threads
// Fork-join pool: run(n, fn) calls fn(0..n-1) spread over the workers and
// the calling thread and returns when all calls are done.  Idle workers
// spin briefly (a layer's two phases follow each other within
// microseconds), then sleep.
class HostPool {
 public:
  explicit HostPool(int workers) {
    for (int i = 0; i < workers; ++i) threads_.emplace_back([this] { loop(); });
  }
  ~HostPool() {
    {
      std::lock_guard<std::mutex> lk(mu_);
      stop_ = true;
      gen_.fetch_add(1);
    }
    cv_.notify_all();
    for (auto& t : threads_) t.join();
  }
  int size() const { return (int)threads_.size() + 1; }

  void run(int n, const std::function<void(int)>& fn) {
    if (n <= 0) return;
    if (threads_.empty() || n == 1) {
      for (int i = 0; i < n; ++i) fn(i);
      return;
    }
    {
      std::lock_guard<std::mutex> lk(mu_);
      fn_ = &fn;
      n_ = n;
      next_.store(0);
      busy_.store((int)threads_.size());
      gen_.fetch_add(1);
    }
    cv_.notify_all();
    work();
    while (busy_.load(std::memory_order_acquire) > 0) _mm_pause();
    fn_ = nullptr;
  }

 private:
  void work() {
    for (int i = next_.fetch_add(1); i < n_; i = next_.fetch_add(1)) (*fn_)(i);
  }
  void loop() {
    uint64_t seen = 0;  // the generation at construction: a run() may come before this thread starts
    for (;;) {
      int spins = 0;
      while (gen_.load(std::memory_order_acquire) == seen && spins < (1 << 14)) {
        _mm_pause();
        ++spins;
      }
      if (gen_.load(std::memory_order_acquire) == seen) {
        std::unique_lock<std::mutex> lk(mu_);
        cv_.wait(lk, [&] { return gen_.load() != seen; });
      }
      seen = gen_.load();
      if (stop_) return;
      work();
      busy_.fetch_sub(1, std::memory_order_release);
    }
  }
  std::vector<std::thread> threads_;
  std::mutex mu_;
  std::condition_variable cv_;
  std::atomic<uint64_t> gen_{0};
  std::atomic<int> next_{0}, busy_{0};
  const std::function<void(int)>* fn_ = nullptr;
  int n_ = 0;
  bool stop_ = false;
};

// One pool per process; calls are serialised (g_exec_mu is held for a whole
// host_experts_ffn), so the pool is never resized while it runs.
std::mutex g_exec_mu;
HostPool* g_pool = nullptr;
int g_pool_threads = 0;

HostPool* pool_for(int threads) {
  if (!g_pool || g_pool_threads != threads) {
    delete g_pool;
    g_pool = new HostPool(threads - 1);
    g_pool_threads = threads;
  }
  return g_pool;
}

constexpr int kRowChunk = 64;  // rows per task

}  // namespace

// All hardware threads but four, left to the GPU runtime and the calling
// thread's own launches (with every core busy the layer loop slowed down
// by up to a third on a 16-core host).
int default_host_threads() {
  const int n = (int)std::min(std::thread::hardware_concurrency(), 64u);
  return n <= 1 ? 1 : n <= 8 ? std::max(1, n / 2) : n - 4;
}

// n_exp experts, expert i at slots[i] (host), over tokens tok[i][0..cnt[i])
// of x [*, H]; writes y rows yrow[i][j] (row index into y [*, H]) .  h is
// scratch of sum(cnt) * I floats.
int host_experts_ffn(int qtype, int H, int I, int n_exp, const uint8_t* const* slots, const int* cnt,
                     const int* const* tok, const int* const* yrow, const float* x, float* y, float* h,
                     int threads, bool vector) {
  std::lock_guard<std::mutex> lk(g_exec_mu);
  HostPool* pool = pool_for(std::max(1, threads));
  const RowDot dot = row_dot_for(qtype, vector && has_avx512());
  std::vector<int> hbase(n_exp + 1, 0);
  for (int i = 0; i < n_exp; ++i) hbase[i + 1] = hbase[i] + cnt[i];
  const int ci = (I + kRowChunk - 1) / kRowChunk, ch = (H + kRowChunk - 1) / kRowChunk;
  const size_t gate = slot_gate_off(qtype, H, I), up = slot_up_off(qtype, H, I), down = slot_down_off(qtype, H, I);
  const size_t rb_h = row_bytes(qtype, H), rb_i = row_bytes(qtype, I);
  // block sums of every token's x and, after the first phase, of every h row
  const int n_rows = hbase[n_exp];
  std::vector<float> xs((size_t)n_rows * (H / kQK)), hs((size_t)n_rows * (I / kQK));
  for (int e = 0; e < n_exp; ++e)
    for (int j = 0; j < cnt[e]; ++j)
      block_sums(x + (size_t)tok[e][j] * H, H, xs.data() + (size_t)(hbase[e] + j) * (H / kQK));
  pool->run(n_exp * ci, [&](int task) {
    const int e = task / ci, r0 = (task % ci) * kRowChunk, r1 = std::min(I, r0 + kRowChunk);
    for (int r = r0; r < r1; ++r) {
      const uint8_t* gr = slots[e] + gate + (size_t)r * rb_h;
      const uint8_t* ur = slots[e] + up + (size_t)r * rb_h;
      for (int j = 0; j < cnt[e]; ++j) {
        const float* xt = x + (size_t)tok[e][j] * H;
        const float* st = xs.data() + (size_t)(hbase[e] + j) * (H / kQK);
        const float g = dot(gr, xt, st, H), u = dot(ur, xt, st, H);
        h[(size_t)(hbase[e] + j) * I + r] = g / (1.0f + std::exp(-g)) * u;
      }
    }
  });
  if (qtype_has_min(qtype))
    for (int i = 0; i < n_rows; ++i) block_sums(h + (size_t)i * I, I, hs.data() + (size_t)i * (I / kQK));
  pool->run(n_exp * ch, [&](int task) {
    const int e = task / ch, r0 = (task % ch) * kRowChunk, r1 = std::min(H, r0 + kRowChunk);
    for (int r = r0; r < r1; ++r) {
      const uint8_t* dr = slots[e] + down + (size_t)r * rb_i;
      for (int j = 0; j < cnt[e]; ++j)
        y[(size_t)yrow[e][j] * H + r] =
            dot(dr, h + (size_t)(hbase[e] + j) * I, hs.data() + (size_t)(hbase[e] + j) * (I / kQK), I);
    }
  });
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

int moe_host_expert_ffn(int qtype, int H, int I, const void* slot, const float* x, int n, float* y, int threads,
                        int vector) {
  clear_error();
  if (!qtype_supported(qtype))
    return set_error(MOE_ERR_UNSUPPORTED_QTYPE, "moe_host_expert_ffn: block type %d is not supported", qtype);
  if (H <= 0 || I <= 0 || H % kGroupWeights || I % kGroupWeights)
    return set_error(MOE_ERR_INVALID_ARG, "moe_host_expert_ffn: H=%d I=%d must be multiples of %d", H, I,
                     kGroupWeights);
  if (n < 0 || threads < 0) return set_error(MOE_ERR_INVALID_ARG, "moe_host_expert_ffn: n=%d threads=%d", n, threads);
  if (n == 0) return MOE_OK;
  if (!slot || !x || !y) return set_error(MOE_ERR_INVALID_ARG, "moe_host_expert_ffn: NULL slot, x or y");
  std::vector<int> tok(n);
  for (int i = 0; i < n; ++i) tok[i] = i;
  std::vector<float> h((size_t)n * I);
  const uint8_t* s = (const uint8_t*)slot;
  const int* tp = tok.data();
  return host_experts_ffn(qtype, H, I, 1, &s, &n, &tp, &tp, x, y, h.data(),
                          threads == 0 ? default_host_threads() : threads, vector != 0);
}

int moe_host_has_avx512(void) { return has_avx512() ? 1 : 0; }

}  // extern "C"
