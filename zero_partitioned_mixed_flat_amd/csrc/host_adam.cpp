// host_adam.cpp -- the C ABI of include/zero_host_adam.h: one rank's shard
// Adam step over host memory, vectorised (AVX-512 or AVX2, F16C for the
// binary16 conversions) and spread over the host cores with OpenMP, as the
// CPU Adam of ZeRO-Offload ("DeepSpeed ZeRO Stages" section 5.1;
// "DeepSpeed ZeRO: Extreme Memory Efficiency", "Offloading the optimizer
// entirely: ZeRO-Offload").  The arithmetic is the GPU library's, operation
// for operation ("DeepSpeed ZeRO Stages" 2.1 equations; "ZeRO Stage 1 Math",
// "Where the 12 bytes come from"), so every instruction set level and the GPU
// give the same bits.
//
// Built with -ffp-contract=off: no multiply is fused with an add, in the
// intrinsic code or in the scalar tails.  Each worker thread runs with
// denormals kept (MXCSR FTZ and DAZ cleared) and round-to-nearest-even.
#include <immintrin.h>
#include <omp.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "zero_host_adam.h"

namespace {

// Elements per chunk: the unit of work of a thread and of the statistics'
// fixed summation order.
constexpr int64_t kChunk = 65536;
constexpr int kLanes = 16;  // interleaved accumulators of the sum of squares

thread_local char g_err[512] = "";

int fail(int status, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return ZERO_HOST_OK;
}

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  if (na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Per-step constants, each computed in double and rounded once.
struct Scalars {
  float b1, omb1, b2, omb2, bc1, bc2, lr, eps;
};

// ------------------------------------------------------------ ISA selection
int best_isa() {
  __builtin_cpu_init();
  if (!__builtin_cpu_supports("f16c")) return ZERO_HOST_ERR_UNSUPPORTED;
  if (__builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
      __builtin_cpu_supports("avx512vl") && __builtin_cpu_supports("avx2"))
    return ZERO_HOST_ISA_AVX512;
  if (__builtin_cpu_supports("avx2")) return ZERO_HOST_ISA_AVX2;
  return ZERO_HOST_ISA_SCALAR;
}

std::atomic<int> g_isa{0};  // 0 = not chosen yet

int current_isa() {
  int isa = g_isa.load(std::memory_order_relaxed);
  if (isa == 0) {
    isa = best_isa();
    g_isa.store(isa, std::memory_order_relaxed);
  }
  return isa;
}

// Keeps IEEE behaviour on this thread for the lifetime of the object.
struct IeeeMode {
  unsigned saved;
  IeeeMode() : saved(_mm_getcsr()) {
    // clear FTZ (bit 15), DAZ (bit 6) and the rounding mode (bits 13-14)
    _mm_setcsr(saved & ~((1u << 15) | (1u << 6) | (3u << 13)));
  }
  ~IeeeMode() { _mm_setcsr(saved); }
};

// Elements of the fp16 copy to write before p16 + lo reaches an `align`-byte
// boundary (p16 is 2-byte aligned).  The SIMD loops write the fp16 copy with
// non-temporal (streaming) stores, which need aligned addresses: it is the
// one output that is not read first, and a plain store would first read each
// of its lines from memory (2 B per parameter of the step's 32; measured on a
// 16-core host, 27.4-28.6 ms against 29.6-30.7 ms for the 375M shard).
inline int64_t p16_head(const uint16_t *p16, int64_t lo, int64_t hi, uintptr_t align) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p16 + lo);
  const int64_t head = static_cast<int64_t>(((align - (a & (align - 1))) & (align - 1)) / 2);
  return head < hi - lo ? head : hi - lo;
}

// ------------------------------------------------------------------ scalar
__attribute__((target("f16c"))) inline float load_grad(const void *grad, int dt, int64_t j) {
  if (dt == ZERO_HOST_F16) return _cvtsh_ss(static_cast<const uint16_t *>(grad)[j]);
  return static_cast<const float *>(grad)[j];
}

inline bool nonfinite_at(const void *grad, int dt, int64_t j) {
  if (dt == ZERO_HOST_F16) return (static_cast<const uint16_t *>(grad)[j] & 0x7C00u) == 0x7C00u;
  uint32_t b;
  std::memcpy(&b, static_cast<const float *>(grad) + j, 4);
  return (b & 0x7F800000u) == 0x7F800000u;
}

__attribute__((target("f16c"))) inline void adam_element(float x, float s, const Scalars &c, float &m, float &v,
                                                           float &th, uint16_t &p) {
  const float g = x * s;
  const float m1 = c.b1 * m + c.omb1 * g;
  const float v1 = c.b2 * v + c.omb2 * (g * g);
  const float mh = m1 / c.bc1;
  const float vh = v1 / c.bc2;
  const float th1 = th - c.lr * (mh / (std::sqrt(vh) + c.eps));
  m = m1;
  v = v1;
  th = th1;
  p = _cvtss_sh(th1, _MM_FROUND_TO_NEAREST_INT);
}

// Statistics of elements [lo, hi) of one chunk starting at `base`: element j
// adds to accumulator (j - base) % 16.
__attribute__((target("f16c"))) void stats_scalar(const void *grad, int dt, int64_t base, int64_t lo, int64_t hi,
                                                  float s, double acc[kLanes], uint32_t &flag) {
  for (int64_t j = lo; j < hi; ++j) {
    flag |= nonfinite_at(grad, dt, j) ? 1u : 0u;
    const double d = static_cast<double>(load_grad(grad, dt, j) * s);
    acc[(j - base) % kLanes] += d * d;
  }
}

__attribute__((target("f16c"))) void apply_scalar(const void *grad, int dt, float *master, float *m, float *v,
                                                  uint16_t *p16, int64_t lo, int64_t hi, const Scalars &c, float s) {
  for (int64_t j = lo; j < hi; ++j) adam_element(load_grad(grad, dt, j), s, c, m[j], v[j], master[j], p16[j]);
}

// -------------------------------------------------------------------- AVX2
#define ZH_AVX2 __attribute__((target("avx2,f16c")))

ZH_AVX2 inline __m256 load8(const void *grad, int dt, int64_t j) {
  if (dt == ZERO_HOST_F16)
    return _mm256_cvtph_ps(_mm_loadu_si128(reinterpret_cast<const __m128i *>(static_cast<const uint16_t *>(grad) + j)));
  return _mm256_loadu_ps(static_cast<const float *>(grad) + j);
}

ZH_AVX2 inline uint32_t nonfinite8(const void *grad, int dt, int64_t j) {
  if (dt == ZERO_HOST_F16) {
    const __m128i h = _mm_loadu_si128(reinterpret_cast<const __m128i *>(static_cast<const uint16_t *>(grad) + j));
    const __m128i e = _mm_and_si128(h, _mm_set1_epi16(0x7C00));
    return _mm_movemask_epi8(_mm_cmpeq_epi16(e, _mm_set1_epi16(0x7C00))) != 0 ? 1u : 0u;
  }
  const __m256i b = _mm256_loadu_si256(reinterpret_cast<const __m256i *>(static_cast<const float *>(grad) + j));
  const __m256i e = _mm256_and_si256(b, _mm256_set1_epi32(0x7F800000));
  return _mm256_movemask_epi8(_mm256_cmpeq_epi32(e, _mm256_set1_epi32(0x7F800000))) != 0 ? 1u : 0u;
}

// One chunk's statistics: 16 lanes as four __m256d accumulators.
ZH_AVX2 void stats_avx2(const void *grad, int dt, int64_t base, int64_t end, float s, double acc[kLanes],
                        uint32_t &flag) {
  __m256d a0 = _mm256_setzero_pd(), a1 = a0, a2 = a0, a3 = a0;
  const __m256 vs = _mm256_set1_ps(s);
  uint32_t f = 0u;
  int64_t j = base;
  for (; j + 16 <= end; j += 16) {
    f |= nonfinite8(grad, dt, j) | nonfinite8(grad, dt, j + 8);
    const __m256 p0 = _mm256_mul_ps(load8(grad, dt, j), vs);
    const __m256 p1 = _mm256_mul_ps(load8(grad, dt, j + 8), vs);
    const __m256d d0 = _mm256_cvtps_pd(_mm256_castps256_ps128(p0));
    const __m256d d1 = _mm256_cvtps_pd(_mm256_extractf128_ps(p0, 1));
    const __m256d d2 = _mm256_cvtps_pd(_mm256_castps256_ps128(p1));
    const __m256d d3 = _mm256_cvtps_pd(_mm256_extractf128_ps(p1, 1));
    a0 = _mm256_add_pd(a0, _mm256_mul_pd(d0, d0));
    a1 = _mm256_add_pd(a1, _mm256_mul_pd(d1, d1));
    a2 = _mm256_add_pd(a2, _mm256_mul_pd(d2, d2));
    a3 = _mm256_add_pd(a3, _mm256_mul_pd(d3, d3));
  }
  _mm256_storeu_pd(acc + 0, a0);
  _mm256_storeu_pd(acc + 4, a1);
  _mm256_storeu_pd(acc + 8, a2);
  _mm256_storeu_pd(acc + 12, a3);
  flag |= f;
  stats_scalar(grad, dt, base, j, end, s, acc, flag);
}

ZH_AVX2 void apply_avx2(const void *grad, int dt, float *master, float *m, float *v, uint16_t *p16, int64_t lo,
                        int64_t hi, const Scalars &c, float s) {
  const __m256 vs = _mm256_set1_ps(s), b1 = _mm256_set1_ps(c.b1), omb1 = _mm256_set1_ps(c.omb1);
  const __m256 b2 = _mm256_set1_ps(c.b2), omb2 = _mm256_set1_ps(c.omb2), bc1 = _mm256_set1_ps(c.bc1);
  const __m256 bc2 = _mm256_set1_ps(c.bc2), lr = _mm256_set1_ps(c.lr), eps = _mm256_set1_ps(c.eps);
  int64_t j = lo + p16_head(p16, lo, hi, 16);
  apply_scalar(grad, dt, master, m, v, p16, lo, j, c, s);
  for (; j + 8 <= hi; j += 8) {
    const __m256 g = _mm256_mul_ps(load8(grad, dt, j), vs);
    const __m256 m0 = _mm256_loadu_ps(m + j), v0 = _mm256_loadu_ps(v + j), t0 = _mm256_loadu_ps(master + j);
    const __m256 m1 = _mm256_add_ps(_mm256_mul_ps(b1, m0), _mm256_mul_ps(omb1, g));
    const __m256 v1 = _mm256_add_ps(_mm256_mul_ps(b2, v0), _mm256_mul_ps(omb2, _mm256_mul_ps(g, g)));
    const __m256 mh = _mm256_div_ps(m1, bc1);
    const __m256 vh = _mm256_div_ps(v1, bc2);
    const __m256 den = _mm256_add_ps(_mm256_sqrt_ps(vh), eps);
    const __m256 t1 = _mm256_sub_ps(t0, _mm256_mul_ps(lr, _mm256_div_ps(mh, den)));
    _mm256_storeu_ps(m + j, m1);
    _mm256_storeu_ps(v + j, v1);
    _mm256_storeu_ps(master + j, t1);
    const __m128i h = _mm256_cvtps_ph(t1, _MM_FROUND_TO_NEAREST_INT);
    _mm_stream_si128(reinterpret_cast<__m128i *>(p16 + j), h);
  }
  _mm_sfence();
  apply_scalar(grad, dt, master, m, v, p16, j, hi, c, s);
}

// ----------------------------------------------------------------- AVX-512
#define ZH_AVX512 __attribute__((target("avx512f,avx512bw,avx512vl,avx2,f16c")))

ZH_AVX512 inline __m512 load16(const void *grad, int dt, int64_t j) {
  if (dt == ZERO_HOST_F16)
    return _mm512_cvtph_ps(
        _mm256_loadu_si256(reinterpret_cast<const __m256i *>(static_cast<const uint16_t *>(grad) + j)));
  return _mm512_loadu_ps(static_cast<const float *>(grad) + j);
}

ZH_AVX512 inline uint32_t nonfinite16(const void *grad, int dt, int64_t j) {
  if (dt == ZERO_HOST_F16) {
    const __m256i h = _mm256_loadu_si256(reinterpret_cast<const __m256i *>(static_cast<const uint16_t *>(grad) + j));
    const __m256i e = _mm256_and_si256(h, _mm256_set1_epi16(0x7C00));
    return _mm256_cmpeq_epi16_mask(e, _mm256_set1_epi16(0x7C00)) != 0 ? 1u : 0u;
  }
  const __m512i b = _mm512_loadu_si512(static_cast<const float *>(grad) + j);
  const __m512i e = _mm512_and_si512(b, _mm512_set1_epi32(0x7F800000));
  return _mm512_cmpeq_epi32_mask(e, _mm512_set1_epi32(0x7F800000)) != 0 ? 1u : 0u;
}

ZH_AVX512 void stats_avx512(const void *grad, int dt, int64_t base, int64_t end, float s, double acc[kLanes],
                            uint32_t &flag) {
  __m512d lo8 = _mm512_setzero_pd(), hi8 = lo8;
  const __m512 vs = _mm512_set1_ps(s);
  uint32_t f = 0u;
  int64_t j = base;
  for (; j + 16 <= end; j += 16) {
    f |= nonfinite16(grad, dt, j);
    const __m512 p = _mm512_mul_ps(load16(grad, dt, j), vs);
    const __m512d d0 = _mm512_cvtps_pd(_mm512_castps512_ps256(p));
    const __m512d d1 = _mm512_cvtps_pd(_mm256_castpd_ps(_mm512_extractf64x4_pd(_mm512_castps_pd(p), 1)));
    lo8 = _mm512_add_pd(lo8, _mm512_mul_pd(d0, d0));
    hi8 = _mm512_add_pd(hi8, _mm512_mul_pd(d1, d1));
  }
  _mm512_storeu_pd(acc + 0, lo8);
  _mm512_storeu_pd(acc + 8, hi8);
  flag |= f;
  stats_scalar(grad, dt, base, j, end, s, acc, flag);
}

ZH_AVX512 void apply_avx512(const void *grad, int dt, float *master, float *m, float *v, uint16_t *p16, int64_t lo,
                            int64_t hi, const Scalars &c, float s) {
  const __m512 vs = _mm512_set1_ps(s), b1 = _mm512_set1_ps(c.b1), omb1 = _mm512_set1_ps(c.omb1);
  const __m512 b2 = _mm512_set1_ps(c.b2), omb2 = _mm512_set1_ps(c.omb2), bc1 = _mm512_set1_ps(c.bc1);
  const __m512 bc2 = _mm512_set1_ps(c.bc2), lr = _mm512_set1_ps(c.lr), eps = _mm512_set1_ps(c.eps);
  int64_t j = lo + p16_head(p16, lo, hi, 32);
  apply_scalar(grad, dt, master, m, v, p16, lo, j, c, s);
  for (; j + 16 <= hi; j += 16) {
    const __m512 g = _mm512_mul_ps(load16(grad, dt, j), vs);
    const __m512 m0 = _mm512_loadu_ps(m + j), v0 = _mm512_loadu_ps(v + j), t0 = _mm512_loadu_ps(master + j);
    const __m512 m1 = _mm512_add_ps(_mm512_mul_ps(b1, m0), _mm512_mul_ps(omb1, g));
    const __m512 v1 = _mm512_add_ps(_mm512_mul_ps(b2, v0), _mm512_mul_ps(omb2, _mm512_mul_ps(g, g)));
    const __m512 mh = _mm512_div_ps(m1, bc1);
    const __m512 vh = _mm512_div_ps(v1, bc2);
    const __m512 den = _mm512_add_ps(_mm512_sqrt_ps(vh), eps);
    const __m512 t1 = _mm512_sub_ps(t0, _mm512_mul_ps(lr, _mm512_div_ps(mh, den)));
    _mm512_storeu_ps(m + j, m1);
    _mm512_storeu_ps(v + j, v1);
    _mm512_storeu_ps(master + j, t1);
    const __m256i h = _mm512_cvtps_ph(t1, _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC);
    _mm256_stream_si256(reinterpret_cast<__m256i *>(p16 + j), h);
  }
  _mm_sfence();
  apply_scalar(grad, dt, master, m, v, p16, j, hi, c, s);
}

// ----------------------------------------------------------------- driver
void stats_chunk(int isa, const void *grad, int dt, int64_t base, int64_t end, float s, double &sumsq,
                 uint32_t &flag) {
  double acc[kLanes] = {0.0};
  uint32_t f = 0u;
  if (isa == ZERO_HOST_ISA_AVX512)
    stats_avx512(grad, dt, base, end, s, acc, f);
  else if (isa == ZERO_HOST_ISA_AVX2)
    stats_avx2(grad, dt, base, end, s, acc, f);
  else
    stats_scalar(grad, dt, base, base, end, s, acc, f);
  double t = acc[0];
  for (int k = 1; k < kLanes; ++k) t += acc[k];
  sumsq = t;
  flag = f;
}

void apply_chunk(int isa, const void *grad, int dt, float *master, float *m, float *v, uint16_t *p16, int64_t lo,
                 int64_t hi, const Scalars &c, float s) {
  if (isa == ZERO_HOST_ISA_AVX512)
    apply_avx512(grad, dt, master, m, v, p16, lo, hi, c, s);
  else if (isa == ZERO_HOST_ISA_AVX2)
    apply_avx2(grad, dt, master, m, v, p16, lo, hi, c, s);
  else
    apply_scalar(grad, dt, master, m, v, p16, lo, hi, c, s);
}

}  // namespace

extern "C" {

int zero_host_adam_set_isa(int32_t level) {
  const int best = best_isa();
  if (best < 0) return fail(best, "set_isa: the CPU lacks F16C");
  if (level < 0 || level > ZERO_HOST_ISA_AVX512) return fail(ZERO_HOST_ERR_INVALID_ARG, "set_isa: bad level %d", level);
  const int isa = (level == 0 || level > best) ? best : level;
  g_isa.store(isa, std::memory_order_relaxed);
  ok();
  return isa;
}

int zero_host_adam_step(const void *grad, int32_t grad_dtype, double inv_grad_scale, float *master, float *exp_avg,
                        float *exp_avg_sq, uint16_t *param16, int64_t len, int64_t step,
                        const zero_host_adam_hparams_t *hp, zero_host_stats_t *stats, int32_t stats_precomputed,
                        int32_t n_threads) {
  if (len < 0) return fail(ZERO_HOST_ERR_INVALID_ARG, "host_adam: len < 0");
  if (grad_dtype != ZERO_HOST_F16 && grad_dtype != ZERO_HOST_F32)
    return fail(ZERO_HOST_ERR_INVALID_ARG, "host_adam: unknown grad dtype");
  if (hp == nullptr || stats == nullptr) return fail(ZERO_HOST_ERR_INVALID_ARG, "host_adam: NULL hp or stats");
  if (len > 0 && (grad == nullptr || master == nullptr || exp_avg == nullptr || exp_avg_sq == nullptr ||
                  param16 == nullptr))
    return fail(ZERO_HOST_ERR_INVALID_ARG, "host_adam: NULL array");
  if (step < 1) return fail(ZERO_HOST_ERR_INVALID_ARG, "host_adam: step must be >= 1");
  if (!(std::isfinite(hp->lr) && hp->lr >= 0.0)) return fail(ZERO_HOST_ERR_INVALID_ARG, "host_adam: bad lr");
  if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0) || !(hp->beta2 >= 0.0 && hp->beta2 < 1.0))
    return fail(ZERO_HOST_ERR_INVALID_ARG, "host_adam: betas must be in [0, 1)");
  if (!(std::isfinite(hp->eps) && hp->eps > 0.0)) return fail(ZERO_HOST_ERR_INVALID_ARG, "host_adam: eps must be > 0");
  if (!(std::isfinite(inv_grad_scale) && inv_grad_scale > 0.0))
    return fail(ZERO_HOST_ERR_INVALID_ARG, "host_adam: inv_grad_scale must be finite and > 0");
  if (!(std::isfinite(hp->max_grad_norm) && hp->max_grad_norm >= 0.0))
    return fail(ZERO_HOST_ERR_INVALID_ARG, "host_adam: max_grad_norm must be finite and >= 0");
  if (n_threads < 0) return fail(ZERO_HOST_ERR_INVALID_ARG, "host_adam: n_threads < 0");
  const auto misaligned = [](const void *q, uintptr_t a) { return (reinterpret_cast<uintptr_t>(q) & (a - 1)) != 0; };
  if (misaligned(grad, grad_dtype == ZERO_HOST_F16 ? 2 : 4) || misaligned(master, 4) || misaligned(exp_avg, 4) ||
      misaligned(exp_avg_sq, 4) || misaligned(param16, 2))
    return fail(ZERO_HOST_ERR_INVALID_ARG, "host_adam: an array is not aligned to its element size");
  if (len > INT64_MAX / 8) return fail(ZERO_HOST_ERR_INVALID_ARG, "host_adam: len too large");
  const size_t n = static_cast<size_t>(len);
  const void *arr[5] = {grad, master, exp_avg, exp_avg_sq, param16};
  const size_t sz[5] = {n * (grad_dtype == ZERO_HOST_F16 ? 2 : 4), n * 4, n * 4, n * 4, n * 2};
  for (int a = 0; a < 5; ++a)
    for (int b = a + 1; b < 5; ++b)
      if (overlap(arr[a], sz[a], arr[b], sz[b])) return fail(ZERO_HOST_ERR_INVALID_ARG, "host_adam: arrays overlap");
  const int isa = current_isa();
  if (isa < 0) return fail(isa, "host_adam: the CPU lacks F16C");

  const float s = static_cast<float>(inv_grad_scale);
  const int64_t nchunks = (len + kChunk - 1) / kChunk;
  const int nt = n_threads > 0 ? n_threads : omp_get_max_threads();

  uint32_t flag;
  double sumsq;
  if (stats_precomputed) {
    flag = stats->overflow != 0u ? 1u : 0u;
    sumsq = stats->sumsq;
  } else {
    std::vector<double> part(static_cast<size_t>(nchunks));
    std::vector<uint32_t> flags(static_cast<size_t>(nchunks));
#pragma omp parallel num_threads(nt)
    {
      IeeeMode mode;
#pragma omp for schedule(static)
      for (int64_t k = 0; k < nchunks; ++k) {
        const int64_t lo = k * kChunk, hi = lo + kChunk < len ? lo + kChunk : len;
        stats_chunk(isa, grad, grad_dtype, lo, hi, s, part[static_cast<size_t>(k)], flags[static_cast<size_t>(k)]);
      }
    }
    flag = 0u;
    sumsq = 0.0;
    for (int64_t k = 0; k < nchunks; ++k) {
      flag |= flags[static_cast<size_t>(k)];
      sumsq += part[static_cast<size_t>(k)];
    }
    stats->overflow = flag;
    stats->reserved = 0u;
    stats->sumsq = sumsq;
  }
  if (flag != 0u || len == 0) return ok();

  Scalars c;
  c.b1 = static_cast<float>(hp->beta1);
  c.omb1 = static_cast<float>(1.0 - hp->beta1);
  c.b2 = static_cast<float>(hp->beta2);
  c.omb2 = static_cast<float>(1.0 - hp->beta2);
  c.bc1 = static_cast<float>(1.0 - std::pow(hp->beta1, static_cast<double>(step)));
  c.bc2 = static_cast<float>(1.0 - std::pow(hp->beta2, static_cast<double>(step)));
  c.lr = static_cast<float>(hp->lr);
  c.eps = static_cast<float>(hp->eps);
  float s_eff = s;
  if (hp->max_grad_norm > 0.0) {
    const double norm = std::sqrt(sumsq);
    if (norm > hp->max_grad_norm) s_eff = static_cast<float>(inv_grad_scale * (hp->max_grad_norm / norm));
  }
#pragma omp parallel num_threads(nt)
  {
    IeeeMode mode;
#pragma omp for schedule(static)
    for (int64_t k = 0; k < nchunks; ++k) {
      const int64_t lo = k * kChunk, hi = lo + kChunk < len ? lo + kChunk : len;
      apply_chunk(isa, grad, grad_dtype, master, exp_avg, exp_avg_sq, param16, lo, hi, c, s_eff);
    }
  }
  return ok();
}

const char *zero_host_last_error(void) { return g_err; }

}  // extern "C"
