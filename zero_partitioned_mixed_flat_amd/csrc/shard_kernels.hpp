// shard_kernels.hpp -- gfx950 kernels of the per-rank ZeRO shard optimizer
// step.  Every kernel is elementwise and bound by HBM bandwidth ("DeepSpeed
// ZeRO Stages" section 5.1: the step is O(1) arithmetic per parameter and
// touches the optimizer state once), so none uses MFMA; the design is about
// bytes in flight and access shape:
//   * in the update and the reduce each lane handles chunks of 4 consecutive
//     elements, so one wave's access to an fp32 stream is one contiguous
//     1 KiB (16 B per lane) and to an fp16 stream one contiguous 512 B (8 B
//     per lane); the read-only statistics pass, the all-gathers and the qwZ
//     encoder/decoder move 16 B of fp16 per lane;
//   * U chunks per lane are loaded before any is used, to keep enough loads
//     outstanding per CU to cover HBM latency;
//   * the update and the reduce run one tile per block over a grid of all
//     tiles, with non-temporal loads and stores (the streams are touched
//     once per step and are far larger than the caches); measured on MI355X
//     this beats grid-stride persistent blocks by 8-10%;
//   * their resident blocks per CU are capped (the host launches them with
//     an otherwise unused dynamic LDS allocation sized for the cap): with 4
//     to 64 concurrent streams, fewer requests in flight per CU let the
//     memory controllers keep DRAM rows open, which measured 6-8% faster
//     than full occupancy;
//   * the statistics pass uses a grid-stride loop over a grid sized from the
//     CU count (each block leaves one partial result), with 16-byte loads, 8
//     per lane in flight at 4 blocks per CU, walking the gradient from its
//     end: non-temporal for the bulk, cached for its first 256 MB, read
//     last, which the update then reads first, from the Infinity Cache
//     (statistics + update 1.638 ms on the 375M shard against 1.660 ms with
//     all loads non-temporal);
//   * reductions of the statistics: per-lane fp64 accumulation, butterfly
//     shuffles inside the wave, LDS across the block's waves, one partial per
//     block, then a single-block pass over the partials in index order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zero_shard.h"

namespace zs {

constexpr int kBlock = 256;        // threads per block (statistics, folds)
constexpr int kReduceBlock = 64;   // threads per block (reduce): one wave
constexpr int kReduceLane = 8;     // consecutive fp16 per lane per slice access (16 bytes)
constexpr int kUpdateBlock = 64;   // threads per block (update): one wave
constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kChunk = 4;          // consecutive elements per lane per access
constexpr int kMaxPartials = 2048; // partials of the grid-stride statistics kernel
constexpr int kFold = kBlock * 16;  // partials folded by one block of the first fold level

// Native vector types for the non-temporal load/store builtins.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ T stream_load(const T *p) {
  return __builtin_nontemporal_load(p);
}
template <typename T>
__device__ __forceinline__ void stream_store(T *p, T v) {
  __builtin_nontemporal_store(v, p);
}

// Streaming stores through a buffer window: a block-uniform base address
// and a size in bytes (accesses past it are dropped by the hardware), with
// the non-temporal and system-scope cache-policy bits (nt sc1; on gfx950 the
// policy operand is sc0 = 1, nt = 2, sc1 = 16).  Measured on MI355X, the
// update's state stores run 2.6% faster this way than as global stores with
// nt alone; loads show no such difference and stay global nt loads.
constexpr int kStreamStorePolicy = 2 | 16;
constexpr int kRawBufferWord3 = 0x00020000;  // raw (untyped) 32-bit buffer access

__device__ __forceinline__ __amdgpu_buffer_rsrc_t store_window(void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, static_cast<int>(bytes), kRawBufferWord3);
}
__device__ __forceinline__ void window_store(__amdgpu_buffer_rsrc_t w, uint32_t byte_off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, w, byte_off, 0, kStreamStorePolicy);
}
__device__ __forceinline__ void window_store(__amdgpu_buffer_rsrc_t w, uint32_t byte_off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), w, byte_off, 0, kStreamStorePolicy);
}
__device__ __forceinline__ void window_store(__amdgpu_buffer_rsrc_t w, uint32_t byte_off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, w, byte_off, 0, kStreamStorePolicy);
}
__device__ __forceinline__ void window_store(__amdgpu_buffer_rsrc_t w, uint32_t byte_off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, w, byte_off, 0, kStreamStorePolicy);
}

// 16-byte loads through a buffer window with the cache policy as an
// immediate: non-temporal (nt) for data read once, or the default policy,
// whose lines stay in the Infinity Cache (MI355X: 256 MB) for a kernel that
// reads them again.  The policy is part of the instruction, so two paths
// with different policies stay two paths; as plain and non-temporal global
// loads the compiler merges them and drops the nt bit.
constexpr int kStreamLoadPolicy = 2;
constexpr int kKeepLoadPolicy = 0;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t load_window(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes), kRawBufferWord3);
}
// Stores with the policy as an immediate, for the same reason: the reduce
// writes the bulk of its sum non-temporal and the last part, which the
// update reads next, with sc1 alone.
constexpr int kPlainStreamStorePolicy = 2;
constexpr int kKeepStorePolicy = 16;
template <int POLICY>
__device__ __forceinline__ void window_store_as(__amdgpu_buffer_rsrc_t w, uint32_t byte_off, const float (&x)[4]) {
  __builtin_amdgcn_raw_buffer_store_b128(
      u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])}, w, byte_off,
      0, POLICY);
}

template <int POLICY>
__device__ __forceinline__ u32x4 window_load(__amdgpu_buffer_rsrc_t w, uint32_t byte_off) {
  const auto r = __builtin_amdgcn_raw_buffer_load_b128(w, byte_off, 0, POLICY);
  return u32x4{r[0], r[1], r[2], r[3]};
}

// Per-step constants, each derived in double on the host and rounded once;
// inv_scale and max_norm stay in double for the clipping factor, which
// depends on the device-resident sum of squares.
struct StepScalars {
  float b1, omb1, b2, omb2, bc1, bc2, lr, eps, s;
  double inv_scale, max_norm;
};

// 1 - beta^t evaluated in double and rounded once to float: the bias
// correction of step t (Kingma & Ba, the Adam paper the "DeepSpeed ZeRO
// Stages" references cite).  Used when t is held in device memory.
__device__ __forceinline__ float bias_correction(double beta, int64_t t) {
  return static_cast<float>(1.0 - pow(beta, static_cast<double>(t)));
}

// The unscale multiplier of this step: s, or with global-norm clipping
// active (max_norm > 0 and sqrt(sumsq) > max_norm) the double product
// inv_scale * (max_norm / sqrt(sumsq)) rounded once to float.
__device__ __forceinline__ float step_scale(const StepScalars &c, const zero_grad_stats_t *stats) {
  if (!(c.max_norm > 0.0)) return c.s;
  const double norm = __builtin_sqrt(stats->sumsq);
  return norm > c.max_norm ? static_cast<float>(c.inv_scale * (c.max_norm / norm)) : c.s;
}

// One block's share of the statistics.
struct Partial {
  double sumsq;
  uint32_t flag;
  uint32_t pad;
};

struct SliceTable {
  const uint16_t *p[ZERO_MAX_SLICES];
};

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

__device__ __forceinline__ uint32_t f2h(float x) {
  // binary32 -> binary16 with the hardware conversion: round to nearest
  // even (the default mode), overflow to inf, subnormals kept.
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(x)));
}

__device__ __forceinline__ bool nonfinite_f32(float x) {
  return (__float_as_uint(x) & 0x7F800000u) == 0x7F800000u;
}

// The overflow test by maxima.  Without its sign bit, an fp16 bit pattern
// is +-inf or NaN exactly when it is >= 0x7C00, and an fp32 one exactly when
// it is >= 0x7F800000.  The streaming kernels keep the running maximum of
// those magnitudes (two fp16 values at a time with one packed 16-bit max)
// and compare once at the end, two instructions per pair of values instead
// of a mask, a compare and a scalar OR per value.
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u16x2 max_mag_f16x2(u16x2 m, uint32_t w) {
  return __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu));
}
__device__ __forceinline__ uint32_t max_mag_f32(uint32_t m, float x) {
  const uint32_t b = __float_as_uint(x) & 0x7FFFFFFFu;
  return b > m ? b : m;
}
__device__ __forceinline__ uint32_t nonfinite_mag_f16x2(u16x2 m) {
  return static_cast<uint32_t>(m.x >= 0x7C00u) | static_cast<uint32_t>(m.y >= 0x7C00u);
}
__device__ __forceinline__ uint32_t nonfinite_mag_f32(uint32_t m) {
  return static_cast<uint32_t>(m >= 0x7F800000u);
}

// The Adam update of one element ("DeepSpeed ZeRO Stages" 2.1 equations;
// "ZeRO Stage 1 Math", "Where the 12 bytes come from"): one IEEE binary32
// operation per operator in the order written, nothing fused.
__device__ __forceinline__ void adam_element(float x, float &m, float &v, float &th,
                                             uint32_t &p16, const StepScalars &c, float s) {
#pragma clang fp contract(off)
  const float g = x * s;
  const float m1 = c.b1 * m + c.omb1 * g;
  const float v1 = c.b2 * v + c.omb2 * (g * g);
  const float mh = m1 / c.bc1;
  const float vh = v1 / c.bc2;
  const float th1 = th - c.lr * (mh / (__builtin_sqrtf(vh) + c.eps));
  m = m1;
  v = v1;
  th = th1;
  p16 = f2h(th1);
}

// Sum of a double and OR of a flag over a block of BS threads; thread 0
// stores them.
template <int BS = kBlock>
__device__ __forceinline__ void block_partial(double ssq, uint32_t flag, Partial *out) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    ssq += __shfl_xor(ssq, off, kWave);
    flag |= __shfl_xor(flag, off, kWave);
  }
  static_assert(BS % kWave == 0, "whole waves");
  if constexpr (BS == kWave) {
    // one wave: the butterfly already left the totals in every lane
    if (threadIdx.x == 0) {
      out->sumsq = ssq;
      out->flag = flag;
      out->pad = 0u;
    }
    return;
  }
  __shared__ double s_ssq[BS / kWave];
  __shared__ uint32_t s_flag[BS / kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  if (lane == 0) {
    s_ssq[wave] = ssq;
    s_flag[wave] = flag;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = s_ssq[0];
    uint32_t f = s_flag[0];
#pragma unroll
    for (int w = 1; w < BS / kWave; ++w) {
      t += s_ssq[w];
      f |= s_flag[w];
    }
    out->sumsq = t;
    out->flag = f;
    out->pad = 0u;
  }
}

// acc + (x*s)^2 in double.  The product x*s is rounded to binary32 (the
// unscaled gradient the update sees); its square has at most 48 significant
// bits and lies between 2^-298 and 2^256, so it is exact in double, and one
// fused multiply-add gives the same result as the square and the add
// performed separately.
__device__ __forceinline__ double add_sq_unscaled(double acc, float x, float s) {
#pragma clang fp contract(off)
  const double d = static_cast<double>(x * s);
  return __builtin_fma(d, d, acc);
}

// ---------------------------------------------------------------- statistics
// Pass 1 of the statistics: per-block flag and sum of squares.  Each lane
// loads 16 bytes per access (8 fp16 or 4 fp32 values), U accesses in flight,
// over a grid-stride loop that walks the tiles from the last to the first.
// Tiles below element keep_below are loaded with the default cache policy
// and the rest with non-temporal loads: they are read last, and the update
// that follows reads the gradient from element 0, so it starts on lines that
// still sit in the Infinity Cache.  (Walking forward and keeping the last
// 256 MB instead, the update reached them only at its end, after some had
// been displaced: the step took 0.2-0.8% longer.)
template <zero_dtype_t DT>
constexpr int stats_per_lane() {
  return DT == ZERO_F16 ? 8 : 4;
}

template <int U, int POLICY>
__device__ __forceinline__ void stats_tile_load(__amdgpu_buffer_rsrc_t w, uint32_t lane_bytes, u32x4 (&raw)[U]) {
#pragma unroll
  for (int k = 0; k < U; ++k) raw[k] = window_load<POLICY>(w, lane_bytes + k * (kBlock * 16u));
}

template <zero_dtype_t DT, int U>
__global__ __launch_bounds__(kBlock) void grad_stats_kernel(const void *__restrict__ grad,
                                                            int64_t len, float s,
                                                            Partial *__restrict__ partials,
                                                            int64_t keep_below) {
  constexpr int kPer = stats_per_lane<DT>();
  constexpr int kElem = DT == ZERO_F16 ? 2 : 4;
  constexpr int64_t kTile = static_cast<int64_t>(kBlock) * kPer * U;
  const int64_t ntiles = (len + kTile - 1) / kTile;
  double acc0 = 0.0, acc1 = 0.0;
  uint32_t flag = 0u;
  u16x2 mag16 = {0, 0};  // running maxima of the magnitudes' bit patterns
  uint32_t mag32 = 0u;
  const uint32_t lane_bytes = threadIdx.x * 16u;
  for (int64_t step = blockIdx.x; step < ntiles; step += gridDim.x) {
    const int64_t base = (ntiles - 1 - step) * kTile;
    if (base + kTile <= len) {
      const auto w = load_window(static_cast<const char *>(grad) + base * kElem, kTile * kElem);
      u32x4 raw[U];
      if (base < keep_below)
        stats_tile_load<U, kKeepLoadPolicy>(w, lane_bytes, raw);
      else
        stats_tile_load<U, kStreamLoadPolicy>(w, lane_bytes, raw);
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const uint32_t wd[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
        if constexpr (DT == ZERO_F16) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            mag16 = max_mag_f16x2(mag16, wd[q]);
            acc0 = add_sq_unscaled(acc0, h2f(wd[q] & 0xFFFFu), s);
            acc1 = add_sq_unscaled(acc1, h2f(wd[q] >> 16), s);
          }
        } else {
          const float x[4] = {__uint_as_float(wd[0]), __uint_as_float(wd[1]), __uint_as_float(wd[2]),
                              __uint_as_float(wd[3])};
#pragma unroll
          for (int q = 0; q < 4; ++q) mag32 = max_mag_f32(mag32, x[q]);
          acc0 = add_sq_unscaled(acc0, x[0], s);
          acc1 = add_sq_unscaled(acc1, x[1], s);
          acc0 = add_sq_unscaled(acc0, x[2], s);
          acc1 = add_sq_unscaled(acc1, x[3], s);
        }
      }
    } else {
      // the ragged last tile, element by element
      const int64_t end = len < base + kTile ? len : base + kTile;
      for (int64_t j = base + threadIdx.x; j < end; j += kBlock) {
        float x;
        if constexpr (DT == ZERO_F16) {
          const uint32_t h = static_cast<const uint16_t *>(grad)[j];
          flag |= static_cast<uint32_t>((h & 0x7C00u) == 0x7C00u);
          x = h2f(h);
        } else {
          x = static_cast<const float *>(grad)[j];
          flag |= static_cast<uint32_t>(nonfinite_f32(x));
        }
        acc0 = add_sq_unscaled(acc0, x, s);
      }
    }
  }
  flag |= nonfinite_mag_f16x2(mag16) | nonfinite_mag_f32(mag32);
  block_partial(acc0 + acc1, flag, &partials[blockIdx.x]);
}

// Pass 2: one block folds the partials in a fixed order: thread t adds
// partials t, t + kBlock, t + 2*kBlock, ... in index order, loading eight of
// them before adding any (one memory round trip per eight instead of one
// each: the partials were just written by blocks on every XCD).
__global__ __launch_bounds__(kBlock) void finalize_stats_kernel(const Partial *__restrict__ partials,
                                                                int nparts,
                                                                zero_grad_stats_t *__restrict__ stats) {
  constexpr int kBatch = 8;
  double ssq = 0.0;
  uint32_t flag = 0u;
  for (int base = 0; base < nparts; base += kBatch * kBlock) {
    Partial p[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int i = base + k * kBlock + static_cast<int>(threadIdx.x);
      p[k] = i < nparts ? partials[i] : Partial{0.0, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      if (base + k * kBlock + static_cast<int>(threadIdx.x) < nparts) ssq += p[k].sumsq;
      flag |= p[k].flag;
    }
  }
  __shared__ Partial total;
  block_partial(ssq, flag, &total);
  __syncthreads();
  if (threadIdx.x == 0) {
    stats->overflow = total.flag != 0u ? 1u : 0u;
    stats->reserved = 0u;
    stats->sumsq = total.sumsq;
  }
}

// First level of folding many partials: block b folds the contiguous range
// [b*kFold, (b+1)*kFold) in a fixed order into out[b].
__global__ __launch_bounds__(kBlock) void fold_partials_kernel(const Partial *__restrict__ in, int64_t n,
                                                               Partial *__restrict__ out) {
  const int64_t begin = static_cast<int64_t>(blockIdx.x) * kFold;
  double ssq = 0.0;
  uint32_t flag = 0u;
#pragma unroll
  for (int i = 0; i < kFold / kBlock; ++i) {
    const int64_t j = begin + i * kBlock + threadIdx.x;
    if (j < n) {
      ssq += in[j].sumsq;
      flag |= in[j].flag;
    }
  }
  block_partial(ssq, flag, &out[blockIdx.x]);
}

// -------------------------------------------------------------------- reduce
// Owner-side reduce of N fp16 slices into fp32, left fold in rank order,
// optionally with the statistics of (sum * s) in the same pass.  One wave
// per tile of kReduceBlock*8*U elements (one partial per block); each lane
// reads 8 consecutive fp16 (16 bytes) of a slice per access, slices G at a
// time with non-temporal loads, so G*U loads are in flight before the
// in-order adds.  The lane's 8 sums pass through LDS so that each store
// instruction writes 1 KB contiguous (two 16-byte stores per lane at a
// 32-byte stride would leave every 32-byte piece half written by each
// instruction, and the counters showed 1.6 times the sum's bytes written).
// The sum is written non-temporal up to element keep_from and with sc1 from
// there on: the update that reads the sum next finds that part in the
// Infinity Cache.
template <bool WITH_STATS, int U, int G>
__global__ __launch_bounds__(kReduceBlock) void grad_reduce_kernel(SliceTable tab, int n, int64_t len,
                                                                   float *__restrict__ out, float s,
                                                                   Partial *__restrict__ partials,
                                                                   int64_t keep_from) {
#pragma clang fp contract(off)
  constexpr int kSpan = kReduceBlock * kReduceLane;
  constexpr int64_t kTile = static_cast<int64_t>(kSpan) * U;
  const int64_t ntiles = (len + kTile - 1) / kTile;
  double acc0 = 0.0, acc1 = 0.0;
  uint32_t flag = 0u;
  uint32_t mag32 = 0u;  // running maximum of the sums' magnitude bit patterns
  // addresses = a tile base that is the same for the whole block (kept in
  // scalar registers) + a 32-bit lane offset; with per-lane 64-bit addresses
  // the compiler serialises the slice loads
  const uint32_t lane = threadIdx.x * kReduceLane;
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t tbase = tile * kTile;
    if (tbase + kTile <= len) {
      float acc[U][kReduceLane];
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const u32x4 raw = stream_load(reinterpret_cast<const u32x4 *>(tab.p[0] + tbase + lane + k * kSpan));
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[k][2 * e] = h2f(w[e] & 0xFFFFu);
          acc[k][2 * e + 1] = h2f(w[e] >> 16);
        }
      }
      for (int r0 = 1; r0 < n; r0 += G) {
        const int cnt = (n - r0) < G ? (n - r0) : G;
        u32x4 raw[G][U];
#pragma unroll
        for (int q = 0; q < G; ++q) {
          if (q < cnt) {
            const uint16_t *p = tab.p[r0 + q] + tbase;
#pragma unroll
            for (int k = 0; k < U; ++k) raw[q][k] = stream_load(reinterpret_cast<const u32x4 *>(p + lane + k * kSpan));
          }
        }
#pragma unroll
        for (int q = 0; q < G; ++q) {
          if (q < cnt) {
#pragma unroll
            for (int k = 0; k < U; ++k) {
              const uint32_t w[4] = {raw[q][k].x, raw[q][k].y, raw[q][k].z, raw[q][k].w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                acc[k][2 * e] = acc[k][2 * e] + h2f(w[e] & 0xFFFFu);
                acc[k][2 * e + 1] = acc[k][2 * e + 1] + h2f(w[e] >> 16);
              }
            }
          }
        }
      }
      // chunk k of the tile: element 8*lane + e sits in lane `lane`; staged so
      // that lane l then holds elements 4l..4l+3 and kSpan/2 + 4l..+3
      __shared__ f32x4 stage[2 * kReduceBlock];
      const auto wo = store_window(out + tbase, kTile * 4);
#pragma unroll
      for (int k = 0; k < U; ++k) {
        stage[2 * threadIdx.x] = f32x4{acc[k][0], acc[k][1], acc[k][2], acc[k][3]};
        stage[2 * threadIdx.x + 1] = f32x4{acc[k][4], acc[k][5], acc[k][6], acc[k][7]};
        __syncthreads();
        const f32x4 lo = stage[threadIdx.x], hi = stage[kReduceBlock + threadIdx.x];
        __syncthreads();
        const float l4[4] = {lo.x, lo.y, lo.z, lo.w}, h4[4] = {hi.x, hi.y, hi.z, hi.w};
        const uint32_t o0 = (k * kSpan + threadIdx.x * 4) * 4u;
        const uint32_t o1 = (k * kSpan + kSpan / 2 + threadIdx.x * 4) * 4u;
        if (tbase >= keep_from) {
          window_store_as<kKeepStorePolicy>(wo, o0, l4);
          window_store_as<kKeepStorePolicy>(wo, o1, h4);
        } else {
          window_store_as<kPlainStreamStorePolicy>(wo, o0, l4);
          window_store_as<kPlainStreamStorePolicy>(wo, o1, h4);
        }
      }
      if constexpr (WITH_STATS) {
#pragma unroll
        for (int k = 0; k < U; ++k) {
#pragma unroll
          for (int e = 0; e < kReduceLane; ++e) {
            mag32 = max_mag_f32(mag32, acc[k][e]);
            if (e & 1)
              acc1 = add_sq_unscaled(acc1, acc[k][e], s);
            else
              acc0 = add_sq_unscaled(acc0, acc[k][e], s);
          }
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < U; ++k) {
#pragma unroll
        for (int e = 0; e < kReduceLane; ++e) {
          const int64_t j = tbase + lane + k * kSpan + e;
          if (j < len) {
            float a = h2f(tab.p[0][j]);
            for (int r = 1; r < n; ++r) a = a + h2f(tab.p[r][j]);
            out[j] = a;
            if constexpr (WITH_STATS) {
              flag |= static_cast<uint32_t>(nonfinite_f32(a));
              acc0 = add_sq_unscaled(acc0, a, s);
            }
          }
        }
      }
    }
  }
  if constexpr (WITH_STATS) {
    flag |= nonfinite_mag_f32(mag32);
    block_partial<kReduceBlock>(acc0 + acc1, flag, &partials[blockIdx.x]);
  }
}

// --------------------------------------------------------------- all-gather
// Concatenation of N fp16 shards into the flat replica: block (x, y) copies
// tile x of shard y (and every gridDim.x-th tile after it, when the shard has
// more tiles than one launch may have blocks), 16 bytes (8 values) per lane
// with non-temporal access; only the part of the shard below psi is copied.
constexpr int kGatherBlock = 64;
constexpr int kGatherU = 1;
constexpr int64_t kGatherTile = static_cast<int64_t>(kGatherBlock) * 8 * kGatherU;
__global__ __launch_bounds__(kGatherBlock) void allgather_kernel(SliceTable tab, int64_t shard_len, int64_t psi,
                                                                 uint16_t *__restrict__ replica) {
  const int r = blockIdx.y;
  const int64_t first = static_cast<int64_t>(r) * shard_len;
  const int64_t real = psi - first < shard_len ? psi - first : shard_len;
  const uint32_t lane = threadIdx.x * 8;
  for (int64_t tbase = static_cast<int64_t>(blockIdx.x) * kGatherTile; tbase < real;
       tbase += static_cast<int64_t>(gridDim.x) * kGatherTile) {
    const uint16_t *src = tab.p[r] + tbase;
    uint16_t *dst = replica + first + tbase;
    if (tbase + kGatherTile <= real) {
      u32x4 x[kGatherU];
#pragma unroll
      for (int k = 0; k < kGatherU; ++k)
        x[k] = stream_load(reinterpret_cast<const u32x4 *>(src + lane + k * kGatherBlock * 8));
#pragma unroll
      for (int k = 0; k < kGatherU; ++k)
        stream_store(reinterpret_cast<u32x4 *>(dst + lane + k * kGatherBlock * 8), x[k]);
    } else {
      const int64_t rem = real - tbase;
      for (int64_t j = threadIdx.x; j < rem; j += kGatherBlock) dst[j] = src[j];
    }
  }
}

// ----------------------------------------------------------------------- qwZ
// Block INT8 codec of the fp16 weights ("DeepSpeed ZeRO Stages" 5.3, qwZ;
// ZeRO++ in "ZeRO Optimization: Stages 1, 2, and 3 Explained"): blocks of
// kQwzBlock consecutive values of a shard, scale = max|x| / 127 in binary32,
// code = clamp(rint(x / scale), -127, 127) with a correctly rounded division
// and ties to even, all codes 0 when the scale is 0; decoding is
// f16(code * scale).  One row of a wave (64 lanes x 4 values) is exactly one
// block, so each block maximum is one wave reduction.
constexpr int kQwzBlock = ZERO_QWZ_BLOCK;
static_assert(kQwzBlock == kWave * kChunk, "a qwZ block is one wave row");

__device__ __forceinline__ float wave_max(float a) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) a = __builtin_fmaxf(a, __shfl_xor(a, off, kWave));
  return a;
}

// Quotients rint(x[e] / scale) of N values of a block with scale > 0.  The
// code is defined by Q = x/scale correctly rounded, then rint(Q); a full
// division per value is costly, so the quotient is first estimated as
// t = x*inv with inv = 1/scale correctly rounded.  |x/scale| <= 127, so
// |t - x/scale| and |Q - x/scale| are below 2^-16 and 2^-17: whenever t lies
// more than 2^-13 from every half-integer, t and Q lie strictly on the same
// side of each of them and rint(t) = rint(Q).  The values closer than that
// (possible ties) get the exact quotient, in a branch that the wave takes
// only when one of its lanes has such a value; the common path has no
// per-value branch.
template <int N>
__device__ __forceinline__ void qwz_quotients(const float (&x)[N], float scale, float (&q)[N]) {
  const float inv = 1.0f / scale;
  uint32_t near_half = 0u;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const float t = x[e] * inv;
    q[e] = __builtin_rintf(t);
    near_half |= static_cast<uint32_t>(!(__builtin_fabsf(t - q[e]) < 0.5f - 0x1p-13f)) << e;
  }
  if (__any(near_half != 0u)) {
#pragma unroll
    for (int e = 0; e < N; ++e)
      if ((near_half >> e) & 1u) q[e] = __builtin_rintf(x[e] / scale);
  }
}

// The code byte of a quotient: clamped to [-127, 127] with one med3.  (With
// scale = max|x|/127 rounded to nearest no quotient rounds beyond 127, so the
// clamp never changes a code; it is kept as the definition states it.)
__device__ __forceinline__ uint32_t qwz_byte(float q) {
  return static_cast<uint32_t>(static_cast<int32_t>(__builtin_amdgcn_fmed3f(q, -127.0f, 127.0f))) & 0xFFu;
}

// Scale of the block held by one wave row, from the lane's 4 values (0 for
// values outside the array), and the lane's 4 codes packed little-endian.
__device__ __forceinline__ float qwz_scale(const float (&x)[kChunk]) {
  float a = 0.0f;
#pragma unroll
  for (int e = 0; e < kChunk; ++e) a = __builtin_fmaxf(a, __builtin_fabsf(x[e]));
  return wave_max(a) / 127.0f;
}

__device__ __forceinline__ uint32_t qwz_pack(const float (&x)[kChunk], float scale) {
  if (scale == 0.0f) return 0u;
  float q[kChunk];
  qwz_quotients(x, scale, q);
  uint32_t w = 0u;
#pragma unroll
  for (int e = 0; e < kChunk; ++e) w |= qwz_byte(q[e]) << (8 * e);
  return w;
}

// f16(code * scale): the product rounded to binary32, then to binary16.
// The empty register constraint makes the rounded product a value of its
// own; without it the compiler fuses the multiply and the narrowing into one
// v_fma_mixlo_f16, which rounds the exact product once and differs from the
// two roundings by an ulp when the binary32 product falls on a binary16 tie.
// For the scales the encoder produces (max|x|/127 of an fp16 block) the two
// agree for every fp16 maximum and every code (checked exhaustively); for
// arbitrary scales about 1 value in 20,000 differs.
__device__ __forceinline__ uint32_t qwz_decode(uint32_t code8, float scale) {
  float p = static_cast<float>(static_cast<int8_t>(static_cast<uint8_t>(code8))) * scale;
  asm("" : "+v"(p));
  return f2h(p);
}

// Standalone encoder and decoder: 8 values per lane (16-byte fp16 and
// 8-byte code accesses), so one 256-value block is a half wave and the block
// maximum a reduction over 32 lanes.
constexpr int kQwzLane = 8;
constexpr int kQwzHalf = kQwzBlock / kQwzLane;  // lanes per block
constexpr int kQwzRow = kWave * kQwzLane;       // values per wave row: 2 blocks
static_assert(kQwzHalf == kWave / 2, "a block is half a wave");

// Maximum over each half wave of non-negative values, on their bit patterns
// (which order like the values): within each row of 16 lanes by four DPP
// steps (swap neighbours, swap pairs, mirror halves of 8, mirror the row),
// then across the two rows of the half wave with v_permlane16_swap.  No LDS
// traffic, unlike the ds_bpermute that shuffles compile to (measured on the
// 375M shard, with the branch-free quotients above: 0.173-0.175 ms against
// 0.176-0.189 ms with shuffles).  Every lane of the wave must be active.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max_step(uint32_t u) {
  const uint32_t o = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(u), CTRL, 0xF, 0xF, false));
  return u > o ? u : o;
}
__device__ __forceinline__ float half_wave_max(float a) {
  uint32_t u = __float_as_uint(a);
  u = dpp_max_step<0xB1>(u);   // quad_perm [1,0,3,2]
  u = dpp_max_step<0x4E>(u);   // quad_perm [2,3,0,1]
  u = dpp_max_step<0x141>(u);  // row_half_mirror
  u = dpp_max_step<0x140>(u);  // row_mirror
  const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(p[0] > p[1] ? p[0] : p[1]);
}

__device__ __forceinline__ float qwz_scale8(const float (&x)[kQwzLane]) {
  float a = 0.0f;
#pragma unroll
  for (int e = 0; e < kQwzLane; ++e) a = __builtin_fmaxf(a, __builtin_fabsf(x[e]));
  return half_wave_max(a) / 127.0f;
}

__device__ __forceinline__ u32x2 qwz_pack8(const float (&x)[kQwzLane], float scale) {
  if (scale == 0.0f) return u32x2{0u, 0u};
  float q[kQwzLane];
  qwz_quotients(x, scale, q);
  uint32_t lo = 0u, hi = 0u;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    lo |= qwz_byte(q[e]) << (8 * e);
    hi |= qwz_byte(q[e + 4]) << (8 * e);
  }
  return u32x2{lo, hi};
}

// fp16 [len] -> codes [len], scales [ceil(len/256)]; U rows of 2 blocks per
// wave, one tile per block.
template <int U>
__global__ __launch_bounds__(kWave) void qwz_quantize_kernel(const uint16_t *__restrict__ x16, int64_t len,
                                                             uint8_t *__restrict__ codes,
                                                             float *__restrict__ scales) {
  constexpr int kRow = kQwzRow;
  constexpr int64_t kTile = static_cast<int64_t>(kRow) * U;
  const int64_t ntiles = (len + kTile - 1) / kTile;
  const uint32_t lane = threadIdx.x * kQwzLane;
  const bool leader = (threadIdx.x & (kQwzHalf - 1)) == 0;
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t tbase = tile * kTile;
    if (tbase + kTile <= len) {
      u32x4 raw[U];
#pragma unroll
      for (int k = 0; k < U; ++k) raw[k] = stream_load(reinterpret_cast<const u32x4 *>(x16 + tbase + lane + k * kRow));
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const float x[kQwzLane] = {h2f(raw[k].x & 0xFFFFu), h2f(raw[k].x >> 16), h2f(raw[k].y & 0xFFFFu),
                                   h2f(raw[k].y >> 16),    h2f(raw[k].z & 0xFFFFu), h2f(raw[k].z >> 16),
                                   h2f(raw[k].w & 0xFFFFu), h2f(raw[k].w >> 16)};
        const float scale = qwz_scale8(x);
        stream_store(reinterpret_cast<u32x2 *>(codes + tbase + lane + k * kRow), qwz_pack8(x, scale));
        if (leader) scales[(tbase + lane + k * kRow) / kQwzBlock] = scale;
      }
    } else {
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const int64_t j0 = tbase + lane + k * kRow;
        float x[kQwzLane];
#pragma unroll
        for (int e = 0; e < kQwzLane; ++e) x[e] = j0 + e < len ? h2f(x16[j0 + e]) : 0.0f;
        const float scale = qwz_scale8(x);
        const u32x2 w = qwz_pack8(x, scale);
#pragma unroll
        for (int e = 0; e < kQwzLane; ++e)
          if (j0 + e < len) codes[j0 + e] = static_cast<uint8_t>((e < 4 ? w.x : w.y) >> (8 * (e & 3)));
        if (leader && j0 < len) scales[j0 / kQwzBlock] = scale;
      }
    }
  }
}

// Receiver side of the quantized all-gather: the N owners' code and scale
// buffers are decoded into the flat fp16 replica; block (x, y) decodes tile
// x of shard y (and every gridDim.x-th tile after it, when the shard has more
// tiles than one launch may have blocks), only the part of the shard below
// psi.
struct QwzTable {
  const uint8_t *codes[ZERO_MAX_SLICES];
  const float *scales[ZERO_MAX_SLICES];
};

template <int U>
__global__ __launch_bounds__(kWave) void qwz_allgather_kernel(QwzTable tab, int64_t shard_len, int64_t psi,
                                                              uint16_t *__restrict__ replica) {
  constexpr int kRow = kQwzRow;
  constexpr int64_t kTile = static_cast<int64_t>(kRow) * U;
  const int r = blockIdx.y;
  const int64_t first = static_cast<int64_t>(r) * shard_len;
  const int64_t real = psi - first < shard_len ? psi - first : shard_len;
  const uint32_t lane = threadIdx.x * kQwzLane;
  for (int64_t tbase = static_cast<int64_t>(blockIdx.x) * kTile; tbase < real;
       tbase += static_cast<int64_t>(gridDim.x) * kTile) {
    const uint8_t *src = tab.codes[r] + tbase;
    const float *sc = tab.scales[r] + tbase / kQwzBlock;
    uint16_t *dst = replica + first + tbase;
    if (tbase + kTile <= real) {
      u32x2 w[U];
      float scale[U];
#pragma unroll
      for (int k = 0; k < U; ++k) {
        w[k] = stream_load(reinterpret_cast<const u32x2 *>(src + lane + k * kRow));
        scale[k] = sc[(lane + k * kRow) / kQwzBlock];
      }
#pragma unroll
      for (int k = 0; k < U; ++k) {
        u32x4 h;
        h.x = qwz_decode(w[k].x, scale[k]) | (qwz_decode(w[k].x >> 8, scale[k]) << 16);
        h.y = qwz_decode(w[k].x >> 16, scale[k]) | (qwz_decode(w[k].x >> 24, scale[k]) << 16);
        h.z = qwz_decode(w[k].y, scale[k]) | (qwz_decode(w[k].y >> 8, scale[k]) << 16);
        h.w = qwz_decode(w[k].y >> 16, scale[k]) | (qwz_decode(w[k].y >> 24, scale[k]) << 16);
        stream_store(reinterpret_cast<u32x4 *>(dst + lane + k * kRow), h);
      }
    } else {
      const int64_t rem = real - tbase;
      for (int64_t j = threadIdx.x; j < rem; j += kWave)
        dst[j] = static_cast<uint16_t>(qwz_decode(src[j], sc[j / kQwzBlock]));
    }
  }
}

// ---------------------------------------------------------------- the update
// Fused single pass over the shard: read g, m, v, master; write m, v, master
// and the fp16 copy (28 B per parameter with an fp16 gradient, 30 B with
// fp32).  With QWZ the fresh fp16 values are also encoded (codes and
// per-block scales, 1 + 4/256 B more per parameter) while still in
// registers.  Every block first reads the device-resident overflow flag and
// leaves before any memory access to the states if it is set.  Launched with
// one block (one wave) per tile of kUpdateBlock*4*U elements.
// With DEV_T the two bias corrections are read from the device-resident
// step counter, where begin_step_kernel stored them for this step (the
// host's values in c are ignored).
template <zero_dtype_t DT, int U, bool QWZ = false, bool DEV_T = false>
__global__ __launch_bounds__(kUpdateBlock) void adam_update_kernel(
    const void *__restrict__ grad, float *__restrict__ master, float *__restrict__ m,
    float *__restrict__ v, uint16_t *__restrict__ p16, int64_t len, StepScalars c,
    const zero_grad_stats_t *__restrict__ stats, uint8_t *__restrict__ codes = nullptr,
    float *__restrict__ scales = nullptr, const zero_step_counter_t *__restrict__ counter = nullptr) {
  static_assert(!QWZ || kUpdateBlock * kChunk == kQwzBlock, "one chunk row per qwZ block");
  if (stats->overflow != 0u) return;
  if constexpr (DEV_T) {
    c.bc1 = counter->bias_correction1;
    c.bc2 = counter->bias_correction2;
  }
  constexpr int kSpan = kUpdateBlock * kChunk;  // elements of one chunk row of the block
  constexpr int64_t kTile = static_cast<int64_t>(kSpan) * U;
  const int64_t ntiles = (len + kTile - 1) / kTile;
  const uint32_t lane = threadIdx.x * kChunk;  // see the note in the reduce kernel
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t tbase = tile * kTile;
    if (tbase + kTile <= len) {
      const float *tm = m + tbase, *tv = v + tbase, *tt0 = master + tbase;
      const auto wm = store_window(m + tbase, kTile * 4), wv = store_window(v + tbase, kTile * 4);
      const auto wt = store_window(master + tbase, kTile * 4), wp = store_window(p16 + tbase, kTile * 2);
      float x[U][kChunk];
      f32x4 mm[U], vv[U], tt[U];
      uint32_t qq[U];  // qwZ: this lane's 4 codes of row k
      float qs[U];     // qwZ: the scale of row k's block
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const uint32_t j = lane + k * kSpan;
        if constexpr (DT == ZERO_F16) {
          const u32x2 raw =
              stream_load(reinterpret_cast<const u32x2 *>(static_cast<const uint16_t *>(grad) + tbase + j));
          x[k][0] = h2f(raw.x & 0xFFFFu);
          x[k][1] = h2f(raw.x >> 16);
          x[k][2] = h2f(raw.y & 0xFFFFu);
          x[k][3] = h2f(raw.y >> 16);
        } else {
          const f32x4 raw = stream_load(reinterpret_cast<const f32x4 *>(static_cast<const float *>(grad) + tbase + j));
          x[k][0] = raw.x;
          x[k][1] = raw.y;
          x[k][2] = raw.z;
          x[k][3] = raw.w;
        }
        mm[k] = stream_load(reinterpret_cast<const f32x4 *>(tm + j));
        vv[k] = stream_load(reinterpret_cast<const f32x4 *>(tv + j));
        tt[k] = stream_load(reinterpret_cast<const f32x4 *>(tt0 + j));
      }
      // formed after the loads are issued, so that with clipping its double
      // square root and divide overlap their latency (measured: 1.548 ms
      // with them ahead of the loads, 1.525 ms here, the same as unclipped)
      const float s = step_scale(c, stats);
#pragma unroll
      for (int k = 0; k < U; ++k) {
        float ma[kChunk] = {mm[k].x, mm[k].y, mm[k].z, mm[k].w};
        float va[kChunk] = {vv[k].x, vv[k].y, vv[k].z, vv[k].w};
        float ta[kChunk] = {tt[k].x, tt[k].y, tt[k].z, tt[k].w};
        uint32_t h[kChunk];
#pragma unroll
        for (int e = 0; e < kChunk; ++e) adam_element(x[k][e], ma[e], va[e], ta[e], h[e], c, s);
        const uint32_t j = lane + k * kSpan;
        window_store(wm, j * 4, f32x4{ma[0], ma[1], ma[2], ma[3]});
        window_store(wv, j * 4, f32x4{va[0], va[1], va[2], va[3]});
        window_store(wt, j * 4, f32x4{ta[0], ta[1], ta[2], ta[3]});
        window_store(wp, j * 2, u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)});
        if constexpr (QWZ) {
          const float w[kChunk] = {h2f(h[0]), h2f(h[1]), h2f(h[2]), h2f(h[3])};
          qs[k] = qwz_scale(w);
          qq[k] = qwz_pack(w, qs[k]);
        }
      }
      if constexpr (QWZ) {
        // The tile's U*256 codes are contiguous; lane l stores 4*U of them
        // with one access: the words of lanes U*(l % (64/U)) + i of row
        // l / (64/U), gathered with shuffles (with U = 1, its own word).
        // One store per lane beat one 4-byte store per row and lane when U
        // was 2.
        constexpr int kLanesPerRow = kWave / U;
        const int l = static_cast<int>(threadIdx.x);
        const int row = l / kLanesPerRow, src = U * (l % kLanesPerRow);
        uint32_t word[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {
          word[i] = 0u;
#pragma unroll
          for (int k = 0; k < U; ++k) {
            const uint32_t x = __shfl(qq[k], src + i, kWave);
            word[i] = row == k ? x : word[i];
          }
        }
        const auto wc = store_window(codes + tbase, kTile);
        if constexpr (U == 1) {
          window_store(wc, 4 * l, word[0]);
        } else if constexpr (U == 2) {
          window_store(wc, 8 * l, u32x2{word[0], word[1]});
        } else {
#pragma unroll
          for (int i = 0; i < U; ++i) window_store(wc, 4 * (U * l + i), word[i]);
        }
        if (l < U) {
          float sc = qs[0];
#pragma unroll
          for (int k = 1; k < U; ++k) sc = l == k ? qs[k] : sc;
          scales[tbase / kQwzBlock + l] = sc;
        }
      }
    } else {
      const float s = step_scale(c, stats);
      // the ragged last tile, element by element
#pragma unroll
      for (int k = 0; k < U; ++k) {
        float w[kChunk];
#pragma unroll
        for (int e = 0; e < kChunk; ++e) {
          const int64_t j = tbase + lane + k * kSpan + e;
          w[e] = 0.0f;
          if (j < len) {
            float x;
            if constexpr (DT == ZERO_F16)
              x = h2f(static_cast<const uint16_t *>(grad)[j]);
            else
              x = static_cast<const float *>(grad)[j];
            float mj = m[j], vj = v[j], tj = master[j];
            uint32_t h;
            adam_element(x, mj, vj, tj, h, c, s);
            m[j] = mj;
            v[j] = vj;
            master[j] = tj;
            p16[j] = static_cast<uint16_t>(h);
            w[e] = h2f(h);
          }
        }
        if constexpr (QWZ) {
          // every lane of the wave takes part in the block maximum
          const float scale = qwz_scale(w);
          const uint32_t q = qwz_pack(w, scale);
          const int64_t j0 = tbase + lane + k * kSpan;
#pragma unroll
          for (int e = 0; e < kChunk; ++e)
            if (j0 + e < len) codes[j0 + e] = static_cast<uint8_t>(q >> (8 * e));
          if (threadIdx.x == 0 && tbase + k * kSpan < len) scales[(tbase + k * kSpan) / kQwzBlock] = scale;
        }
      }
    }
  }
}

// Opens a step numbered on the device: t = applied + 1, the two bias
// corrections for t stored into the counter for the update to read, and the
// step counted (applied = t) unless the statistics flag it as skipped.  One
// thread, launched after the statistics and before the update on the same
// stream; the update reads only the bias corrections, so counting here
// rather than after it changes nothing.
__global__ void begin_step_kernel(const zero_grad_stats_t *__restrict__ stats, zero_step_counter_t *__restrict__ counter,
                                  double beta1, double beta2) {
  if (threadIdx.x != 0) return;
  const int64_t t = counter->applied + 1;
  counter->bias_correction1 = bias_correction(beta1, t);
  counter->bias_correction2 = bias_correction(beta2, t);
  if (stats->overflow == 0u) counter->applied = t;
}

}  // namespace zs
