// testkit.hip -- seeded synthetic inputs (Philox4x32-10 + Box-Muller) and
// plain streaming reference kernels; see zero_testkit.h.  Nothing
// here is, or includes, code of the optimizer library.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>

#include "zero_testkit.h"

namespace {

constexpr int kBlock = 256;

struct U4 {
  uint32_t x, y, z, w;
};

// Philox4x32-10 (Salmon et al., SC'11): ten rounds of two 32x32->64-bit
// multiplies with the Weyl key schedule.
__device__ __forceinline__ U4 philox(U4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * c.x;
    const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * c.z;
    const uint32_t hi0 = static_cast<uint32_t>(p0 >> 32), lo0 = static_cast<uint32_t>(p0);
    const uint32_t hi1 = static_cast<uint32_t>(p1 >> 32), lo1 = static_cast<uint32_t>(p1);
    c = U4{hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0};
  }
  return c;
}

__device__ __forceinline__ U4 draw(uint64_t seed, uint32_t stream, int64_t j, uint32_t d) {
  const uint64_t uj = static_cast<uint64_t>(j);
  return philox(U4{static_cast<uint32_t>(uj), static_cast<uint32_t>(uj >> 32), stream, d},
                static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
}

__device__ __forceinline__ double unit53(uint32_t a, uint32_t b) {
  return (static_cast<double>(a >> 5) * 67108864.0 + static_cast<double>(b >> 6) + 0.5) *
         1.1102230246251565404e-16;  // 2^-53
}

// Both Box-Muller normals of one Philox block.
__device__ __forceinline__ void normals(U4 w, double &z0, double &z1) {
  const double u1 = unit53(w.x, w.y), u2 = unit53(w.z, w.w);
  const double r = sqrt(-2.0 * log(u1));
  const double a = 6.283185307179586476925 * u2;
  z0 = r * cos(a);
  z1 = r * sin(a);
}

__device__ __forceinline__ uint16_t to_half_bits(double x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(static_cast<float>(x)));
}

__global__ void philox_kernel(uint32_t *out, int64_t n, uint64_t seed, uint32_t stream) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(kBlock) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kBlock) {
    const U4 w = draw(seed, stream, i, 0u);
    out[4 * i + 0] = w.x;
    out[4 * i + 1] = w.y;
    out[4 * i + 2] = w.z;
    out[4 * i + 3] = w.w;
  }
}

__global__ void normal_f32_kernel(float *out, int64_t n, double mean, double std, int abs_value,
                                  uint64_t seed, uint32_t stream) {
  for (int64_t j = blockIdx.x * static_cast<int64_t>(kBlock) + threadIdx.x; j < n;
       j += static_cast<int64_t>(gridDim.x) * kBlock) {
    double z0, z1;
    normals(draw(seed, stream, j, 0u), z0, z1);
    double x = mean + std * z0;
    if (abs_value) x = fabs(x);
    out[j] = static_cast<float>(x);
  }
}

__global__ void normal_f16_kernel(uint16_t *out, int64_t n, double scale, uint64_t seed, uint32_t stream) {
  for (int64_t j = blockIdx.x * static_cast<int64_t>(kBlock) + threadIdx.x; j < n;
       j += static_cast<int64_t>(gridDim.x) * kBlock) {
    double z0, z1;
    normals(draw(seed, stream, j, 0u), z0, z1);
    out[j] = to_half_bits(scale * z0);
  }
}

__global__ void student_t3_f16_kernel(uint16_t *out, int64_t n, double scale, int redraw, uint64_t seed,
                                      uint32_t stream) {
  for (int64_t j = blockIdx.x * static_cast<int64_t>(kBlock) + threadIdx.x; j < n;
       j += static_cast<int64_t>(gridDim.x) * kBlock) {
    uint16_t h = 0;
    const int attempts = redraw ? 8 : 1;
    for (int a = 0; a < attempts; ++a) {
      double z0, z1, z2, z3;
      normals(draw(seed, stream, j, 2u * a), z0, z1);
      normals(draw(seed, stream, j, 2u * a + 1u), z2, z3);
      const double t = z0 / sqrt((z1 * z1 + z2 * z2 + z3 * z3) / 3.0);
      h = to_half_bits(scale * t);
      if ((h & 0x7C00u) != 0x7C00u) break;
      if (redraw && a == attempts - 1) h = static_cast<uint16_t>((h & 0x8000u) | 0x7BFFu);
    }
    out[j] = h;
  }
}

__global__ void inject_inf_kernel(uint16_t *out, int64_t n, double prob, uint64_t seed, uint32_t stream) {
  for (int64_t j = blockIdx.x * static_cast<int64_t>(kBlock) + threadIdx.x; j < n;
       j += static_cast<int64_t>(gridDim.x) * kBlock) {
    const U4 w = draw(seed, stream, j, 0u);
    if (unit53(w.x, w.y) < prob) out[j] = 0x7C00u;
  }
}

// Reference streaming kernels in the shapes that measured fastest on MI355X:
// copy = one 16-byte non-temporal load and store per lane, 64-lane blocks,
// one block per 256 floats; read = four 16-byte non-temporal loads per lane
// per iteration over a grid of four blocks per CU.  (The read-modify-write
// reference, which uses the library's store policy, is in probes.hip.)
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kCopyBlock = 64;

__global__ __launch_bounds__(kCopyBlock) void copy_f32_kernel(const f32x4 *__restrict__ src, f32x4 *__restrict__ dst,
                                                              int64_t n4, const float *__restrict__ src_tail,
                                                              float *__restrict__ dst_tail, int tail) {
  const int64_t i = blockIdx.x * static_cast<int64_t>(kCopyBlock) + threadIdx.x;
  if (i < n4) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
  if (blockIdx.x == 0 && static_cast<int>(threadIdx.x) < tail) dst_tail[threadIdx.x] = src_tail[threadIdx.x];
}

__global__ __launch_bounds__(kBlock) void read_f32_kernel(const f32x4 *__restrict__ src, int64_t n4,
                                                          float *__restrict__ sink, int sink_len) {
  constexpr int U = 4;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock * U;
  float acc = 0.f;
  for (int64_t base = blockIdx.x * static_cast<int64_t>(kBlock) * U; base < n4; base += stride) {
    f32x4 x[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int64_t i = base + k * kBlock + threadIdx.x;
      x[k] = i < n4 ? __builtin_nontemporal_load(src + i) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int k = 0; k < U; ++k) acc += x[k].x + x[k].y + x[k].z + x[k].w;
  }
  __shared__ float s[kBlock];
  s[threadIdx.x] = acc;
  __syncthreads();
  for (int w = kBlock / 2; w > 0; w >>= 1) {
    if (static_cast<int>(threadIdx.x) < w) s[threadIdx.x] += s[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0 && static_cast<int>(blockIdx.x) < sink_len) sink[blockIdx.x] = s[0];
}

// Many-slice streaming reference: the shape of the optimizer library's
// owner-side reduce (tiles of 1024 elements per 128-thread block, two chunks
// of four elements per lane, four slices' loads in flight, six blocks per
// CU), with XOR in place of any arithmetic.
constexpr int kSlicesMax = 64;
struct Slices {
  const uint16_t *p[kSlicesMax];
};
constexpr int kSliceBlock = 128;
constexpr int kSliceSpan = kSliceBlock * 4;
constexpr int64_t kSliceTile = kSliceSpan * 2;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kSliceBlock) void read_slices_kernel(Slices tab, int n, int64_t len, uint32_t *out,
                                                                  uint32_t *sink, int sink_len) {
  const int64_t tbase = blockIdx.x * kSliceTile;
  const uint32_t lane = threadIdx.x * 4;
  uint32_t w[2][2] = {{0u, 0u}, {0u, 0u}};
  uint32_t tail = 0u;
  if (tbase + kSliceTile <= len) {
    for (int r0 = 0; r0 < n; r0 += 4) {
      u32x2 raw[4][2];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (r0 + q < n) {
#pragma unroll
          for (int k = 0; k < 2; ++k)
            raw[q][k] = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(tab.p[r0 + q] + tbase + lane + k * kSliceSpan));
        }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (r0 + q < n) {
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            w[k][0] ^= raw[q][k].x;
            w[k][1] ^= raw[q][k].y;
          }
        }
    }
    if (out != nullptr) {
#pragma unroll
      for (int k = 0; k < 2; ++k)
        __builtin_nontemporal_store(u32x4{w[k][0] & 0xFFFFu, w[k][0] >> 16, w[k][1] & 0xFFFFu, w[k][1] >> 16},
                                    reinterpret_cast<u32x4 *>(out + tbase + lane + k * kSliceSpan));
    }
  } else {
    for (int64_t j = tbase + threadIdx.x; j < len; j += kSliceBlock) {
      uint32_t x = 0u;
      for (int r = 0; r < n; ++r) x ^= tab.p[r][j];
      if (out != nullptr) out[j] = x;
      tail ^= x;
    }
  }
  uint32_t x = tail ^ (w[0][0] & 0xFFFFu) ^ (w[0][0] >> 16) ^ (w[0][1] & 0xFFFFu) ^ (w[0][1] >> 16) ^
               (w[1][0] & 0xFFFFu) ^ (w[1][0] >> 16) ^ (w[1][1] & 0xFFFFu) ^ (w[1][1] >> 16);
  __shared__ uint32_t s[kSliceBlock];
  s[threadIdx.x] = x;
  __syncthreads();
  for (int h = kSliceBlock / 2; h > 0; h >>= 1) {
    if (static_cast<int>(threadIdx.x) < h) s[threadIdx.x] ^= s[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0 && static_cast<int>(blockIdx.x) < sink_len) sink[blockIdx.x] = s[0];
}

int cu_count() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c > 0) cus = c;
  }
  return cus;
}

int grid_for(int64_t n) {
  const int64_t need = (n + kBlock - 1) / kBlock;
  const int64_t cap = static_cast<int64_t>(cu_count()) * 8;
  const int64_t g = need < cap ? need : cap;
  return static_cast<int>(g < 1 ? 1 : g);
}

thread_local char g_err[256] = "";

// Drops an error left by an earlier, unrelated HIP call on this thread.
void clear_stale_error() { (void)hipGetLastError(); }

int launched() {
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return 0;
  std::snprintf(g_err, sizeof g_err, "%s", hipGetErrorString(e));
  return -4;
}

}  // namespace

extern "C" {

int zero_testkit_philox(uint32_t *out, int64_t n_blocks, uint64_t seed, uint32_t stream, hipStream_t stream_) {
  if (n_blocks < 0 || (n_blocks > 0 && out == nullptr)) return -1;
  if (n_blocks == 0) return 0;
  clear_stale_error();
  philox_kernel<<<grid_for(n_blocks), kBlock, 0, stream_>>>(out, n_blocks, seed, stream);
  return launched();
}

int zero_testkit_normal_f32(float *out, int64_t n, double mean, double std, int32_t abs_value, uint64_t seed,
                            uint32_t stream, hipStream_t stream_) {
  if (n < 0 || (n > 0 && out == nullptr) || !std::isfinite(mean) || !std::isfinite(std)) return -1;
  if (n == 0) return 0;
  clear_stale_error();
  normal_f32_kernel<<<grid_for(n), kBlock, 0, stream_>>>(out, n, mean, std, abs_value, seed, stream);
  return launched();
}

int zero_testkit_normal_f16(uint16_t *out, int64_t n, double scale, uint64_t seed, uint32_t stream,
                            hipStream_t stream_) {
  if (n < 0 || (n > 0 && out == nullptr) || !std::isfinite(scale)) return -1;
  if (n == 0) return 0;
  clear_stale_error();
  normal_f16_kernel<<<grid_for(n), kBlock, 0, stream_>>>(out, n, scale, seed, stream);
  return launched();
}

int zero_testkit_student_t3_f16(uint16_t *out, int64_t n, double scale, int32_t redraw_overflow, uint64_t seed,
                                uint32_t stream, hipStream_t stream_) {
  if (n < 0 || (n > 0 && out == nullptr) || !std::isfinite(scale)) return -1;
  if (n == 0) return 0;
  clear_stale_error();
  student_t3_f16_kernel<<<grid_for(n), kBlock, 0, stream_>>>(out, n, scale, redraw_overflow, seed, stream);
  return launched();
}

int zero_testkit_inject_inf_f16(uint16_t *out, int64_t n, double prob, uint64_t seed, uint32_t stream,
                                hipStream_t stream_) {
  if (n < 0 || (n > 0 && out == nullptr) || !(prob >= 0.0 && prob <= 1.0)) return -1;
  if (n == 0) return 0;
  clear_stale_error();
  inject_inf_kernel<<<grid_for(n), kBlock, 0, stream_>>>(out, n, prob, seed, stream);
  return launched();
}

int zero_testkit_copy_f32(const float *src, float *dst, int64_t n, hipStream_t stream_) {
  if (n < 0 || (n > 0 && (src == nullptr || dst == nullptr))) return -1;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u) return -1;
  if (n == 0) return 0;
  const int64_t n4 = n / 4;
  const int tail = static_cast<int>(n - n4 * 4);
  const int64_t blocks = (n4 + kCopyBlock - 1) / kCopyBlock;
  if (blocks > INT32_MAX) return -1;
  clear_stale_error();
  copy_f32_kernel<<<static_cast<unsigned>(blocks < 1 ? 1 : blocks), kCopyBlock, 0, stream_>>>(
      reinterpret_cast<const f32x4 *>(src), reinterpret_cast<f32x4 *>(dst), n4, src + n4 * 4, dst + n4 * 4, tail);
  return launched();
}

int zero_testkit_read_f32(const float *src, int64_t n, float *sink, int32_t sink_len, hipStream_t stream_) {
  if (n < 0 || sink_len < 1 || sink == nullptr || (n > 0 && src == nullptr)) return -1;
  if (reinterpret_cast<uintptr_t>(src) & 15u) return -1;
  const int64_t n4 = n / 4;
  const int64_t need = (n4 + 4 * kBlock - 1) / (4 * kBlock);
  const int64_t cap = static_cast<int64_t>(cu_count()) * 4;
  const int grid = static_cast<int>(need < 1 ? 1 : (need < cap ? need : cap));
  clear_stale_error();
  read_f32_kernel<<<grid, kBlock, 0, stream_>>>(reinterpret_cast<const f32x4 *>(src), n4, sink, sink_len);
  return launched();
}

int zero_testkit_read_slices(const uint16_t *const *slices, int32_t n, int64_t len, uint32_t *out, uint32_t *sink,
                             int32_t sink_len, hipStream_t stream_) {
  if (slices == nullptr || n < 1 || n > kSlicesMax || len < 0 || len % 4 != 0 || sink == nullptr || sink_len < 1)
    return -1;
  if (reinterpret_cast<uintptr_t>(out) & 15u) return -1;
  Slices tab{};
  for (int r = 0; r < n; ++r) {
    if ((slices[r] == nullptr && len > 0) || (reinterpret_cast<uintptr_t>(slices[r]) & 15u)) return -1;
    tab.p[r] = slices[r];
  }
  const int64_t blocks = (len + kSliceTile - 1) / kSliceTile;
  if (blocks > static_cast<int64_t>(UINT32_MAX) / kSliceBlock) return -1;
  // six resident blocks per CU, as the reduce runs: an otherwise unused
  // dynamic LDS allocation leaves room for no more
  int dev = 0, lds_cu = 0, occ = 0;
  size_t lds = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) == hipSuccess &&
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, read_slices_kernel, kSliceBlock, 0) == hipSuccess &&
      occ > 6) {
    for (int b = (lds_cu / 6) & ~127; b >= 128; b -= 128) {
      int o = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, read_slices_kernel, kSliceBlock, b) != hipSuccess) break;
      if (o == 6) {
        lds = static_cast<size_t>(b);
        break;
      }
      if (o > 6) break;
    }
  }
  if (blocks == 0) return 0;
  clear_stale_error();
  read_slices_kernel<<<static_cast<unsigned>(blocks), kSliceBlock, lds, stream_>>>(tab, n, len, out, sink, sink_len);
  return launched();
}

const char *zero_testkit_last_error(void) { return g_err; }

}  // extern "C"
