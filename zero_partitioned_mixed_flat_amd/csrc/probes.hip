// probes.hip -- device probes of the optimizer library's own code (its
// arithmetic helpers and its streaming-store policy); see
// zero_probes.h.  Used by the tests and the benchmark only.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#include "shard_kernels.hpp"
#include "zero_probes.h"

namespace {

constexpr int kProbeBlock = 256;
constexpr int kRmwBlock = 64;

// The library's arithmetic primitives, built with the library's flags:
// binary32 division and square root, the binary32 -> binary16 conversion
// of the fp16 write-back and the binary16 -> binary32 decode.
__global__ void arith_kernel(const float *a, const float *b, const uint16_t *h, int64_t n, float *quot, float *root,
                             uint16_t *half, float *wide) {
  for (int64_t j = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; j < n;
       j += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    quot[j] = a[j] / b[j];
    root[j] = __builtin_sqrtf(a[j]);
    half[j] = static_cast<uint16_t>(zs::f2h(a[j]));
    wide[j] = zs::h2f(h[j]);
  }
}

// The library's device-side bias correction 1 - beta^t for given t.
__global__ void bias_correction_kernel(double beta, const int64_t *t, int64_t n, float *out) {
  for (int64_t j = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; j < n;
       j += static_cast<int64_t>(gridDim.x) * blockDim.x)
    out[j] = zs::bias_correction(beta, t[j]);
}

// In-place read-modify-write of whole 16-byte chunks (x += 1), the access
// type of the optimizer's state streams: non-temporal loads, and stores
// through a buffer window with the library's streaming-store policy.
__global__ __launch_bounds__(kRmwBlock) void rmw_f32_kernel(float *__restrict__ p, int64_t n4) {
  const int64_t base = blockIdx.x * static_cast<int64_t>(kRmwBlock);
  if (base >= n4) return;
  const int64_t i = base + threadIdx.x;
  const auto w = zs::store_window(p + 4 * base, kRmwBlock * 16);
  if (i < n4) {
    zs::f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const zs::f32x4 *>(p) + i);
    x += 1.0f;
    zs::window_store(w, threadIdx.x * 16, x);
  }
}

int grid_for(int64_t n) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c > 0) cus = c;
  }
  const int64_t need = (n + kProbeBlock - 1) / kProbeBlock;
  const int64_t cap = static_cast<int64_t>(cus) * 8;
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

int zero_probes_arith_f32(const float *a, const float *b, const uint16_t *h, int64_t n, float *quot, float *root,
                          uint16_t *half, float *wide, hipStream_t stream_) {
  if (n < 0) return -1;
  if (n > 0 && (a == nullptr || b == nullptr || h == nullptr || quot == nullptr || root == nullptr ||
                half == nullptr || wide == nullptr))
    return -1;
  if (n == 0) return 0;
  clear_stale_error();
  arith_kernel<<<grid_for(n), kProbeBlock, 0, stream_>>>(a, b, h, n, quot, root, half, wide);
  return launched();
}

int zero_probes_bias_correction(double beta, const int64_t *t, int64_t n, float *out, hipStream_t stream_) {
  if (n < 0 || (n > 0 && (t == nullptr || out == nullptr))) return -1;
  if (n == 0) return 0;
  clear_stale_error();
  bias_correction_kernel<<<grid_for(n), kProbeBlock, 0, stream_>>>(beta, t, n, out);
  return launched();
}

int zero_probes_rmw_f32(float *p, int64_t n, hipStream_t stream_) {
  if (n < 0 || (n > 0 && p == nullptr)) return -1;
  if (reinterpret_cast<uintptr_t>(p) & 15u) return -1;
  const int64_t n4 = n / 4;
  const int64_t blocks = (n4 + kRmwBlock - 1) / kRmwBlock;
  if (blocks > INT32_MAX) return -1;
  if (blocks == 0) return 0;
  clear_stale_error();
  rmw_f32_kernel<<<static_cast<unsigned>(blocks), kRmwBlock, 0, stream_>>>(p, n4);
  return launched();
}

const char *zero_probes_last_error(void) { return g_err; }

}  // extern "C"
