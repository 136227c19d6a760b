// zero_shard.hip -- host side of the C ABI declared in include/zero_shard.h:
// argument validation, the per-step scalars, launch configuration.
//
// Sources: "DeepSpeed ZeRO Stages" (sections 2, 2.1, 3.1-3.3), "ZeRO Stage 1
// Math" ("The core idea", "Where the 12 bytes come from", "The per-step
// mechanics"), "ZeRO Optimization: Stages 1, 2, and 3 Explained" (Stage 2,
// mixed precision), "DeepSpeed ZeRO: Extreme Memory Efficiency" (three
// stages, communication, the optimizer configuration).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "shard_kernels.hpp"
#include "zero_shard.h"

namespace {

// Launch shape.  Update and reduce: U chunks of 4 elements per lane per
// tile, one block per tile.  Statistics: U 16-byte accesses per lane per
// tile, grid capped at kBlocksPerCU blocks per CU.
constexpr int kUpdateU = 1;      // plain update
constexpr int kUpdateQwzU = 1;   // with the qwZ encoder
constexpr int kStatsU = 8;
constexpr int kReduceU = 2;
constexpr int kReduceG = 4;
constexpr int64_t kReduceTile = static_cast<int64_t>(zs::kReduceBlock) * zs::kReduceLane * kReduceU;
constexpr int kBlocksPerCU = 4;
// Resident blocks per CU of the streaming kernels (see shard_kernels.hpp).
constexpr int kUpdateBlocksPerCU = 12;
constexpr int kUpdateQwzBlocksPerCU = 16;
constexpr int kReduceBlocksPerCU = 6;
// qwZ encoder and decoder: wave rows (512 values) per tile.
constexpr int kQwzEncU = 4;
constexpr int kQwzDecU = 1;
// Bytes at the start of the gradient that the statistics read (last) with
// the default cache policy, so that the update finds them in the Infinity
// Cache (256 MB on MI355X).  Measured on the 375M shard (fp16 gradient,
// 750 MB), with the bytes at the end kept and read forward: statistics +
// update 1.638 ms with 256 MB, 1.660 ms with none, 1.641 with 192 MB,
// 1.638-1.640 with 288-384 MB, 1.659 with the whole gradient.  Read from the
// end with the first 256 MB kept, the step took 1.673-1.675 ms against
// 1.677-1.687 ms forward on a slower box (192 MB: 1.680-1.683, 320 MB:
// 1.672-1.674, none: 1.700-1.703).
constexpr int64_t kStatsKeepBytes = int64_t{256} << 20;
// Bytes at the end of the reduce's fp32 sum written with sc1 instead of nt,
// for the same reason.  Measured on the 7.5B / N = 64 shard (469 MB sum):
// update 0.512-0.514 ms against 0.529-0.530 ms, and the reduce itself
// 15 us faster (two runs); 128 and 384 MB gained less.
constexpr int64_t kReduceKeepBytes = int64_t{256} << 20;

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
  return ZERO_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [a, a+na) and [b, b+nb) share a byte.
bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  if (na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Compute units of the current device, cached per device.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_cache[kMaxDevices];

int cu_count(int *out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ZERO_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev >= 0 && dev < kMaxDevices) {
    const int cached = g_cu_cache[dev].load(std::memory_order_relaxed);
    if (cached > 0) {
      *out = cached;
      return ZERO_OK;
    }
  }
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess || cus <= 0)
    return fail(ZERO_ERR_HIP, "hipDeviceGetAttribute(CU count): %s", hipGetErrorString(e));
  if (dev >= 0 && dev < kMaxDevices) g_cu_cache[dev].store(cus, std::memory_order_relaxed);
  *out = cus;
  return ZERO_OK;
}

int64_t ceil_div(int64_t a, int64_t b) { return a / b + (a % b != 0 ? 1 : 0); }

// Most blocks of `block` threads one launch may have along x: HIP takes the
// grid's size in work-items as a 32-bit count.  The kernels that could need
// more tiles than this walk the rest with a grid-stride loop.
constexpr int64_t max_grid_x(int block) { return static_cast<int64_t>(UINT32_MAX) / block; }

// Dynamic LDS bytes per block that leave room for exactly `target` resident
// blocks of `kernel` on a CU (0 when the kernel's own resources already allow
// no more than that, or when no size gives exactly `target`).  Found once per
// device and kernel with the occupancy API and cached.
enum CapKernel {
  kCapUpdateF16,
  kCapUpdateF32,
  kCapUpdateQwzF16,
  kCapUpdateQwzF32,
  kCapUpdateF16T,
  kCapUpdateF32T,
  kCapUpdateQwzF16T,
  kCapUpdateQwzF32T,
  kCapReduceStats,
  kCapReduce,
  kCapKinds
};
std::atomic<int> g_lds_cache[kMaxDevices][kCapKinds];
std::atomic<bool> g_lds_init{false};

template <typename K>
int occupancy_cap_lds(CapKernel which, K kernel, int block, int target, size_t *lds_out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ZERO_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (!g_lds_init.load(std::memory_order_acquire)) {
    for (auto &row : g_lds_cache)
      for (auto &x : row) x.store(-1, std::memory_order_relaxed);
    g_lds_init.store(true, std::memory_order_release);
  }
  if (dev >= 0 && dev < kMaxDevices) {
    const int cached = g_lds_cache[dev][which].load(std::memory_order_relaxed);
    if (cached >= 0) {
      *lds_out = static_cast<size_t>(cached);
      return ZERO_OK;
    }
  }
  int lds_cu = 0, lds_block = 0, occ = 0;
  e = hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&lds_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, block, 0);
  if (e != hipSuccess) return fail(ZERO_ERR_HIP, "occupancy query: %s", hipGetErrorString(e));
  int chosen = 0;
  if (occ > target && lds_cu > 0) {
    // start at an even share of the CU's LDS and step down until exactly
    // `target` blocks fit
    int lds = (lds_cu / target) & ~127;
    if (lds > lds_block) lds = lds_block & ~127;
    for (int i = 0; i < 64 && lds >= 128; ++i, lds -= 128) {
      int o = 0;
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, kernel, block, static_cast<size_t>(lds));
      if (e != hipSuccess) return fail(ZERO_ERR_HIP, "occupancy query: %s", hipGetErrorString(e));
      if (o == target) {
        chosen = lds;
        break;
      }
      if (o > target) break;
    }
  }
  if (dev >= 0 && dev < kMaxDevices) g_lds_cache[dev][which].store(chosen, std::memory_order_relaxed);
  *lds_out = static_cast<size_t>(chosen);
  return ZERO_OK;
}

int grid_for(int64_t len, int64_t tile, int cus, int cap) {
  const int64_t tiles = ceil_div(len, tile);
  int64_t g = static_cast<int64_t>(cus) * kBlocksPerCU;
  if (g > cap) g = cap;
  if (g > tiles) g = tiles;
  return static_cast<int>(g < 1 ? 1 : g);
}

// An error recorded by an earlier, unrelated HIP call on this thread (the
// runtime keeps the last one) is dropped before a launch, so that the check
// after it reports only what the launch itself did.
void clear_stale_error() { (void)hipGetLastError(); }

int check_launch(const char *what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ZERO_ERR_HIP, "%s launch: %s", what, hipGetErrorString(e));
  return ZERO_OK;
}

bool scale_valid(double s) { return std::isfinite(s) && s > 0.0; }

// Partials of the reduce: one per tile (at least one, for len = 0), then the
// first-level folds of kFold partials each.
int64_t reduce_partials(int64_t len) {
  const int64_t t = ceil_div(len, kReduceTile);
  return t < 1 ? 1 : t;
}
int64_t fold_blocks(int64_t nparts) { return ceil_div(nparts, zs::kFold); }

// Folds `nparts` per-block partials in `ws` into `stats`, in a fixed order:
// directly when they fit one block's pass, else through one fold level.
int finalize(zs::Partial *parts, int64_t nparts, zero_grad_stats_t *stats, hipStream_t stream) {
  if (nparts <= zs::kFold) {
    zs::finalize_stats_kernel<<<1, zs::kBlock, 0, stream>>>(parts, static_cast<int>(nparts), stats);
    return check_launch("finalize_stats_kernel");
  }
  const int64_t nfold = fold_blocks(nparts);
  zs::Partial *folded = parts + nparts;
  zs::fold_partials_kernel<<<static_cast<unsigned>(nfold), zs::kBlock, 0, stream>>>(parts, nparts, folded);
  const int st = check_launch("fold_partials_kernel");
  if (st != ZERO_OK) return st;
  zs::finalize_stats_kernel<<<1, zs::kBlock, 0, stream>>>(folded, static_cast<int>(nfold), stats);
  return check_launch("finalize_stats_kernel");
}

// Statistics of `grad` into `stats` through the partials in `ws`.
int launch_stats(const void *grad, zero_dtype_t dt, int64_t len, float s, zero_grad_stats_t *stats,
                 void *ws, hipStream_t stream) {
  int cus = 0;
  int st = cu_count(&cus);
  if (st != ZERO_OK) return st;
  const int64_t tile = static_cast<int64_t>(zs::kBlock) * kStatsU *
                       (dt == ZERO_F16 ? zs::stats_per_lane<ZERO_F16>() : zs::stats_per_lane<ZERO_F32>());
  const int grid = grid_for(len, tile, cus, zs::kMaxPartials);
  zs::Partial *parts = static_cast<zs::Partial *>(ws);
  const int64_t keep = kStatsKeepBytes / (dt == ZERO_F16 ? 2 : 4);
  const int64_t keep_below = len < keep ? len : keep;
  clear_stale_error();
  if (dt == ZERO_F16)
    zs::grad_stats_kernel<ZERO_F16, kStatsU><<<grid, zs::kBlock, 0, stream>>>(grad, len, s, parts, keep_below);
  else
    zs::grad_stats_kernel<ZERO_F32, kStatsU><<<grid, zs::kBlock, 0, stream>>>(grad, len, s, parts, keep_below);
  st = check_launch("grad_stats_kernel");
  if (st != ZERO_OK) return st;
  return finalize(parts, grid, stats, stream);
}

}  // namespace

extern "C" {

int zero_partition_layout(int64_t psi, int32_t n_ranks, int32_t rank, int64_t align,
                          zero_layout_t *out) {
  if (out == nullptr) return fail(ZERO_ERR_INVALID_ARG, "layout: out is NULL");
  if (psi < 0) return fail(ZERO_ERR_INVALID_ARG, "layout: psi < 0");
  if (n_ranks < 1) return fail(ZERO_ERR_INVALID_ARG, "layout: n_ranks < 1");
  if (rank < 0 || rank >= n_ranks) return fail(ZERO_ERR_INVALID_ARG, "layout: rank out of range");
  if (align < 1 || (align & (align - 1)) != 0)
    return fail(ZERO_ERR_INVALID_ARG, "layout: align must be a positive power of two");
  // the flat space is cut into rows of n_ranks*align elements; each rank
  // takes `align` elements of every row, as one contiguous block
  if (align > INT64_MAX / n_ranks) return fail(ZERO_ERR_INT_OVERFLOW, "layout: n_ranks*align overflows");
  const int64_t row = align * n_ranks;
  const int64_t rows = ceil_div(psi, row);
  if (rows > INT64_MAX / row) return fail(ZERO_ERR_INT_OVERFLOW, "layout: padded size overflows");
  const int64_t shard = rows * align;
  const int64_t first = shard * rank;
  out->psi = psi;
  out->psi_padded = rows * row;
  out->shard_len = shard;
  out->offset = first;
  out->real_len = psi <= first ? 0 : (psi - first < shard ? psi - first : shard);
  return ok();
}

int zero_model_state_bytes(double psi, int32_t n_ranks, int32_t stage, double K, double *out_bytes) {
  if (out_bytes == nullptr) return fail(ZERO_ERR_INVALID_ARG, "model_state_bytes: out is NULL");
  if (!(psi >= 0.0) || n_ranks < 1 || !(K >= 0.0) || stage < 0 || stage > 3)
    return fail(ZERO_ERR_INVALID_ARG, "model_state_bytes: bad argument");
  // bytes per parameter: fp16 compute copy 2, fp16 gradient 2, optimizer K;
  // each stage divides one more of them by N (P_os, P_os+g, P_os+g+p)
  const double n = n_ranks;
  const double param = stage >= 3 ? 2.0 / n : 2.0;
  const double grad = stage >= 2 ? 2.0 / n : 2.0;
  const double opt = stage >= 1 ? K / n : K;
  *out_bytes = (param + grad + opt) * psi;
  return ok();
}

size_t zero_workspace_bytes(int64_t len) {
  if (len < 0) return 0;
  // the larger of the statistics kernel's partials and the reduce's (one per
  // tile of kReduceTile elements plus their first fold level)
  const int64_t red = reduce_partials(len) + fold_blocks(reduce_partials(len));
  const int64_t n = red > zs::kMaxPartials ? red : zs::kMaxPartials;
  return static_cast<size_t>(n) * sizeof(zs::Partial);
}

int zero_shard_grad_stats(const void *grad, int32_t grad_dtype, int64_t len, double inv_grad_scale,
                          zero_grad_stats_t *stats, void *ws, size_t ws_bytes, hipStream_t stream) {
  if (len < 0) return fail(ZERO_ERR_INVALID_ARG, "grad_stats: len < 0");
  if (grad_dtype != ZERO_F16 && grad_dtype != ZERO_F32)
    return fail(ZERO_ERR_INVALID_ARG, "grad_stats: unknown grad dtype");
  if ((grad == nullptr && len > 0) || stats == nullptr || ws == nullptr)
    return fail(ZERO_ERR_INVALID_ARG, "grad_stats: NULL pointer");
  if (!scale_valid(inv_grad_scale))
    return fail(ZERO_ERR_INVALID_ARG, "grad_stats: inv_grad_scale must be finite and > 0");
  if (!aligned16(grad) || !aligned16(stats) || !aligned16(ws))
    return fail(ZERO_ERR_MISALIGNED, "grad_stats: device pointers must be 16-byte aligned");
  if (ws_bytes < zero_workspace_bytes(len)) return fail(ZERO_ERR_WORKSPACE, "grad_stats: workspace too small");
  const size_t gbytes = static_cast<size_t>(len) * (grad_dtype == ZERO_F16 ? 2 : 4);
  if (overlap(grad, gbytes, stats, sizeof(zero_grad_stats_t)) || overlap(grad, gbytes, ws, ws_bytes) ||
      overlap(stats, sizeof(zero_grad_stats_t), ws, ws_bytes))
    return fail(ZERO_ERR_INVALID_ARG, "grad_stats: grad, stats and workspace must not overlap");
  const int st = launch_stats(grad, grad_dtype == ZERO_F16 ? ZERO_F16 : ZERO_F32, len,
                              static_cast<float>(inv_grad_scale), stats, ws, stream);
  return st == ZERO_OK ? ok() : st;
}

int zero_shard_grad_reduce(const uint16_t *const *slices, int32_t n_slices, int64_t len, float *out_sum,
                           zero_grad_stats_t *stats, double inv_grad_scale, void *ws, size_t ws_bytes,
                           hipStream_t stream) {
  if (n_slices < 1 || n_slices > ZERO_MAX_SLICES)
    return fail(ZERO_ERR_INVALID_ARG, "grad_reduce: n_slices must be in [1, %d]", ZERO_MAX_SLICES);
  if (len < 0) return fail(ZERO_ERR_INVALID_ARG, "grad_reduce: len < 0");
  if (slices == nullptr || (out_sum == nullptr && len > 0))
    return fail(ZERO_ERR_INVALID_ARG, "grad_reduce: NULL pointer");
  if (!scale_valid(inv_grad_scale))
    return fail(ZERO_ERR_INVALID_ARG, "grad_reduce: inv_grad_scale must be finite and > 0");
  if (len > INT64_MAX / 4) return fail(ZERO_ERR_INT_OVERFLOW, "grad_reduce: len too large");
  zs::SliceTable tab{};
  for (int r = 0; r < n_slices; ++r) {
    if (slices[r] == nullptr && len > 0) return fail(ZERO_ERR_INVALID_ARG, "grad_reduce: slice %d is NULL", r);
    if (!aligned16(slices[r])) return fail(ZERO_ERR_MISALIGNED, "grad_reduce: slice %d misaligned", r);
    if (overlap(slices[r], static_cast<size_t>(len) * 2, out_sum, static_cast<size_t>(len) * 4))
      return fail(ZERO_ERR_INVALID_ARG, "grad_reduce: out_sum overlaps slice %d", r);
    tab.p[r] = slices[r];
  }
  if (!aligned16(out_sum)) return fail(ZERO_ERR_MISALIGNED, "grad_reduce: out_sum misaligned");
  if (stats != nullptr) {
    if (ws == nullptr) return fail(ZERO_ERR_INVALID_ARG, "grad_reduce: workspace is NULL");
    if (!aligned16(stats) || !aligned16(ws))
      return fail(ZERO_ERR_MISALIGNED, "grad_reduce: stats/workspace misaligned");
    if (ws_bytes < zero_workspace_bytes(len)) return fail(ZERO_ERR_WORKSPACE, "grad_reduce: workspace too small");
    // the statistics and the workspace are written: they may share no byte
    // with each other, the sum or a slice
    const size_t sb = sizeof(zero_grad_stats_t), ob = static_cast<size_t>(len) * 4;
    if (overlap(stats, sb, ws, ws_bytes) || overlap(stats, sb, out_sum, ob) || overlap(ws, ws_bytes, out_sum, ob))
      return fail(ZERO_ERR_INVALID_ARG, "grad_reduce: stats, workspace and out_sum must not overlap");
    for (int r = 0; r < n_slices; ++r)
      if (overlap(slices[r], static_cast<size_t>(len) * 2, stats, sb) ||
          overlap(slices[r], static_cast<size_t>(len) * 2, ws, ws_bytes))
        return fail(ZERO_ERR_INVALID_ARG, "grad_reduce: stats or workspace overlaps slice %d", r);
  }
  // one block per tile (each writes its own partial); beyond the launch
  // limit the blocks take several tiles each
  const int64_t tiles = reduce_partials(len);
  const int64_t nparts = tiles < max_grid_x(zs::kReduceBlock) ? tiles : max_grid_x(zs::kReduceBlock);
  const unsigned grid = static_cast<unsigned>(nparts);
  const float s = static_cast<float>(inv_grad_scale);
  int st;
  size_t lds = 0;
  const int64_t keep = kReduceKeepBytes / 4;
  const int64_t keep_from = len > keep ? len - keep : 0;
  if (stats != nullptr) {
    st = occupancy_cap_lds(kCapReduceStats, zs::grad_reduce_kernel<true, kReduceU, kReduceG>, zs::kReduceBlock,
                           kReduceBlocksPerCU, &lds);
    if (st != ZERO_OK) return st;
    zs::Partial *parts = static_cast<zs::Partial *>(ws);
    clear_stale_error();
    zs::grad_reduce_kernel<true, kReduceU, kReduceG><<<grid, zs::kReduceBlock, lds, stream>>>(
        tab, n_slices, len, out_sum, s, parts, keep_from);
    st = check_launch("grad_reduce_kernel");
    if (st != ZERO_OK) return st;
    st = finalize(parts, nparts, stats, stream);
    if (st != ZERO_OK) return st;
  } else if (len > 0) {
    st = occupancy_cap_lds(kCapReduce, zs::grad_reduce_kernel<false, kReduceU, kReduceG>, zs::kReduceBlock,
                           kReduceBlocksPerCU, &lds);
    if (st != ZERO_OK) return st;
    clear_stale_error();
    zs::grad_reduce_kernel<false, kReduceU, kReduceG><<<grid, zs::kReduceBlock, lds, stream>>>(
        tab, n_slices, len, out_sum, s, nullptr, keep_from);
    st = check_launch("grad_reduce_kernel");
    if (st != ZERO_OK) return st;
  }
  return ok();
}

int zero_shard_allgather(const uint16_t *const *shards, int32_t n_ranks, int64_t shard_len, int64_t psi,
                         uint16_t *replica, hipStream_t stream) {
  if (n_ranks < 1 || n_ranks > ZERO_MAX_SLICES)
    return fail(ZERO_ERR_INVALID_ARG, "allgather: n_ranks must be in [1, %d]", ZERO_MAX_SLICES);
  if (shard_len < 0 || shard_len % 8 != 0)
    return fail(ZERO_ERR_INVALID_ARG, "allgather: shard_len must be a non-negative multiple of 8");
  if (shard_len > INT64_MAX / ZERO_MAX_SLICES / 2) return fail(ZERO_ERR_INT_OVERFLOW, "allgather: shard_len too large");
  if (psi < 0 || psi > shard_len * n_ranks) return fail(ZERO_ERR_INVALID_ARG, "allgather: psi out of range");
  if (shards == nullptr || (replica == nullptr && psi > 0)) return fail(ZERO_ERR_INVALID_ARG, "allgather: NULL pointer");
  if (!aligned16(replica)) return fail(ZERO_ERR_MISALIGNED, "allgather: replica misaligned");
  zs::SliceTable tab{};
  for (int r = 0; r < n_ranks; ++r) {
    const int64_t first = static_cast<int64_t>(r) * shard_len;
    const int64_t real = psi - first < shard_len ? (psi - first > 0 ? psi - first : 0) : shard_len;
    if (shards[r] == nullptr && real > 0) return fail(ZERO_ERR_INVALID_ARG, "allgather: shard %d is NULL", r);
    if (!aligned16(shards[r])) return fail(ZERO_ERR_MISALIGNED, "allgather: shard %d misaligned", r);
    if (overlap(shards[r], static_cast<size_t>(shard_len) * 2, replica, static_cast<size_t>(psi) * 2))
      return fail(ZERO_ERR_INVALID_ARG, "allgather: replica overlaps shard %d", r);
    tab.p[r] = shards[r];
  }
  if (psi == 0 || shard_len == 0) return ok();
  const int64_t tiles = ceil_div(shard_len, zs::kGatherTile);
  const int64_t gx = tiles < max_grid_x(zs::kGatherBlock) ? tiles : max_grid_x(zs::kGatherBlock);
  clear_stale_error();
  zs::allgather_kernel<<<dim3(static_cast<unsigned>(gx), static_cast<unsigned>(n_ranks)), zs::kGatherBlock, 0,
                         stream>>>(tab, shard_len, psi, replica);
  const int st = check_launch("allgather_kernel");
  return st == ZERO_OK ? ok() : st;
}

}  // extern "C"

namespace {

int64_t qwz_scales_len(int64_t len) { return ceil_div(len, zs::kQwzBlock); }

// ------------------------------------------------------------------ scratch
// The per-block partials of the statistics for zero_shard_adam_step_noalloc,
// in the library's own device memory: one copy of this array per device,
// held until the process ends.  The statistics kernel writes at most
// kMaxPartials of them (its grid is capped there whatever the length), and
// every partial the finalize reads is written earlier in the same call, so
// nothing in it has to start at zero.  Host code never passes `scratch`
// itself to a kernel (on the host that name is only a stand-in): it passes
// the device address hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = sizeof(zs::Partial) * zs::kMaxPartials;
static __device__ __align__(256) zs::Partial scratch[zs::kMaxPartials];
static_assert(sizeof(scratch) == kScratchBytes && kScratchBytes == ZERO_NOALLOC_SCRATCH_BYTES,
              "scratch holds the statistics' partials");

std::atomic<void *> g_scratch[kMaxDevices];

// The current device's address of `scratch`, looked up on the first call on
// that device and kept.
int scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ZERO_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(ZERO_ERR_HIP, "device %d: the static scratch is kept for devices 0..%d only", dev, kMaxDevices - 1);
  void *p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(ZERO_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return ZERO_OK;
}

// Capped-occupancy launch of one instantiation of the update kernel, one
// block per tile.  Measured on the 375M shard: the plain update is fastest
// with 1 chunk per lane at 12 blocks per CU (1.546 ms; 2 chunks at 8 blocks:
// 1.607 ms), the update with the qwZ encoder with 1 chunk at 16 blocks
// (1.655 ms; 2 chunks at 8 or 10 blocks: 1.696 and 1.672 ms).
template <zero_dtype_t DT, bool QWZ, bool DEV_T>
int launch_update(CapKernel cap, const void *grad, float *master, float *m, float *v, uint16_t *p16, int64_t len,
                  const zs::StepScalars &c, const zero_grad_stats_t *stats, uint8_t *codes, float *scales,
                  const zero_step_counter_t *counter, hipStream_t stream) {
  constexpr int U = QWZ ? kUpdateQwzU : kUpdateU;
  constexpr int cap_blocks = QWZ ? kUpdateQwzBlocksPerCU : kUpdateBlocksPerCU;
  constexpr int64_t tile = static_cast<int64_t>(zs::kUpdateBlock) * zs::kChunk * U;
  const int64_t tiles = ceil_div(len, tile);
  const unsigned grid = static_cast<unsigned>(tiles < max_grid_x(zs::kUpdateBlock) ? tiles : max_grid_x(zs::kUpdateBlock));
  size_t lds = 0;
  const int st = occupancy_cap_lds(cap, zs::adam_update_kernel<DT, U, QWZ, DEV_T>, zs::kUpdateBlock, cap_blocks, &lds);
  if (st != ZERO_OK) return st;
  clear_stale_error();
  zs::adam_update_kernel<DT, U, QWZ, DEV_T><<<grid, zs::kUpdateBlock, lds, stream>>>(
      grad, master, m, v, p16, len, c, stats, codes, scales, counter);
  return check_launch("adam_update_kernel");
}

// The update, with the qwZ encoding of its fp16 output into codes and
// scales when qwz is set, and with the step number read from (and counted
// into) the device-resident counter when applied != NULL.
// With use_scratch the statistics' partials go to the library's static
// scratch instead of a caller's workspace (ws and ws_bytes are then ignored);
// its address is looked up after every argument has been validated.
int adam_step_impl(const void *grad, int32_t grad_dtype_in, double inv_grad_scale, float *master,
                   float *exp_avg, float *exp_avg_sq, uint16_t *param16, bool qwz, int8_t *codes, float *scales,
                   int64_t len, int64_t step, zero_step_counter_t *applied, const zero_adam_hparams_t *hp,
                   zero_grad_stats_t *stats, int32_t stats_precomputed, void *ws, size_t ws_bytes,
                   bool use_scratch, hipStream_t stream) {
  if (use_scratch) {
    ws = nullptr;
    ws_bytes = 0;
  }
  const bool dev_t = applied != nullptr;
  if (len < 0) return fail(ZERO_ERR_INVALID_ARG, "adam_step: len < 0");
  if (grad_dtype_in != ZERO_F16 && grad_dtype_in != ZERO_F32)
    return fail(ZERO_ERR_INVALID_ARG, "adam_step: unknown grad dtype");
  const zero_dtype_t grad_dtype = grad_dtype_in == ZERO_F16 ? ZERO_F16 : ZERO_F32;
  if (hp == nullptr || stats == nullptr) return fail(ZERO_ERR_INVALID_ARG, "adam_step: NULL hp or stats");
  if (len > 0 && (grad == nullptr || master == nullptr || exp_avg == nullptr || exp_avg_sq == nullptr ||
                  param16 == nullptr))
    return fail(ZERO_ERR_INVALID_ARG, "adam_step: NULL array");
  if (!dev_t && step < 1) return fail(ZERO_ERR_INVALID_ARG, "adam_step: step must be >= 1");
  if (!aligned16(applied)) return fail(ZERO_ERR_MISALIGNED, "adam_step: step counter misaligned");
  if (!(std::isfinite(hp->lr) && hp->lr >= 0.0)) return fail(ZERO_ERR_INVALID_ARG, "adam_step: bad lr");
  if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0) || !(hp->beta2 >= 0.0 && hp->beta2 < 1.0))
    return fail(ZERO_ERR_INVALID_ARG, "adam_step: betas must be in [0, 1)");
  if (!(std::isfinite(hp->eps) && hp->eps > 0.0)) return fail(ZERO_ERR_INVALID_ARG, "adam_step: eps must be > 0");
  if (!scale_valid(inv_grad_scale))
    return fail(ZERO_ERR_INVALID_ARG, "adam_step: inv_grad_scale must be finite and > 0");
  if (!(std::isfinite(hp->max_grad_norm) && hp->max_grad_norm >= 0.0))
    return fail(ZERO_ERR_INVALID_ARG, "adam_step: max_grad_norm must be finite and >= 0");
  if (len > INT64_MAX / 4) return fail(ZERO_ERR_INT_OVERFLOW, "adam_step: len too large");
  if (qwz && len > 0 && (codes == nullptr || scales == nullptr))
    return fail(ZERO_ERR_INVALID_ARG, "adam_step: NULL qwZ codes or scales");
  if (!aligned16(grad) || !aligned16(master) || !aligned16(exp_avg) || !aligned16(exp_avg_sq) ||
      !aligned16(param16) || !aligned16(stats) || !aligned16(codes) || !aligned16(scales))
    return fail(ZERO_ERR_MISALIGNED, "adam_step: device pointers must be 16-byte aligned");
  if (!stats_precomputed && !use_scratch) {
    if (ws == nullptr) return fail(ZERO_ERR_INVALID_ARG, "adam_step: workspace is NULL");
    if (!aligned16(ws)) return fail(ZERO_ERR_MISALIGNED, "adam_step: workspace misaligned");
    if (ws_bytes < zero_workspace_bytes(len))
      return fail(ZERO_ERR_WORKSPACE, "adam_step: workspace of %zu bytes, %zu needed", ws_bytes,
                  zero_workspace_bytes(len));
  }
  const size_t n = static_cast<size_t>(len);
  const size_t gbytes = n * (grad_dtype == ZERO_F16 ? 2 : 4);
  // the arrays, the qwZ outputs, the step counter, the statistics and the
  // workspace (the last three when present): no two may share a byte
  constexpr int kArgs = 10;
  const void *arr[kArgs] = {grad, master, exp_avg, exp_avg_sq, param16, codes, scales, applied, stats, ws};
  const size_t sz[kArgs] = {gbytes, n * 4, n * 4, n * 4, n * 2, qwz ? n : 0,
                            qwz ? static_cast<size_t>(qwz_scales_len(len)) * 4 : 0,
                            dev_t ? sizeof(zero_step_counter_t) : 0u, sizeof(zero_grad_stats_t),
                            stats_precomputed ? 0u : ws_bytes};
  static const char *const names[kArgs] = {"grad", "master", "exp_avg", "exp_avg_sq", "param16",
                                           "qwZ codes", "qwZ scales", "step counter", "stats", "workspace"};
  for (int a = 0; a < kArgs; ++a)
    for (int b = a + 1; b < kArgs; ++b)
      if (overlap(arr[a], sz[a], arr[b], sz[b]))
        return fail(ZERO_ERR_INVALID_ARG, "adam_step: %s overlaps %s", names[a], names[b]);

  // Per-step scalars: each is evaluated in double and rounded once to float.
  zs::StepScalars c;
  c.b1 = static_cast<float>(hp->beta1);
  c.omb1 = static_cast<float>(1.0 - hp->beta1);
  c.b2 = static_cast<float>(hp->beta2);
  c.omb2 = static_cast<float>(1.0 - hp->beta2);
  // with a device-resident step number begin_step_kernel forms these
  c.bc1 = dev_t ? 1.0f : static_cast<float>(1.0 - std::pow(hp->beta1, static_cast<double>(step)));
  c.bc2 = dev_t ? 1.0f : static_cast<float>(1.0 - std::pow(hp->beta2, static_cast<double>(step)));
  c.lr = static_cast<float>(hp->lr);
  c.eps = static_cast<float>(hp->eps);
  c.s = static_cast<float>(inv_grad_scale);
  c.inv_scale = inv_grad_scale;
  c.max_norm = hp->max_grad_norm;

  int st;
  if (!stats_precomputed) {
    if (use_scratch) {
      // the statistics write one partial per block, at most kMaxPartials
      // whatever the length: exactly what the scratch holds
      st = scratch_address(&ws);
      if (st != ZERO_OK) return st;
    }
    st = launch_stats(grad, grad_dtype, len, c.s, stats, ws, stream);
    if (st != ZERO_OK) return st;
  }
  if (dev_t) {
    // opens the step (bias corrections for t, counted unless skipped), also
    // when len == 0
    clear_stale_error();
    zs::begin_step_kernel<<<1, zs::kWave, 0, stream>>>(stats, applied, hp->beta1, hp->beta2);
    st = check_launch("begin_step_kernel");
    if (st != ZERO_OK) return st;
  }
  if (len > 0) {
    uint8_t *c8 = reinterpret_cast<uint8_t *>(codes);
    const bool f16 = grad_dtype == ZERO_F16;
    const int key = (f16 ? 0 : 1) | (qwz ? 2 : 0) | (dev_t ? 4 : 0);
    switch (key) {
      case 0: st = launch_update<ZERO_F16, false, false>(kCapUpdateF16, grad, master, exp_avg, exp_avg_sq, param16, len, c, stats, nullptr, nullptr, nullptr, stream); break;
      case 1: st = launch_update<ZERO_F32, false, false>(kCapUpdateF32, grad, master, exp_avg, exp_avg_sq, param16, len, c, stats, nullptr, nullptr, nullptr, stream); break;
      case 2: st = launch_update<ZERO_F16, true, false>(kCapUpdateQwzF16, grad, master, exp_avg, exp_avg_sq, param16, len, c, stats, c8, scales, nullptr, stream); break;
      case 3: st = launch_update<ZERO_F32, true, false>(kCapUpdateQwzF32, grad, master, exp_avg, exp_avg_sq, param16, len, c, stats, c8, scales, nullptr, stream); break;
      case 4: st = launch_update<ZERO_F16, false, true>(kCapUpdateF16T, grad, master, exp_avg, exp_avg_sq, param16, len, c, stats, nullptr, nullptr, applied, stream); break;
      case 5: st = launch_update<ZERO_F32, false, true>(kCapUpdateF32T, grad, master, exp_avg, exp_avg_sq, param16, len, c, stats, nullptr, nullptr, applied, stream); break;
      case 6: st = launch_update<ZERO_F16, true, true>(kCapUpdateQwzF16T, grad, master, exp_avg, exp_avg_sq, param16, len, c, stats, c8, scales, applied, stream); break;
      default: st = launch_update<ZERO_F32, true, true>(kCapUpdateQwzF32T, grad, master, exp_avg, exp_avg_sq, param16, len, c, stats, c8, scales, applied, stream); break;
    }
    if (st != ZERO_OK) return st;
  }
  return ok();
}

}  // namespace

extern "C" {

int zero_shard_adam_step(const void *grad, int32_t grad_dtype, double inv_grad_scale, float *master,
                         float *exp_avg, float *exp_avg_sq, uint16_t *param16, int64_t len, int64_t step,
                         const zero_adam_hparams_t *hp, zero_grad_stats_t *stats, int32_t stats_precomputed,
                         void *ws, size_t ws_bytes, hipStream_t stream) {
  return adam_step_impl(grad, grad_dtype, inv_grad_scale, master, exp_avg, exp_avg_sq, param16, false, nullptr,
                        nullptr, len, step, nullptr, hp, stats, stats_precomputed, ws, ws_bytes, false,
                        stream);
}

int zero_shard_adam_step_qwz(const void *grad, int32_t grad_dtype, double inv_grad_scale, float *master,
                             float *exp_avg, float *exp_avg_sq, uint16_t *param16, int8_t *codes, float *scales,
                             int64_t len, int64_t step, const zero_adam_hparams_t *hp, zero_grad_stats_t *stats,
                             int32_t stats_precomputed, void *ws, size_t ws_bytes, hipStream_t stream) {
  return adam_step_impl(grad, grad_dtype, inv_grad_scale, master, exp_avg, exp_avg_sq, param16, true, codes, scales,
                        len, step, nullptr, hp, stats, stats_precomputed, ws, ws_bytes, false,
                        stream);
}

int zero_shard_adam_step_device_t(const void *grad, int32_t grad_dtype, double inv_grad_scale, float *master,
                                  float *exp_avg, float *exp_avg_sq, uint16_t *param16, int8_t *codes,
                                  float *scales, int64_t len, zero_step_counter_t *applied_steps,
                                  const zero_adam_hparams_t *hp, zero_grad_stats_t *stats,
                                  int32_t stats_precomputed, void *ws, size_t ws_bytes, hipStream_t stream) {
  if (applied_steps == nullptr) return fail(ZERO_ERR_INVALID_ARG, "adam_step_device_t: NULL step counter");
  if ((codes == nullptr) != (scales == nullptr))
    return fail(ZERO_ERR_INVALID_ARG, "adam_step_device_t: qwZ codes and scales go together");
  const bool qwz = codes != nullptr;
  return adam_step_impl(grad, grad_dtype, inv_grad_scale, master, exp_avg, exp_avg_sq, param16, qwz, codes, scales,
                        len, 1, applied_steps, hp, stats, stats_precomputed, ws, ws_bytes, false,
                        stream);
}

int zero_shard_adam_step_noalloc(const void *grad, int32_t grad_dtype, double inv_grad_scale, float *master,
                                 float *exp_avg, float *exp_avg_sq, uint16_t *param16, int64_t len, int64_t step,
                                 const zero_adam_hparams_t *hp, zero_grad_stats_t *stats,
                                 int32_t stats_precomputed, hipStream_t stream) {
  return adam_step_impl(grad, grad_dtype, inv_grad_scale, master, exp_avg, exp_avg_sq, param16, false, nullptr,
                        nullptr, len, step, nullptr, hp, stats, stats_precomputed, nullptr, 0, true, stream);
}

int zero_qwz_quantize(const uint16_t *x16, int64_t len, int8_t *codes, float *scales, hipStream_t stream) {
  if (len < 0) return fail(ZERO_ERR_INVALID_ARG, "qwz_quantize: len < 0");
  if (len > INT64_MAX / 4) return fail(ZERO_ERR_INT_OVERFLOW, "qwz_quantize: len too large");
  if (len > 0 && (x16 == nullptr || codes == nullptr || scales == nullptr))
    return fail(ZERO_ERR_INVALID_ARG, "qwz_quantize: NULL pointer");
  if (!aligned16(x16) || !aligned16(codes) || !aligned16(scales))
    return fail(ZERO_ERR_MISALIGNED, "qwz_quantize: device pointers must be 16-byte aligned");
  const size_t n = static_cast<size_t>(len), ns = static_cast<size_t>(qwz_scales_len(len)) * 4;
  if (overlap(x16, n * 2, codes, n) || overlap(x16, n * 2, scales, ns) || overlap(codes, n, scales, ns))
    return fail(ZERO_ERR_INVALID_ARG, "qwz_quantize: arrays overlap");
  if (len == 0) return ok();
  constexpr int64_t tile = static_cast<int64_t>(zs::kQwzRow) * kQwzEncU;
  const int64_t tiles = ceil_div(len, tile);
  const unsigned grid = static_cast<unsigned>(tiles < max_grid_x(zs::kWave) ? tiles : max_grid_x(zs::kWave));
  clear_stale_error();
  zs::qwz_quantize_kernel<kQwzEncU><<<grid, zs::kWave, 0, stream>>>(x16, len, reinterpret_cast<uint8_t *>(codes),
                                                                 scales);
  const int st = check_launch("qwz_quantize_kernel");
  return st == ZERO_OK ? ok() : st;
}

int zero_qwz_allgather(const int8_t *const *codes, const float *const *scales, int32_t n_ranks, int64_t shard_len,
                       int64_t psi, uint16_t *replica, hipStream_t stream) {
  if (n_ranks < 1 || n_ranks > ZERO_MAX_SLICES)
    return fail(ZERO_ERR_INVALID_ARG, "qwz_allgather: n_ranks must be in [1, %d]", ZERO_MAX_SLICES);
  if (shard_len < 0 || shard_len % 8 != 0)
    return fail(ZERO_ERR_INVALID_ARG, "qwz_allgather: shard_len must be a non-negative multiple of 8");
  if (shard_len > INT64_MAX / ZERO_MAX_SLICES / 2)
    return fail(ZERO_ERR_INT_OVERFLOW, "qwz_allgather: shard_len too large");
  if (psi < 0 || psi > shard_len * n_ranks) return fail(ZERO_ERR_INVALID_ARG, "qwz_allgather: psi out of range");
  if (codes == nullptr || scales == nullptr || (replica == nullptr && psi > 0))
    return fail(ZERO_ERR_INVALID_ARG, "qwz_allgather: NULL pointer");
  if (!aligned16(replica)) return fail(ZERO_ERR_MISALIGNED, "qwz_allgather: replica misaligned");
  const size_t ns = static_cast<size_t>(qwz_scales_len(shard_len)) * 4;
  zs::QwzTable tab{};
  for (int r = 0; r < n_ranks; ++r) {
    const int64_t first = static_cast<int64_t>(r) * shard_len;
    const int64_t real = psi - first < shard_len ? (psi - first > 0 ? psi - first : 0) : shard_len;
    if ((codes[r] == nullptr || scales[r] == nullptr) && real > 0)
      return fail(ZERO_ERR_INVALID_ARG, "qwz_allgather: shard %d is NULL", r);
    if (!aligned16(codes[r]) || !aligned16(scales[r]))
      return fail(ZERO_ERR_MISALIGNED, "qwz_allgather: shard %d misaligned", r);
    if (overlap(codes[r], static_cast<size_t>(shard_len), replica, static_cast<size_t>(psi) * 2) ||
        overlap(scales[r], ns, replica, static_cast<size_t>(psi) * 2))
      return fail(ZERO_ERR_INVALID_ARG, "qwz_allgather: replica overlaps shard %d", r);
    tab.codes[r] = reinterpret_cast<const uint8_t *>(codes[r]);
    tab.scales[r] = scales[r];
  }
  if (psi == 0 || shard_len == 0) return ok();
  constexpr int64_t tile = static_cast<int64_t>(zs::kQwzRow) * kQwzDecU;
  const int64_t tiles = ceil_div(shard_len, tile);
  const int64_t gx = tiles < max_grid_x(zs::kWave) ? tiles : max_grid_x(zs::kWave);
  clear_stale_error();
  zs::qwz_allgather_kernel<kQwzDecU><<<dim3(static_cast<unsigned>(gx), static_cast<unsigned>(n_ranks)), zs::kWave, 0,
                                    stream>>>(tab, shard_len, psi, replica);
  const int st = check_launch("qwz_allgather_kernel");
  return st == ZERO_OK ? ok() : st;
}

const char *zero_status_string(int status) {
  switch (status) {
    case ZERO_OK: return "ok";
    case ZERO_ERR_INVALID_ARG: return "invalid argument";
    case ZERO_ERR_MISALIGNED: return "device pointer not 16-byte aligned";
    case ZERO_ERR_WORKSPACE: return "workspace missing or too small";
    case ZERO_ERR_HIP: return "HIP runtime error";
    case ZERO_ERR_INT_OVERFLOW: return "size overflows 64 bits";
    default: return "unknown status";
  }
}

const char *zero_last_error(void) { return g_err; }

int zero_shard_abi_version(void) { return ZERO_SHARD_ABI_VERSION; }

}  // extern "C"
