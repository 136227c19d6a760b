/*
 * zero_shard.h -- C ABI of the per-rank ZeRO shard optimizer step on one
 * MI355X (gfx950): the partition of the flat parameter space, the owner-side
 * gradient reduce, the gradient statistics, the fused mixed-precision Adam
 * update of one rank's owned partition, the all-gather of the fp16 shards and
 * its block-INT8 (qwZ) variant.
 *
 * Sources, cited by page title and section:
 *   [ZS]  "DeepSpeed ZeRO Stages"
 *   [S1M] "ZeRO Stage 1 Math"
 *   [ZOS] "ZeRO Optimization: Stages 1, 2, and 3 Explained"
 *   [DZE] "DeepSpeed ZeRO: Extreme Memory Efficiency"
 *
 * Conventions for every entry point:
 *   - No exceptions cross the ABI; every call returns a zero_status_t (or a
 *     size / string as documented), and on failure zero_last_error() holds
 *     a message for the calling thread.  Arguments are validated before
 *     anything is enqueued, so a validation error enqueues nothing; a launch
 *     failure (ZERO_ERR_HIP) may leave earlier kernels of the same call
 *     enqueued.
 *   - Device pointers are HIP device allocations on the current device and
 *     must be 16-byte aligned (ZERO_ERR_MISALIGNED otherwise).  Every array
 *     is owned by the caller; the library never allocates or frees device
 *     memory and keeps no state between calls, apart from per-device caches
 *     of the CU count and of the launch-shape LDS sizes, and the fixed
 *     32 KiB scratch array of zero_shard_adam_step_noalloc (part of the
 *     library's code object, one copy per device).  The caches are filled
 *     by the first call of each kind on a device, with occupancy queries;
 *     make that first call outside HIP graph capture.  After it, every call
 *     enqueues kernels only (no memset, copy or allocation) and can be
 *     captured into a graph.
 *   - Arrays a call writes (outputs, the statistics, the workspace) must not
 *     share a byte with any other array of the same call
 *     (ZERO_ERR_INVALID_ARG otherwise).
 *   - Device work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream) and the call returns without synchronising; outputs, including
 *     the device-resident zero_grad_stats_t, are valid once the stream has
 *     passed that point.
 *   - Lengths are element counts.  A length of 0 is valid.
 *   - Floating point: binary32 arithmetic with round-to-nearest-even, no
 *     contraction, correctly rounded division and square root, subnormals
 *     kept; fp16 conversion is round-to-nearest-even.
 */
#ifndef ZERO_SHARD_H
#define ZERO_SHARD_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZERO_SHARD_ABI_VERSION 7
/* Largest number of simulated rank slices one reduce call accepts. */
#define ZERO_MAX_SLICES 64
/* Values per qwZ quantization block (one binary32 scale each). */
#define ZERO_QWZ_BLOCK 256

typedef enum {
  ZERO_OK = 0,
  ZERO_ERR_INVALID_ARG = -1,   /* a null pointer, a bad size or hyperparameter */
  ZERO_ERR_MISALIGNED = -2,    /* a device pointer not 16-byte aligned */
  ZERO_ERR_WORKSPACE = -3,     /* workspace missing or smaller than required */
  ZERO_ERR_HIP = -4,           /* a HIP runtime call or launch failed */
  ZERO_ERR_INT_OVERFLOW = -5   /* a size does not fit in 64 bits */
} zero_status_t;

/* Element type of a gradient argument.  Entry points take it as int32_t, so
 * that any value a C caller passes is well defined and rejected when it is
 * not one of these. */
typedef enum { ZERO_F16 = 1, ZERO_F32 = 2 } zero_dtype_t;

/* One rank's shard of the flat parameter index space [0, psi). */
typedef struct {
  int64_t psi;        /* total number of parameters */
  int64_t psi_padded; /* n_ranks * shard_len (>= psi) */
  int64_t shard_len;  /* elements every rank holds, a multiple of align */
  int64_t offset;     /* first flat index of this rank's shard = rank * shard_len */
  int64_t real_len;   /* elements of the shard below psi (the rest is padding) */
} zero_layout_t;

/* Adam hyperparameters, named as in the optimizer block of the DeepSpeed
 * configuration shown on [DZE] (lr, betas, eps).  No weight decay.
 * max_grad_norm: global-norm gradient clipping ([ZS] section 2.1: clipping
 * needs ||g||_2 over all of P, one scalar all-reduce).  When > 0 and the
 * norm sqrt(stats->sumsq) of the unscaled gradient exceeds it, the gradient
 * is multiplied by max_grad_norm / norm; the factor is folded into the
 * unscale multiplier, (float)(inv_grad_scale * factor) computed in double and
 * rounded once.  0 disables clipping (the multiplier is then exactly
 * (float)inv_grad_scale). */
typedef struct {
  double lr;
  double beta1;
  double beta2;
  double eps;
  double max_grad_norm;
} zero_adam_hparams_t;

/* Device-resident result of the gradient statistics. */
typedef struct {
  uint32_t overflow; /* 1 if any gradient element is +-inf or NaN, else 0 */
  uint32_t reserved; /* written as 0 */
  double sumsq;      /* sum over the shard of (f32(x_j) * inv_grad_scale)^2,
                        accumulated in fp64; unspecified when overflow = 1 */
} zero_grad_stats_t;

/* Device-resident step counter of zero_shard_adam_step_device_t (16 bytes,
 * 16-byte aligned).  The caller zeroes it before the first step. */
typedef struct {
  int64_t applied;          /* steps applied so far; read and advanced on the
                               device */
  float bias_correction1;   /* written by each call: (float)(1 - beta1^t) for
                               the t of that call */
  float bias_correction2;   /* the same for beta2 */
} zero_step_counter_t;

/*
 * zero_partition_layout -- the disjoint, padded shard of `rank`.
 * [ZS] section 2 defines the partition (disjoint index sets whose union is
 * every parameter, each of size about psi/N, owned exclusively by one rank);
 * [S1M] "The core idea" assigns shard i to rank i; [ZS] section 3.2 keeps the
 * gradients in one flat contiguous buffer.  Shards are equal contiguous
 * blocks in rank order: shard_len = ceil(psi / (n_ranks*align)) * align,
 * offset = rank*shard_len, real_len = clamp(psi - offset, 0, shard_len).
 * Host arithmetic only.  Errors: out NULL, psi < 0, n_ranks < 1, rank not in
 * [0, n_ranks), align < 1 or not a power of two -> ZERO_ERR_INVALID_ARG;
 * n_ranks*align or psi_padded above INT64_MAX -> ZERO_ERR_INT_OVERFLOW.
 */
int zero_partition_layout(int64_t psi, int32_t n_ranks, int32_t rank,
                          int64_t align, zero_layout_t *out);

/*
 * zero_model_state_bytes -- model-state bytes per GPU for ZeRO stage 0..3
 * (0 = plain data parallelism) with optimizer multiplier K (12 for
 * mixed-precision Adam): [ZS] section 1.2 and sections 3.1-3.3; [DZE] "Three
 * stages of partitioning".  Host arithmetic only.  Errors: out_bytes NULL,
 * psi < 0, n_ranks < 1, stage not in 0..3, K < 0 -> ZERO_ERR_INVALID_ARG.
 */
int zero_model_state_bytes(double psi, int32_t n_ranks, int32_t stage,
                           double K, double *out_bytes);

/*
 * zero_workspace_bytes -- bytes of device workspace that the statistics of a
 * shard of `len` elements need: per-block partial results, 16 bytes per
 * 1024 elements (about 0.8% of an fp16 gradient of that length) and never
 * less than 32 KiB.  The same buffer may be reused by consecutive calls on one stream;
 * calls that share it must not run concurrently.  Returns 0 for len < 0.
 */
size_t zero_workspace_bytes(int64_t len);

/*
 * zero_shard_grad_reduce -- owner-side arithmetic of the gradient
 * reduce-scatter ([ZS] sections 3.1-3.2: rank i receives the fully reduced
 * gradient of P_i, reduced into the owner's buffer; [DZE] communication
 * section: the reduce-scatter sums), for N simulated ranks whose fp16
 * gradient slices of this shard already sit in this GPU's memory.
 *   slices          host array of n_slices device pointers, slice r holding
 *                   `len` fp16 values (binary16 bit patterns) of rank r
 *   out_sum         device fp32 [len]: out[j] = left fold in fp32 of
 *                   f32(slice_0[j]) + f32(slice_1[j]) + ... in rank order
 *   stats           device zero_grad_stats_t or NULL; when given, the
 *                   overflow flag and sum of squares of (out[j] *
 *                   inv_grad_scale) are computed in the same pass, so that a
 *                   following zero_shard_adam_step can skip its own pass
 *                   (stats_precomputed = 1, same inv_grad_scale)
 *   inv_grad_scale  multiplier applied to out[j] for the statistics only
 *   ws, ws_bytes    device workspace of >= zero_workspace_bytes(len) bytes,
 *                   needed only when stats is not NULL
 * The sum is not averaged: a caller that wants the mean folds 1/N into
 * inv_grad_scale.  The last 256 MiB of out_sum are written so that they
 * stay in the Infinity Cache: an update of the same shard enqueued right
 * after this call reads them from there.  Errors: n_slices not in
 * [1, ZERO_MAX_SLICES], len < 0,
 * a NULL slice/out pointer (len > 0), inv_grad_scale not finite or <= 0,
 * out_sum overlapping a slice -> ZERO_ERR_INVALID_ARG; misaligned pointer ->
 * ZERO_ERR_MISALIGNED; short workspace -> ZERO_ERR_WORKSPACE.
 */
int zero_shard_grad_reduce(const uint16_t *const *slices, int32_t n_slices,
                           int64_t len, float *out_sum,
                           zero_grad_stats_t *stats, double inv_grad_scale,
                           void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * zero_shard_allgather -- the all-gather of the refreshed fp16 shards
 * ([S1M] "The per-step mechanics", beat 4: every rank broadcasts its fresh
 * fp16 shard and all ranks end with the identical fp16 model; [ZS] section
 * 3.1), for N simulated owners whose shard buffers sit in this GPU's memory:
 * the flat fp16 replica of psi parameters is the concatenation of the shards
 * in rank order, padding left out.
 *   shards      host array of n_ranks device pointers, each shard_len fp16
 *               values (binary16 bit patterns)
 *   shard_len   the layout's shard_len; a multiple of 8
 *   psi         number of parameters; replica[r*shard_len + j] = shards[r][j]
 *               for every r, j with r*shard_len + j < psi
 *   replica     device [psi] fp16, written
 * Errors: n_ranks not in [1, ZERO_MAX_SLICES], shard_len < 0 or not a
 * multiple of 8, psi < 0 or > n_ranks*shard_len, a NULL pointer (psi > 0),
 * replica overlapping a shard -> ZERO_ERR_INVALID_ARG; misaligned pointer ->
 * ZERO_ERR_MISALIGNED.
 */
int zero_shard_allgather(const uint16_t *const *shards, int32_t n_ranks,
                         int64_t shard_len, int64_t psi, uint16_t *replica,
                         hipStream_t stream);

/*
 * zero_shard_grad_stats -- overflow flag and sum of squares of the shard's
 * gradient.  [ZS] section 2.1: global clipping needs ||g||_2 over all of P,
 * one extra scalar all-reduce; this is the shard-local share.  The overflow
 * check (any +-inf/NaN) is the loss-scaling guard of mixed-precision
 * training; the pages name mixed precision ([ZS] section 1.2, fp16 enabled
 * in the configurations of section 8) but do not spell the check out.
 *   grad       device [len] of fp16 bit patterns (ZERO_F16) or fp32 (ZERO_F32)
 *   stats      device zero_grad_stats_t, written
 * Two kernels: per-block partials into `ws`, then one block sums them in a
 * fixed order (the result is deterministic run to run).  The gradient is
 * read from its end to its start, and its first 256 MiB (read last) so that
 * they stay in the Infinity Cache: an update enqueued right after this call
 * starts on them and reads them from there.  Errors as for the reduce.
 */
int zero_shard_grad_stats(const void *grad, int32_t grad_dtype,
                          int64_t len, double inv_grad_scale,
                          zero_grad_stats_t *stats, void *ws, size_t ws_bytes,
                          hipStream_t stream);

/*
 * zero_shard_adam_step -- the local optimizer step of one rank on its owned
 * shard ([S1M] "The per-step mechanics", beat 3; [ZS] section 2.1 Fact 1:
 * the update is elementwise, so the shard update is exact on its own).  Per
 * element, in binary32 ([ZS] section 2.1 equations; [S1M] "Where the 12 bytes
 * come from"; [ZOS] Stage 2: the shard's gradient is converted to fp32, the
 * fp32 states and master are updated, the fp16 copy is refreshed):
 *   g   = f32(grad[j]) * s
 *   m'  = b1*m + (1-b1)*g              v' = b2*v + (1-b2)*(g*g)
 *   th' = th - lr * ((m'/(1-b1^t)) / (sqrt(v'/(1-b2^t)) + eps))
 *   param16[j] = f16(th')
 * with s = inv_grad_scale and the scalars b1, 1-b1, b2, 1-b2, 1-b1^t, 1-b2^t,
 * lr, eps, s each computed in double on the host and rounded once to float.
 *   grad            device [len], fp16 bits or fp32 per grad_dtype (read only)
 *   master, exp_avg, exp_avg_sq   device fp32 [len], updated in place
 *   param16         device [len] fp16 bits, written (the shard's slice of the
 *                   flat compute copy)
 *   step            t >= 1, the number of this applied step
 *   hp              host pointer to the hyperparameters
 *   stats           device zero_grad_stats_t; computed here unless
 *                   stats_precomputed != 0, in which case it must already
 *                   hold the statistics of this same gradient and scale
 *   ws, ws_bytes    device workspace (>= zero_workspace_bytes(len)) when the
 *                   statistics are computed here; ignored otherwise
 * Overflow: when stats->overflow is 1 every block exits before touching the
 * states; master, exp_avg, exp_avg_sq and param16 keep their bits and the
 * caller should not advance t (the decision never needs a host sync).
 * Clipping (hp->max_grad_norm > 0) reads stats->sumsq on the device; with
 * stats_precomputed the caller may pass statistics summed over all ranks
 * (the all-reduced flag and sum of squares), which clips to the global norm.
 * Arrays must not overlap one another.  Errors: len < 0, a NULL pointer,
 * step < 1, lr < 0 or not finite, beta not in [0,1), eps <= 0, inv_grad_scale
 * not finite or <= 0, max_grad_norm < 0 or not finite, overlapping arrays
 * -> ZERO_ERR_INVALID_ARG; misaligned
 * pointer -> ZERO_ERR_MISALIGNED; short workspace -> ZERO_ERR_WORKSPACE.
 */
int zero_shard_adam_step(const void *grad, int32_t grad_dtype,
                         double inv_grad_scale, float *master, float *exp_avg,
                         float *exp_avg_sq, uint16_t *param16, int64_t len,
                         int64_t step, const zero_adam_hparams_t *hp,
                         zero_grad_stats_t *stats, int32_t stats_precomputed,
                         void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * zero_shard_adam_step_qwz -- zero_shard_adam_step that also encodes the
 * fresh fp16 shard for a quantized all-gather ([ZS] section 5.3, qwZ: the
 * fp16 weights travel as INT8 with one scale per block; [ZOS] ZeRO++: small
 * blocks with their own scale factors, dequantized to fp16 on receipt).
 * Same arguments, semantics and errors as zero_shard_adam_step, plus
 *   codes    device int8 [len], written: codes[j] = clamp(rint(f32(param16[j])
 *            / scale_b), -127, 127) for j in block b = j / ZERO_QWZ_BLOCK
 *            (0 when scale_b is 0)
 *   scales   device fp32 [ceil(len / ZERO_QWZ_BLOCK)], written: scale_b =
 *            max over the block of |f32(param16[j])| / 127
 * Blocks start at element 0 of the shard; the last may be short.  The codes
 * are those of zero_qwz_quantize applied to the param16 this call writes,
 * computed while the values are still in registers (1 + 4/256 bytes more per
 * parameter instead of a second pass of 3 + 4/256).  On overflow nothing is
 * written, codes and scales included.  Codes of a block holding a non-finite
 * fp16 weight are unspecified.  codes and scales must not overlap each other
 * or the other arrays.
 */
int zero_shard_adam_step_qwz(const void *grad, int32_t grad_dtype,
                             double inv_grad_scale, float *master,
                             float *exp_avg, float *exp_avg_sq,
                             uint16_t *param16, int8_t *codes, float *scales,
                             int64_t len, int64_t step,
                             const zero_adam_hparams_t *hp,
                             zero_grad_stats_t *stats,
                             int32_t stats_precomputed, void *ws,
                             size_t ws_bytes, hipStream_t stream);

/*
 * zero_shard_adam_step_device_t -- zero_shard_adam_step (or, with codes and
 * scales, zero_shard_adam_step_qwz) with the step number held in device
 * memory, so that a captured HIP graph of the step can be replayed step
 * after step with no host synchronisation: the bias corrections need t, and
 * t must not advance over a skipped step (the overflow flag lives on the
 * device).  Bias correction as in zero_shard_adam_step (Kingma & Ba, cited
 * by [ZS]): bc = (float)(1 - beta^t) in double, here evaluated by the
 * kernel.
 *   applied_steps   device zero_step_counter_t; applied holds the number
 *                   of steps applied so far (0 before the first) and must be
 *                   >= 0.  This call uses t = applied + 1: a one-thread
 *                   kernel enqueued before the update stores the two bias
 *                   corrections for t into the counter (the update reads
 *                   them from there) and adds 1 to applied when the step
 *                   applies (flag 0).
 *   codes, scales   both NULL (no encoding) or both set (as in
 *                   zero_shard_adam_step_qwz)
 * Other arguments, semantics and errors as zero_shard_adam_step; a NULL
 * counter, only one of codes/scales, or a counter overlapping another
 * argument -> ZERO_ERR_INVALID_ARG.
 */
int zero_shard_adam_step_device_t(const void *grad, int32_t grad_dtype,
                                  double inv_grad_scale, float *master,
                                  float *exp_avg, float *exp_avg_sq,
                                  uint16_t *param16, int8_t *codes,
                                  float *scales, int64_t len,
                                  zero_step_counter_t *applied_steps,
                                  const zero_adam_hparams_t *hp,
                                  zero_grad_stats_t *stats,
                                  int32_t stats_precomputed, void *ws,
                                  size_t ws_bytes, hipStream_t stream);

/*
 * zero_shard_adam_step_noalloc -- zero_shard_adam_step for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  It takes no workspace.  When the
 * statistics are computed here (stats_precomputed = 0), their per-block
 * partial results go to a scratch array the library holds in device memory:
 * ZERO_NOALLOC_SCRATCH_BYTES (32 KiB), one copy per device, kept until the
 * process ends.  The statistics kernel's grid is capped at 2048 blocks of
 * one 16-byte partial each whatever the length, so that size covers every
 * len and the call refuses none for lack of scratch (were a launch to need
 * more, the call would return ZERO_ERR_WORKSPACE and enqueue nothing).  The
 * call allocates nothing: on its first use on a device it looks up that
 * device's address of the array (make that first call outside graph
 * capture, as for every entry point), and after that it only enqueues
 * kernels.
 * Every call on one device uses that device's one scratch array and leaves
 * its own partials in it.  Each call writes every partial before reading
 * it, so nothing has to be cleared between calls, but calls that overlap in
 * time on one device (on two streams, or from two host threads without
 * ordering) race on the array and may produce wrong statistics, and with
 * them a wrong skip or clipping decision: order such calls on one stream.
 * Arguments, semantics, results and errors otherwise as
 * zero_shard_adam_step (with stats_precomputed != 0 no scratch is used).
 */
#define ZERO_NOALLOC_SCRATCH_BYTES 32768
int zero_shard_adam_step_noalloc(const void *grad, int32_t grad_dtype,
                                 double inv_grad_scale, float *master,
                                 float *exp_avg, float *exp_avg_sq,
                                 uint16_t *param16, int64_t len, int64_t step,
                                 const zero_adam_hparams_t *hp,
                                 zero_grad_stats_t *stats,
                                 int32_t stats_precomputed,
                                 hipStream_t stream);

/*
 * zero_qwz_quantize -- the qwZ encoder on its own ([ZS] section 5.3; [ZOS]
 * ZeRO++): blocks of ZERO_QWZ_BLOCK consecutive values from element 0, the
 * last possibly short; scale_b = max|x| / 127 in binary32 and code =
 * clamp(rint(x / scale_b), -127, 127) with one correctly rounded division and
 * ties to even, all codes 0 when scale_b is 0.
 *   x16      device fp16 [len] (binary16 bit patterns), finite values; codes
 *            of a block holding +-inf or NaN are unspecified
 *   codes    device int8 [len], written
 *   scales   device fp32 [ceil(len / ZERO_QWZ_BLOCK)], written
 * Errors: len < 0, a NULL pointer (len > 0), overlapping arrays ->
 * ZERO_ERR_INVALID_ARG; misaligned pointer -> ZERO_ERR_MISALIGNED.
 */
int zero_qwz_quantize(const uint16_t *x16, int64_t len, int8_t *codes,
                      float *scales, hipStream_t stream);

/*
 * zero_qwz_allgather -- receiver side of the quantized all-gather ([ZS]
 * section 5.3, qwZ; [ZOS] ZeRO++: received INT8 weights are dequantized back
 * to fp16 before use): the N owners' encoded shards, already in this GPU's
 * memory, are decoded into the flat fp16 replica:
 *   replica[r*shard_len + j] = f16(f32(codes[r][j]) * scales[r][j / 256])
 * (one binary32 product, round to nearest even) for every r, j with
 * r*shard_len + j < psi; padding is not written.
 *   codes, scales   host arrays of n_ranks device pointers: shard_len int8
 *                   codes and ceil(shard_len / 256) fp32 scales per rank,
 *                   as zero_qwz_quantize or zero_shard_adam_step_qwz write
 *   shard_len       the layout's shard_len; a multiple of 8
 *   replica         device [psi] fp16, written
 * Errors as for zero_shard_allgather.
 */
int zero_qwz_allgather(const int8_t *const *codes,
                       const float *const *scales, int32_t n_ranks,
                       int64_t shard_len, int64_t psi, uint16_t *replica,
                       hipStream_t stream);

/* ZERO_SHARD_ABI_VERSION as the library was built, so that a binding can
 * refuse a library built from another version of this header.  Host only;
 * no error. */
int zero_shard_abi_version(void);

/* Static text for a status code. */
const char *zero_status_string(int status);

/* Message of the last failed call on the calling thread ("" if none). */
const char *zero_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* ZERO_SHARD_H */
