/*
 * zero_host_adam.h -- C ABI of the multi-core host implementation of one
 * rank's shard Adam step: the same step as zero_shard_adam_step, run over
 * host memory on all host cores with SIMD (AVX-512 or AVX2 with F16C): the
 * CPU Adam of ZeRO-Offload ("DeepSpeed ZeRO Stages" section 5.1: the fp32
 * states and the update move to the CPU, made viable by a hand-tuned SIMD +
 * OpenMP Adam; "DeepSpeed ZeRO: Extreme Memory Efficiency", "Offloading the
 * optimizer entirely: ZeRO-Offload"; "ZeRO Optimization: Stages 1, 2, and 3
 * Explained", ZeRO-Offload: the step is elementwise and runs well on CPUs).
 *
 * Arithmetic: identical to the GPU library's -- per element, one IEEE
 * binary32 operation per operator in the order
 *   g = f32(grad[j]) * s
 *   m' = b1*m + (1-b1)*g            v' = b2*v + (1-b2)*(g*g)
 *   th' = th - lr * ((m'/(1-b1^t)) / (sqrt(v'/(1-b2^t)) + eps))
 *   param16[j] = f16(th')           (round to nearest even)
 * with no contraction, correctly rounded division and square root and
 * subnormals kept; the nine scalars are computed in double and rounded once.
 * Every instruction set level gives the same bits.  The overflow flag and the
 * sum of squares of g = f32(grad[j]) * inv_grad_scale (in double) come from
 * the same call; the sum is formed in a fixed order (16 interleaved
 * accumulators per 65,536-element chunk, chunks summed in index order), so it
 * does not depend on the thread count or the instruction set.
 *
 * Conventions: host pointers, caller-owned; no allocation beyond a per-call
 * array of per-chunk partials; every call returns a status (0 = ok) and on
 * failure writes nothing, with zero_host_last_error() holding a message for
 * the calling thread.  The host library is independent of the GPU library.
 */
#ifndef ZERO_HOST_ADAM_H
#define ZERO_HOST_ADAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZERO_HOST_OK 0
#define ZERO_HOST_ERR_INVALID_ARG (-1)
#define ZERO_HOST_ERR_UNSUPPORTED (-6) /* the CPU lacks F16C (x86-64-v3) */

#define ZERO_HOST_F16 1 /* gradient as binary16 bit patterns */
#define ZERO_HOST_F32 2 /* gradient as binary32 */

/* Instruction set levels: 1 = scalar (F16C), 2 = AVX2 + F16C, 3 = AVX-512. */
#define ZERO_HOST_ISA_SCALAR 1
#define ZERO_HOST_ISA_AVX2 2
#define ZERO_HOST_ISA_AVX512 3

typedef struct {
  double lr, beta1, beta2, eps;
  double max_grad_norm; /* > 0: clip to this global 2-norm; 0: off */
} zero_host_adam_hparams_t;

typedef struct {
  uint32_t overflow; /* 1 if any gradient value is +-inf or NaN */
  uint32_t reserved;
  double sumsq;      /* sum of (f32(grad[j]) * inv_grad_scale)^2 in double */
} zero_host_stats_t;

/*
 * zero_host_adam_step -- the whole shard step on the CPU: statistics of the
 * gradient (unless stats_precomputed != 0, in which case *stats must hold
 * them, e.g. all-reduced over ranks), then, if the flag is 0, the update of
 * master / exp_avg / exp_avg_sq in place and the fp16 copy.  When the flag
 * is 1 nothing is written and the caller should not advance t.  Clipping
 * (hp->max_grad_norm > 0): when sqrt(sumsq) > max_grad_norm the unscale
 * multiplier becomes (float)(inv_grad_scale * (max_grad_norm/sqrt(sumsq))),
 * evaluated in double.
 *   grad        host [len], binary16 bits (ZERO_HOST_F16) or binary32
 *   master, exp_avg, exp_avg_sq   host fp32 [len], updated in place
 *   param16     host [len] binary16 bits, written
 *   stats       host, written (or read when stats_precomputed)
 *   n_threads   OpenMP threads; 0 = the OpenMP default
 * Each array must be aligned to its element size (2 bytes for binary16, 4
 * for binary32), as any C array of that type is.
 * Errors: len < 0, NULL pointer (len > 0), unknown dtype, step < 1, lr < 0
 * or not finite, beta not in [0,1), eps <= 0, inv_grad_scale not finite or
 * <= 0, max_grad_norm < 0 or not finite, n_threads < 0, overlapping or
 * misaligned arrays -> ZERO_HOST_ERR_INVALID_ARG; no F16C ->
 * ZERO_HOST_ERR_UNSUPPORTED.
 */
int zero_host_adam_step(const void *grad, int32_t grad_dtype,
                        double inv_grad_scale, float *master, float *exp_avg,
                        float *exp_avg_sq, uint16_t *param16, int64_t len,
                        int64_t step, const zero_host_adam_hparams_t *hp,
                        zero_host_stats_t *stats, int32_t stats_precomputed,
                        int32_t n_threads);

/*
 * zero_host_adam_set_isa -- choose the instruction set level for later calls
 * in this process: 0 = the best the CPU supports, or one of the
 * ZERO_HOST_ISA_* levels (lowered to what the CPU supports).  Returns the
 * level now in use, or ZERO_HOST_ERR_INVALID_ARG / ZERO_HOST_ERR_UNSUPPORTED.
 * Every level computes the same bits; this exists to test that and to time
 * them.  Not synchronised with calls running on other threads.
 */
int zero_host_adam_set_isa(int32_t level);

/* Message of the last failed call on the calling thread ("" if none). */
const char *zero_host_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* ZERO_HOST_ADAM_H */
