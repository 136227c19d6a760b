/*
 * zero_oracle.h -- plain, slow, single-threaded CPU oracle of one ZeRO rank's
 * optimizer step over its owned partition of the flat parameter space.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this code: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no source with the HIP library.
 *
 * Sources (four web pages on DeepSpeed ZeRO; citations name page and section):
 *   [ZS]  "DeepSpeed ZeRO Stages" (yiqiao-yin.github.io deepspeed-course)
 *   [S1M] "ZeRO Stage 1 Math" (aicassindra.com, transformer_math)
 *   [ZOS] "ZeRO Optimization: Stages 1, 2, and 3 Explained" (mbrenndoerfer.com)
 *   [DZE] "DeepSpeed ZeRO: Extreme Memory Efficiency" (aicomputerinstitute.com)
 *
 * Floating point: every float operation below is one IEEE-754 binary32
 * operation with round-to-nearest-even, evaluated in the order written, with
 * no contraction (built with -ffp-contract=off, SSE arithmetic, no fast-math).
 *
 * Parity status per function (what pins it, see tests/test_oracle_*.py):
 *   zo_partition_layout     pinned: brute-force partition properties, config shard sizes
 *   zo_model_state_bytes    pinned: every worked memory figure printed on the pages
 *   zo_f16_to_f32           pinned: exhaustive over 65,536 codes vs numpy
 *   zo_f32_to_f16           pinned: exhaustive over 2^32 codes vs numpy / F16C
 *   zo_grad_reduce          pinned: exact integer sums, identity at N=1, fp32 error bound,
 *                                   hand-worked order-dependent case
 *   zo_allgather            pinned: numpy concatenation of the real parts, scatter/gather
 *                                   round trip through the partition layout
 *   zo_qwz_*                pinned: exact multiples of a power-of-two scale, ties to even,
 *                                   zero blocks, the +-127 extremes, round-trip error bound
 *   zo_grad_stats_*         pinned: injected-inf counts, exact rational sum of squares
 *   zo_adam_*               pinned: t=1 closed form, constant-gradient closed forms,
 *                                   pure-decay closed forms, high-precision evaluation,
 *                                   separability and skip invariants
 *   zo_clip_factor          pinned: the clipped gradient's norm equals max_norm
 *                                   (exact rational check), no-op below the bound
 */
#ifndef ZERO_ORACLE_H
#define ZERO_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes (same meaning as the library's, defined independently) */
#define ZO_OK 0
#define ZO_ERR_INVALID_ARG (-1)
#define ZO_ERR_INT_OVERFLOW (-5)

/* ---- partition of the flat index set ----------------------------------
 * [ZS] section 2 defines a partition of the parameter indices {1..Psi} into
 * disjoint sets P_1..P_N whose union is everything, each of size about Psi/N,
 * rank i owning P_i; [S1M] "The core idea" assigns shard i to rank i.
 * Reading: equal contiguous blocks in rank order, each padded to a multiple
 * of `align` (a power of two), L = ceil(Psi / (N*align)) * align.
 * out[0..4] = {psi, psi_padded = N*L, shard_len = L, offset = rank*L,
 *              real_len = clamp(psi - offset, 0, L)}.                      */
int zo_partition_layout(int64_t psi, int32_t n_ranks, int32_t rank,
                        int64_t align, int64_t out[5]);

/* ---- model-state memory per GPU in bytes ------------------------------
 * [ZS] section 1.2 (M_DP = (4+K) Psi), sections 3.1-3.3 (M1, M2, M3);
 * [DZE] "Three stages of partitioning" (the same four formulas).
 * stage 0 = plain data parallelism.  Returns a negative value on bad input. */
double zo_model_state_bytes(double psi, int32_t n_ranks, int32_t stage,
                            double K);

/* ---- binary16 <-> binary32 (IEEE-754 definitions) ---------------------
 * [S1M] "Where the 12 bytes come from": the master copy is rounded down to
 * fp16 for the forward pass; read as round-to-nearest-even.                 */
float zo_f16_to_f32(uint16_t h);
uint16_t zo_f32_to_f16(float x);
void zo_f16_to_f32_array(const uint16_t *in, float *out, int64_t n);
void zo_f32_to_f16_array(const float *in, uint16_t *out, int64_t n);

/* ---- owner-side arithmetic of the gradient reduce-scatter -------------
 * [ZS] section 3.1 (rank i receives the fully reduced gradient for P_i) and
 * section 3.2 (gradients reduced into the owner's buffer); [DZE]
 * "communication" (the reduce-scatter sums).  out[j] = left fold in fp32 of
 * f32(slices[0][j]) + f32(slices[1][j]) + ... in rank order.               */
void zo_grad_reduce(const uint16_t *const *slices, int32_t n_slices,
                    int64_t len, float *out);

/* ---- all-gather of the refreshed fp16 shards ---------------------------
 * [S1M] "The per-step mechanics" beat 4 and [ZS] section 3.1: every rank's
 * fresh fp16 shard is gathered so all ranks hold the identical full fp16
 * model.  On one GPU: the N shard buffers (shard_len each) are concatenated
 * into the flat replica of psi parameters; element j of rank r lands at
 * r*shard_len + j when that is below psi (padding is not copied).         */
void zo_allgather(const uint16_t *const *shards, int32_t n_ranks,
                  int64_t shard_len, int64_t psi, uint16_t *replica);

/* ---- qwZ: block INT8 quantization of the outgoing fp16 weights --------
 * [ZS] section 5.3 (qwZ: fp16 weights sent as INT8 with per-block scales)
 * and the ZeRO++ discussion of [ZOS] (small blocks, each with its own scale;
 * dequantized back to fp16 on receipt).  Block size, scale and rounding are
 * not on the pages; reading: blocks of ZO_QWZ_BLOCK consecutive values of the
 * flat shard, symmetric scale = max|x| / 127 (binary32), code =
 * clamp(rint(x / scale), -127, 127) with x / scale one correctly rounded
 * binary32 division and rint ties-to-even; a block whose max is 0 has scale
 * 0 and all codes 0.  Dequantization: f16(code * scale), one binary32
 * product then round-to-nearest-even.  Inputs are finite fp16 values.      */
#define ZO_QWZ_BLOCK 256
void zo_qwz_quantize(const uint16_t *x16, int64_t len, int8_t *codes,
                     float *scales);
void zo_qwz_dequantize(const int8_t *codes, const float *scales, int64_t len,
                       uint16_t *out16);

/* ---- gradient statistics: overflow flag and sum of squares ------------
 * [ZS] section 2.1 (global clipping needs ||g||_2 over all of P, one scalar
 * all-reduce): the shard-local share is sum_j g_j^2 with g_j = f32(x_j)*s.
 * The overflow flag (any +-inf or NaN in the step's gradient input) is not
 * on the pages; it is the mixed-precision loss-scaling check.  sumsq is
 * accumulated in double with Neumaier compensation.                       */
void zo_grad_stats_f16(const uint16_t *grad, int64_t len, double inv_scale,
                       uint32_t *overflow, double *sumsq);
void zo_grad_stats_f32(const float *grad, int64_t len, double inv_scale,
                       uint32_t *overflow, double *sumsq);

/* ---- Adam on the owned shard -------------------------------------------
 * [ZS] section 2.1 Fact 1 (the Adam equations), [S1M] "Where the 12 bytes
 * come from" (the same update with bias-corrected hats), [ZOS] Stage 2
 * mixed-precision paragraph (grad to fp32, update fp32 states, refresh fp16
 * copy).  Bias correction follows Kingma & Ba as cited by [ZS] references:
 * mhat = m/(1-b1^t), vhat = v/(1-b2^t).  Per-step scalars are derived in
 * double and rounded once to float:
 *   s[0]=b1 s[1]=1-b1 s[2]=b2 s[3]=1-b2 s[4]=1-b1^t s[5]=1-b2^t
 *   s[6]=lr s[7]=eps s[8]=inv_scale                                       */
int zo_adam_scalars(double lr, double beta1, double beta2, double eps,
                    double inv_scale, int64_t step, float s[9]);

/* Global-norm gradient clipping ([ZS] section 2.1: clipping needs ||g||_2
 * over all of P, one scalar all-reduce).  The pages do not spell the rule
 * out; reading: with norm = sqrt(sumsq) of the unscaled gradient, the
 * gradient is multiplied by max_norm / norm when max_norm > 0 and norm >
 * max_norm, else left alone.  Returns that factor (1 when not clipping).
 * The step folds it into the unscale multiplier: s = (float)(inv_scale *
 * factor), one rounding, computed in double. */
double zo_clip_factor(double sumsq, double max_norm);

/* One element: g = f32(x)*s; m1 = b1*m + (1-b1)*g; v1 = b2*v + (1-b2)*(g*g);
 * mh = m1/bc1; vh = v1/bc2; th1 = th - lr*(mh/(sqrt(vh)+eps)); p = f16(th1). */
void zo_adam_element(float x, const float s[9], float *master, float *m,
                     float *v, uint16_t *p16);

/* Apply the update to `len` elements when `overflow` is 0; when it is 1
 * nothing is written (the step is skipped).  grad is fp16 bits or fp32.     */
int zo_adam_apply_f16(const uint16_t *grad, float *master, float *m, float *v,
                      uint16_t *p16, int64_t len, int64_t step, double lr,
                      double beta1, double beta2, double eps, double inv_scale,
                      uint32_t overflow);
int zo_adam_apply_f32(const float *grad, float *master, float *m, float *v,
                      uint16_t *p16, int64_t len, int64_t step, double lr,
                      double beta1, double beta2, double eps, double inv_scale,
                      uint32_t overflow);

/* Whole step on a shard: statistics of the gradient, then the gated update
 * (clipped to max_norm when max_norm > 0, from the shard's own sum of
 * squares).  Returns ZO_OK or ZO_ERR_INVALID_ARG; *overflow and *sumsq are
 * outputs.                                                                */
int zo_shard_adam_step_f16(const uint16_t *grad, float *master, float *m,
                           float *v, uint16_t *p16, int64_t len, int64_t step,
                           double lr, double beta1, double beta2, double eps,
                           double inv_scale, double max_norm,
                           uint32_t *overflow, double *sumsq);
int zo_shard_adam_step_f32(const float *grad, float *master, float *m,
                           float *v, uint16_t *p16, int64_t len, int64_t step,
                           double lr, double beta1, double beta2, double eps,
                           double inv_scale, double max_norm,
                           uint32_t *overflow, double *sumsq);

#ifdef __cplusplus
}
#endif
#endif /* ZERO_ORACLE_H */
