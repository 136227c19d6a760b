/*
 * zero_oracle.c -- plain single-threaded CPU oracle (TEST INFRASTRUCTURE
 * ONLY; see zero_oracle.h for the sources, the citation key and what pins
 * each function).  Scalar loops, no SIMD, no blocking, no reordering.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math -fPIC -shared
 */
#include "zero_oracle.h"

#include <math.h>
#include <stddef.h>
#include <string.h>

/* ------------------------------------------------------------------ layout */

/* [ZS] section 2 (the partition definition), [S1M] "The core idea" (shard i
 * to rank i), [ZS] section 3.2 (the flat contiguous gradient buffer).  The
 * shard length is the smallest multiple of `align` that lets N equal shards
 * cover Psi. */
int zo_partition_layout(int64_t psi, int32_t n_ranks, int32_t rank,
                        int64_t align, int64_t out[5]) {
  if (out == NULL || psi < 0 || n_ranks < 1 || rank < 0 || rank >= n_ranks ||
      align < 1 || (align & (align - 1)) != 0)
    return ZO_ERR_INVALID_ARG;
  if (align > INT64_MAX / n_ranks) return ZO_ERR_INT_OVERFLOW;
  const int64_t unit = (int64_t)n_ranks * align; /* one aligned row over N */
  const int64_t rows = psi / unit + (psi % unit != 0 ? 1 : 0);
  if (rows > INT64_MAX / unit) return ZO_ERR_INT_OVERFLOW;
  const int64_t shard = rows * align;
  const int64_t offset = (int64_t)rank * shard;
  int64_t real = psi - offset;
  if (real < 0) real = 0;
  if (real > shard) real = shard;
  out[0] = psi;
  out[1] = shard * n_ranks;
  out[2] = shard;
  out[3] = offset;
  out[4] = real;
  return ZO_OK;
}

/* ------------------------------------------------------------ memory model */

/* [ZS] section 1.2: M_DP = 2Psi + 2Psi + K Psi; section 3.1: M1 = 4Psi +
 * K Psi/N; section 3.2: M2 = 2Psi + (2+K) Psi/N; section 3.3: M3 =
 * (4+K) Psi/N.  [DZE] "Three stages of partitioning" gives the same. */
double zo_model_state_bytes(double psi, int32_t n_ranks, int32_t stage,
                            double K) {
  if (!(psi >= 0.0) || n_ranks < 1 || !(K >= 0.0)) return -1.0;
  const double n = (double)n_ranks;
  switch (stage) {
    case 0: return 2.0 * psi + 2.0 * psi + K * psi;
    case 1: return 2.0 * psi + 2.0 * psi + K * psi / n;
    case 2: return 2.0 * psi + (2.0 * psi + K * psi) / n;
    case 3: return (2.0 * psi + 2.0 * psi + K * psi) / n;
    default: return -1.0;
  }
}

/* ------------------------------------------------------- binary16 formats */

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits.  Exponent field 0 = zero/subnormal (value f * 2^-24), 31 = inf/NaN,
 * otherwise (1024 + f) * 2^(e - 25). */
float zo_f16_to_f32(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int e = (h >> 10) & 31;
  const int f = h & 1023;
  float mag;
  if (e == 0)
    mag = ldexpf((float)f, -24);
  else if (e == 31)
    mag = (f == 0) ? INFINITY : NAN;
  else
    mag = ldexpf((float)(1024 + f), e - 25);
  return sign ? -mag : mag;
}

/* Round a binary32 value to the nearest binary16 value, ties to even.
 * Below 2^-14 the binary16 grid spacing is 2^-24 (subnormals); above it the
 * spacing is 2^(floor(log2|x|) - 10).  |x|/spacing is exact in double; it is
 * rounded to an integer with ties to even, and the result re-encoded.  A
 * rounded magnitude above 65504 (the largest finite binary16) is infinity. */
uint16_t zo_f32_to_f16(float x) {
  uint32_t bits;
  memcpy(&bits, &x, sizeof bits);
  const uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
  if (isnan(x)) return (uint16_t)(sign | 0x7E00u);
  if (isinf(x)) return (uint16_t)(sign | 0x7C00u);
  const double a = fabs((double)x);
  if (a == 0.0) return sign;
  int e2;
  (void)frexp(a, &e2); /* a in [2^(e2-1), 2^e2) */
  const double spacing = (a < 0x1p-14) ? 0x1p-24 : ldexp(1.0, (e2 - 1) - 10);
  const double r = nearbyint(a / spacing) * spacing; /* ties to even */
  if (r > 65504.0) return (uint16_t)(sign | 0x7C00u);
  if (r == 0.0) return sign;
  if (r < 0x1p-14) return (uint16_t)(sign | (uint16_t)(r * 0x1p24));
  int er;
  (void)frexp(r, &er); /* r in [2^(er-1), 2^er) */
  const int biased = (er - 1) + 15;
  const int frac = (int)(ldexp(r, -(er - 1)) * 1024.0) - 1024;
  return (uint16_t)(sign | (uint16_t)(biased << 10) | (uint16_t)frac);
}

void zo_f16_to_f32_array(const uint16_t *in, float *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = zo_f16_to_f32(in[i]);
}

void zo_f32_to_f16_array(const float *in, uint16_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = zo_f32_to_f16(in[i]);
}

/* ------------------------------------------------------------------ reduce */

/* Reduce-scatter, owner side ([ZS] sections 3.1-3.2, [DZE]
 * "communication"): the sum over ranks, folded left in rank order, one
 * binary32 addition per term. */
void zo_grad_reduce(const uint16_t *const *slices, int32_t n_slices,
                    int64_t len, float *out) {
  for (int64_t j = 0; j < len; ++j) {
    float acc = zo_f16_to_f32(slices[0][j]);
    for (int32_t r = 1; r < n_slices; ++r)
      acc = acc + zo_f16_to_f32(slices[r][j]);
    out[j] = acc;
  }
}

/* --------------------------------------------------------------- all-gather */

/* [S1M] "The per-step mechanics" beat 4: the flat fp16 replica is the
 * concatenation of the ranks' shards in rank order, padding left out. */
void zo_allgather(const uint16_t *const *shards, int32_t n_ranks,
                  int64_t shard_len, int64_t psi, uint16_t *replica) {
  for (int32_t r = 0; r < n_ranks; ++r)
    for (int64_t j = 0; j < shard_len; ++j) {
      const int64_t flat = (int64_t)r * shard_len + j;
      if (flat < psi) replica[flat] = shards[r][j];
    }
}

/* --------------------------------------------------------------------- qwZ */

/* [ZS] section 5.3 qwZ; the block rule is a reading (zero_oracle.h). */
void zo_qwz_quantize(const uint16_t *x16, int64_t len, int8_t *codes,
                     float *scales) {
  for (int64_t lo = 0; lo < len; lo += ZO_QWZ_BLOCK) {
    const int64_t hi = (lo + ZO_QWZ_BLOCK < len) ? lo + ZO_QWZ_BLOCK : len;
    float amax = 0.0f;
    for (int64_t j = lo; j < hi; ++j) {
      const float a = fabsf(zo_f16_to_f32(x16[j]));
      if (a > amax) amax = a;
    }
    const float scale = amax / 127.0f;
    scales[lo / ZO_QWZ_BLOCK] = scale;
    for (int64_t j = lo; j < hi; ++j) {
      float q = 0.0f;
      if (scale != 0.0f) {
        q = rintf(zo_f16_to_f32(x16[j]) / scale); /* ties to even */
        if (q > 127.0f) q = 127.0f;
        if (q < -127.0f) q = -127.0f;
      }
      codes[j] = (int8_t)q;
    }
  }
}

void zo_qwz_dequantize(const int8_t *codes, const float *scales, int64_t len,
                       uint16_t *out16) {
  for (int64_t j = 0; j < len; ++j)
    out16[j] = zo_f32_to_f16((float)codes[j] * scales[j / ZO_QWZ_BLOCK]);
}

/* ------------------------------------------------------------------- stats */

/* Neumaier's compensated summation: sum + comp is the running total. */
static void neumaier_add(double *sum, double *comp, double x) {
  const double t = *sum + x;
  if (fabs(*sum) >= fabs(x))
    *comp += (*sum - t) + x;
  else
    *comp += (x - t) + *sum;
  *sum = t;
}

static void stats_value(float x, float s, uint32_t *flag, double *sum,
                        double *comp) {
  if (!isfinite(x)) *flag = 1u;
  const float g = x * s;          /* unscaled gradient, as the step sees it */
  const double d = (double)g;
  neumaier_add(sum, comp, d * d); /* the square of a float is exact in double */
}

void zo_grad_stats_f16(const uint16_t *grad, int64_t len, double inv_scale,
                       uint32_t *overflow, double *sumsq) {
  const float s = (float)inv_scale;
  uint32_t flag = 0u;
  double sum = 0.0, comp = 0.0;
  for (int64_t j = 0; j < len; ++j)
    stats_value(zo_f16_to_f32(grad[j]), s, &flag, &sum, &comp);
  *overflow = flag;
  *sumsq = sum + comp;
}

void zo_grad_stats_f32(const float *grad, int64_t len, double inv_scale,
                       uint32_t *overflow, double *sumsq) {
  const float s = (float)inv_scale;
  uint32_t flag = 0u;
  double sum = 0.0, comp = 0.0;
  for (int64_t j = 0; j < len; ++j) stats_value(grad[j], s, &flag, &sum, &comp);
  *overflow = flag;
  *sumsq = sum + comp;
}

/* -------------------------------------------------------------------- Adam */

static int hparams_valid(double lr, double beta1, double beta2, double eps,
                         double inv_scale, int64_t step) {
  return step >= 1 && isfinite(lr) && lr >= 0.0 && beta1 >= 0.0 &&
         beta1 < 1.0 && beta2 >= 0.0 && beta2 < 1.0 && isfinite(eps) &&
         eps > 0.0 && isfinite(inv_scale) && inv_scale > 0.0;
}

int zo_adam_scalars(double lr, double beta1, double beta2, double eps,
                    double inv_scale, int64_t step, float s[9]) {
  if (!hparams_valid(lr, beta1, beta2, eps, inv_scale, step))
    return ZO_ERR_INVALID_ARG;
  s[0] = (float)beta1;
  s[1] = (float)(1.0 - beta1);
  s[2] = (float)beta2;
  s[3] = (float)(1.0 - beta2);
  s[4] = (float)(1.0 - pow(beta1, (double)step));
  s[5] = (float)(1.0 - pow(beta2, (double)step));
  s[6] = (float)lr;
  s[7] = (float)eps;
  s[8] = (float)inv_scale;
  return ZO_OK;
}

/* [ZS] section 2.1 (global clipping needs the 2-norm over all of P); the
 * rule itself is a reading, see zero_oracle.h. */
double zo_clip_factor(double sumsq, double max_norm) {
  if (!(max_norm > 0.0)) return 1.0;
  const double norm = sqrt(sumsq);
  return norm > max_norm ? max_norm / norm : 1.0;
}

/* [ZS] section 2.1 Fact 1 and [S1M] "Where the 12 bytes come from": the
 * moment updates, the bias-corrected hats, the master-weight step with eps
 * outside the square root, then the fp16 compute copy. */
void zo_adam_element(float x, const float s[9], float *master, float *m,
                     float *v, uint16_t *p16) {
  const float b1 = s[0], omb1 = s[1], b2 = s[2], omb2 = s[3];
  const float bc1 = s[4], bc2 = s[5], lr = s[6], eps = s[7], inv = s[8];
  const float g = x * inv;
  const float m1 = b1 * *m + omb1 * g;
  const float v1 = b2 * *v + omb2 * (g * g);
  const float mh = m1 / bc1;
  const float vh = v1 / bc2;
  const float th1 = *master - lr * (mh / (sqrtf(vh) + eps));
  *m = m1;
  *v = v1;
  *master = th1;
  *p16 = zo_f32_to_f16(th1);
}

int zo_adam_apply_f16(const uint16_t *grad, float *master, float *m, float *v,
                      uint16_t *p16, int64_t len, int64_t step, double lr,
                      double beta1, double beta2, double eps, double inv_scale,
                      uint32_t overflow) {
  float s[9];
  const int st = zo_adam_scalars(lr, beta1, beta2, eps, inv_scale, step, s);
  if (st != ZO_OK) return st;
  if (overflow) return ZO_OK; /* skipped step: nothing is written */
  for (int64_t j = 0; j < len; ++j)
    zo_adam_element(zo_f16_to_f32(grad[j]), s, &master[j], &m[j], &v[j],
                    &p16[j]);
  return ZO_OK;
}

int zo_adam_apply_f32(const float *grad, float *master, float *m, float *v,
                      uint16_t *p16, int64_t len, int64_t step, double lr,
                      double beta1, double beta2, double eps, double inv_scale,
                      uint32_t overflow) {
  float s[9];
  const int st = zo_adam_scalars(lr, beta1, beta2, eps, inv_scale, step, s);
  if (st != ZO_OK) return st;
  if (overflow) return ZO_OK;
  for (int64_t j = 0; j < len; ++j)
    zo_adam_element(grad[j], s, &master[j], &m[j], &v[j], &p16[j]);
  return ZO_OK;
}

int zo_shard_adam_step_f16(const uint16_t *grad, float *master, float *m,
                           float *v, uint16_t *p16, int64_t len, int64_t step,
                           double lr, double beta1, double beta2, double eps,
                           double inv_scale, double max_norm,
                           uint32_t *overflow, double *sumsq) {
  float s[9];
  if (zo_adam_scalars(lr, beta1, beta2, eps, inv_scale, step, s) != ZO_OK ||
      !isfinite(max_norm) || max_norm < 0.0)
    return ZO_ERR_INVALID_ARG;
  zo_grad_stats_f16(grad, len, inv_scale, overflow, sumsq);
  if (*overflow) return ZO_OK; /* skipped step: nothing is written */
  const double scale = inv_scale * zo_clip_factor(*sumsq, max_norm);
  return zo_adam_apply_f16(grad, master, m, v, p16, len, step, lr, beta1,
                           beta2, eps, scale, 0u);
}

int zo_shard_adam_step_f32(const float *grad, float *master, float *m,
                           float *v, uint16_t *p16, int64_t len, int64_t step,
                           double lr, double beta1, double beta2, double eps,
                           double inv_scale, double max_norm,
                           uint32_t *overflow, double *sumsq) {
  float s[9];
  if (zo_adam_scalars(lr, beta1, beta2, eps, inv_scale, step, s) != ZO_OK ||
      !isfinite(max_norm) || max_norm < 0.0)
    return ZO_ERR_INVALID_ARG;
  zo_grad_stats_f32(grad, len, inv_scale, overflow, sumsq);
  if (*overflow) return ZO_OK; /* skipped step: nothing is written */
  const double scale = inv_scale * zo_clip_factor(*sumsq, max_norm);
  return zo_adam_apply_f32(grad, master, m, v, p16, len, step, lr, beta1,
                           beta2, eps, scale, 0u);
}
