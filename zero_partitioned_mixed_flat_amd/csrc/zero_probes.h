/*
 * zero_probes.h -- device probes of the optimizer library's own code, for
 * the tests and the benchmark: they run the library's arithmetic helpers
 * and its streaming-store policy on given inputs, so that tests can compare
 * them with host IEEE results and the benchmark can measure the attainable
 * rate of a read-modify-write stream.  Built from the library's kernel
 * header into a library of their own (libzero_probes.so); the seeded input
 * generators (zero_testkit.h) share none of this code.
 *
 * All calls validate their arguments, enqueue on `stream_` (a hipStream_t)
 * and return 0 on success, -1 on a bad argument, -4 on a HIP error.
 * Pointers are caller-owned device memory.
 */
#ifndef ZERO_PROBES_H
#define ZERO_PROBES_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* quot[j] = a[j] / b[j], root[j] = sqrt(a[j]), half[j] = binary16 of a[j]
 * and wide[j] = binary32 of the binary16 code h[j], each with the primitive
 * and build flags of the optimizer library (correctly rounded division and
 * square root, round-to-nearest-even conversion, subnormals kept).  All
 * arrays hold n elements. */
int zero_probes_arith_f32(const float *a, const float *b, const uint16_t *h, int64_t n, float *quot,
                          float *root, uint16_t *half, float *wide, hipStream_t stream_);

/* out[j] = the library's device-side bias correction (float)(1 - beta^t[j])
 * for n step numbers t. */
int zero_probes_bias_correction(double beta, const int64_t *t, int64_t n, float *out, hipStream_t stream_);

/* In place: p[j] += 1 over the first floor(n/4)*4 floats (8 B of traffic
 * per element), non-temporal loads and the library's streaming-store policy:
 * the attainable rate of the optimizer's read-modify-write streams.  p is
 * 16-byte aligned. */
int zero_probes_rmw_f32(float *p, int64_t n, hipStream_t stream_);

/* Text of the HIP error behind the last -4 on the calling thread. */
const char *zero_probes_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* ZERO_PROBES_H */
