/*
 * zero_testkit.h -- seeded synthetic inputs and plain streaming reference
 * kernels, for the tests and the benchmark of the shard optimizer step.
 * Nothing here computes any part of the optimizer step or includes the
 * optimizer library's code (its probes are in zero_probes.h); the same
 * generated device buffers feed both the HIP library and (after a copy to
 * the host) the CPU oracle.
 *
 * Generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC'11), a counter-based generator: element j
 * of a tensor is a pure function of (seed, stream, j), so any element can be
 * regenerated alone.  Key = (seed low 32, seed high 32); counter = (j low 32,
 * j high 32, stream, draw).  Uniforms on (0,1) take 53 bits from two output
 * words: ((w_a >> 5) * 2^26 + (w_b >> 6) + 0.5) * 2^-53.  Normals by
 * Box-Muller in double: sqrt(-2 ln u1) * (cos, sin)(2 pi u2).
 *
 * All calls validate their arguments, enqueue on `stream_` (a hipStream_t)
 * and return 0 on success, -1 on a bad argument, -4 on a HIP error.
 * Output pointers are caller-owned device memory.
 */
#ifndef ZERO_TESTKIT_H
#define ZERO_TESTKIT_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Raw Philox4x32-10 blocks: out[4*i .. 4*i+3] for counter (i, 0, stream, 0)
 * under key (seed low, seed high).  For known-answer checks. */
int zero_testkit_philox(uint32_t *out, int64_t n_blocks, uint64_t seed, uint32_t stream,
                        hipStream_t stream_);

/* out[j] = (float)(mean + std * z_j), z_j standard normal (first Box-Muller
 * output of draw 0); when abs_value != 0 the magnitude |mean + std*z_j|. */
int zero_testkit_normal_f32(float *out, int64_t n, double mean, double std, int32_t abs_value,
                            uint64_t seed, uint32_t stream, hipStream_t stream_);

/* out[j] = binary16 bits of (half)(float)(scale * z_j), z_j standard normal. */
int zero_testkit_normal_f16(uint16_t *out, int64_t n, double scale, uint64_t seed, uint32_t stream,
                            hipStream_t stream_);

/* out[j] = binary16 bits of (half)(float)(scale * t_j), t_j Student-t with 3
 * degrees of freedom, t = z0 / sqrt((z1^2 + z2^2 + z3^2) / 3) from two
 * Philox draws.  When redraw_overflow != 0, a value whose binary16 would be
 * infinite is drawn again (up to 8 attempts, then clamped to +-65504), so the
 * result is finite everywhere. */
int zero_testkit_student_t3_f16(uint16_t *out, int64_t n, double scale, int32_t redraw_overflow,
                                uint64_t seed, uint32_t stream, hipStream_t stream_);

/* Sets out[j] to +inf (0x7C00) where the uniform of (seed, stream, j) is
 * below `prob`; other elements are left as they are. */
int zero_testkit_inject_inf_f16(uint16_t *out, int64_t n, double prob, uint64_t seed, uint32_t stream,
                                hipStream_t stream_);

/* Plain streaming kernels that set the attainable HBM ceiling and calibrate
 * the FETCH_SIZE / WRITE_SIZE counters: dst = src over n floats (8 B of
 * traffic per element; 16-byte aligned pointers); and a read of the first
 * floor(n/4)*4 floats whose per-block sums go to sink[block] for the blocks
 * below sink_len (4 B per element; at most 4 blocks per CU are launched). */
int zero_testkit_copy_f32(const float *src, float *dst, int64_t n, hipStream_t stream_);
int zero_testkit_read_f32(const float *src, int64_t n, float *sink, int32_t sink_len,
                          hipStream_t stream_);

/* Streaming reference of many-slice traffic: reads n (1..64) slices of
 * len binary16 values each, in tiles of 1024 elements per 128-thread block
 * with four slices' loads in flight and at most six blocks per CU.  When
 * out is not NULL, out[j] (32-bit) = XOR over the slices of slices[r][j]
 * (zero-extended), so the traffic is n*2 + 4 bytes per element; when out is
 * NULL nothing but sink is written (n*2 bytes per element).  sink[b] for the
 * blocks b below sink_len = XOR over block b's elements and slices of the
 * zero-extended values.  len must be a multiple of 4 and the pointers
 * 16-byte aligned. */
int zero_testkit_read_slices(const uint16_t *const *slices, int32_t n, int64_t len, uint32_t *out,
                             uint32_t *sink, int32_t sink_len, hipStream_t stream_);

/* Text of the HIP error behind the last -4 on the calling thread. */
const char *zero_testkit_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* ZERO_TESTKIT_H */
