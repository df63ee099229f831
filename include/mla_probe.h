/* Achievable-peak probe for MI355X (gfx950).
 *
 * A MEASUREMENT HOOK, not part of the decode path: it runs the matrix-core
 * shapes the decode kernels use with every CU busy, so that the rate the chip
 * actually reaches can be set beside the published dense peaks (bf16 and
 * fp16 2.5 PFLOP/s, fp8 5.0 PFLOP/s) that the roofline fractions are taken
 * against. `bench.py --peaks` reports it together with the rates of torch's
 * device copy and fill.
 *
 * Built as its own library, mla_paged_decode_04_amd/libmla_probe.so.
 */
#ifndef MLA_PROBE_H
#define MLA_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_PROBE_MFMA_16X16X32_BF16 = 0,   /* v_mfma_f32_16x16x32_bf16 */
  MLA_PROBE_MFMA_32X32X16_BF16 = 1,   /* v_mfma_f32_32x32x16_bf16 */
  MLA_PROBE_MFMA_16X16X128_FP8 = 2    /* v_mfma_scale_f32_16x16x128_f8f6f4, e4m3fn x e4m3fn, unit scales */
} mla_probe_shape_t;

/* Workgroup size of mla_probe_mfma: 8 waves of 64 lanes. */
#define MLA_PROBE_THREADS 512
/* Independent accumulator chains per wave, so that MFMA latency is covered. */
#define MLA_PROBE_CHAINS 8

/* Floating-point operations of one mla_probe_mfma launch (host only):
 * workgroups x 8 waves x iters x MLA_PROBE_CHAINS x 2 M N K of the shape.
 * Returns 0 for an unknown shape or a count below 1. */
double mla_probe_mfma_flops(int32_t shape, int32_t workgroups, int32_t iters);

/* The value each thread writes (host only): the sum of its accumulator
 * elements after the launch, when every operand element is x (exactly
 * representable in bf16 and e4m3fn, e.g. 2^-4): MLA_PROBE_CHAINS x (elements
 * per lane) x iters x K x x^2. Returns 0 for an unknown shape. */
double mla_probe_mfma_expected(int32_t shape, int32_t iters, float x);

/* Launches `workgroups` workgroups of MLA_PROBE_THREADS threads on `stream`
 * (a hipStream_t; null = the default stream). Each wave runs `iters` rounds
 * of MLA_PROBE_CHAINS independent MFMAs of `shape` on register operands whose
 * elements all equal x (rounded to the operand type on the device), then every
 * thread writes the sum of its accumulator elements to out[workgroup *
 * MLA_PROBE_THREADS + thread].
 *   out: device memory for workgroups * MLA_PROBE_THREADS floats, owned by the
 *        caller; nothing is retained after the call.
 * Returns 0 when launched; 1 for an invalid argument (unknown shape,
 * workgroups or iters below 1, workgroups above 2^20, iters above 2^24, null
 * out), in which case nothing is launched; 2 when the launch itself failed. */
int32_t mla_probe_mfma(int32_t shape, int32_t workgroups, int32_t iters, float x, float* out,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PROBE_H */
