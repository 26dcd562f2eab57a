/*
 * gqa_probe.h -- achievable-peak probes of the MI355X, exported by the same
 * library as gqa_attn.h for measurement only: no part of the attention path
 * calls them. They give the two ceilings the attention kernels are held
 * against on the machine at hand, next to the published peaks (bf16 dense
 * MFMA 2.5 PFLOP/s, HBM3E 8 TB/s): the matrix-core rate of the instruction
 * the attention products use, and the rate at which a plain read streams a
 * buffer from HBM. Both time each launch with HIP events recorded by the
 * launch itself, on a private stream, after the device is idle, and return
 * the median over `reps` launches. Errors are gqa_status codes with a
 * message in gqa_attn_last_error().
 */
#ifndef GQA_PROBE_H
#define GQA_PROBE_H

#include <stdint.h>

#include "gqa_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* v_mfma_f32_32x32x16_bf16 throughput: waves_per_simd (1..8) waves on every
 * SIMD of every CU, each running `iters` rounds of four independent
 * accumulator chains. FLOPs per launch = CUs x 4 SIMDs x waves_per_simd x
 * iters x 4 x 32768. Returns the median TFLOP/s and milliseconds. The
 * probe allocates (and frees) its small output buffer. */
gqa_status gqa_probe_mfma_bf16(int32_t waves_per_simd, int32_t iters, int32_t reps, double* tflops,
                               double* ms);

/* Streaming read: launch k reads copy k % n_copies of `buf` (device, 16-byte
 * aligned, n_copies x bytes, bytes a multiple of 16) with 16-byte loads,
 * grid-stride over 8 workgroups of 256 threads per CU. Returns the median
 * GB/s (bytes / launch time) and microseconds. Rotating over copies larger
 * than the 256 MB Infinity Cache keeps the bytes coming from HBM. */
gqa_status gqa_probe_read(const void* buf, int64_t bytes, int32_t n_copies, int32_t reps, double* gbps,
                          double* us);

#ifdef __cplusplus
}
#endif

#endif /* GQA_PROBE_H */
