/*
 * pmn_probe.h -- measurement kernels of libpmn.so. They are not part of the layer: they give the
 * benchmark the roofs it rates the layer's kernels against, measured on the same chip in the same
 * run (HBM bandwidth for a kernel's own read:write mix, and the throughput of each MFMA
 * instruction the grouped GEMMs issue). Conventions (device pointers, asynchronous on `stream`,
 * PMN_E* status codes, no allocation) are those of pmn.h.
 */
#ifndef PMN_PROBE_H
#define PMN_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "pmn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Streams `units` units through HBM. A unit reads read_kb contiguous KB of src and writes
 * write_kb contiguous KB of dst (src holds units * read_kb KB, dst units * write_kb KB; both
 * 16-byte aligned). Every access is 16 bytes wide and one wavefront handles one unit at a time;
 * `grid` workgroups of 256 threads stride over the units. hints: bit 0 = nontemporal loads, bit 1
 * = nontemporal stores (0..3, else PMN_EINVAL). The written bytes are a function of every byte
 * read. read_kb + write_kb > 0 (PMN_ESHAPE).
 */
int pmn_probe_stream(const void* src, void* dst, int64_t units, int read_kb, int write_kb, int grid, int hints,
                     pmn_stream_t stream);

/* Floats pmn_probe_mfma writes to `sink` (one per thread of the launch). */
size_t pmn_probe_mfma_sink_floats(int waves_per_simd, int workgroups);

/*
 * Matrix-core throughput of one MFMA instruction: `workgroups` workgroups of 4 * waves_per_simd
 * wavefronts (1 or 2) each run `iters` iterations of independent accumulator chains on constant
 * operands, with no memory traffic. kind: 0 v_mfma_f32_32x32x16_f16, 1 v_mfma_f32_16x16x32_f16,
 * 2 block-scaled 32x32x64 on E4M3, 3 block-scaled 16x16x128 on E4M3, 4 block-scaled 32x32x64 on
 * E2M1; 5 and 6: v_mfma_f32_32x32x16_f16 and v_mfma_f32_16x16x32_f16 on a 128 x 128 tile per
 * wavefront with the forward GEMM's dequantization interleaved (one FP4 -> fp16 conversion and
 * one packed multiply per two operand values, the same per flop for both), one wavefront per
 * SIMD only and an even iters (PMN_ESHAPE otherwise). *flops (host) receives the launch's
 * floating-point operations; time the launch on `stream` to get the rate. With one workgroup per
 * compute unit (workgroups = 256) the kernel runs exactly waves_per_simd wavefronts on every SIMD.
 */
int pmn_probe_mfma(int kind, int waves_per_simd, int workgroups, int iters, float* sink, double* flops,
                   pmn_stream_t stream);

/*
 * Verification of the activation quantizer's division-free reciprocal: adds to *mismatches (a
 * device counter the caller zeroes) the number of fp32 values d whose bit patterns lie in
 * [first_bits, last_bits] for which that reciprocal differs in any bit from the IEEE quotient
 * 1.0f / d. first_bits <= last_bits (PMN_ESHAPE).
 */
int pmn_probe_recip_check(uint32_t first_bits, uint32_t last_bits, unsigned long long* mismatches,
                          pmn_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PMN_PROBE_H */
