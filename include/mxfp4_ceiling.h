/*
 * mxfp4_ceiling.h -- C ABI of libmxfp4_ceiling.so: practical ceilings of the MI355X (gfx950)
 * for the two bounds of libmxfp4.so's kernels, measured with plain kernels of known work, so
 * that a kernel's throughput can be stated against what the board sustains as well as against
 * its published peaks (HBM 8 TB/s; dense MXFP4 matrix cores 10.1 PFLOP/s).
 *
 * No passage of the method defines these operations. They measure the machine for the method's
 * two kinds of kernel: the quantizers stream an operand from HBM once and write codes and
 * scales; the GEMMs run the block-scaled FP4 matrix product (gist.science summary of "MXFP4
 * LLM pretraining", section 방법론: all three GEMMs of a linear layer in MXFP4).
 *
 * Conventions: pointers are DEVICE pointers owned by the caller; `stream` is a hipStream_t
 * passed as void* (NULL = the default stream); each call enqueues one kernel and returns at
 * once. Return value: 0 on success, 1 for a NULL pointer, 2 for a size outside the stated range
 * or a misaligned pointer (nothing is launched), 3 when the launch fails.
 */
#ifndef MXFP4_CEILING_H_
#define MXFP4_CEILING_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read of src[0, bytes), every byte once, with 16-byte nontemporal loads.
 * bytes: a positive multiple of 16; src 16-byte aligned. sink: one 32-bit word that a lane
 * overwrites only when the XOR of the words it read equals `never` (this store keeps the loads
 * alive; its value means nothing). */
int mxfp4_ceiling_read(const void *src, size_t bytes, uint32_t never, uint32_t *sink, void *stream);

/* Streaming write: every 32-bit word of dst[0, bytes) = pattern, with 16-byte stores.
 * bytes: a positive multiple of 16; dst 16-byte aligned. */
int mxfp4_ceiling_write(void *dst, size_t bytes, uint32_t pattern, void *stream);

/* Streaming copy dst[0, bytes) = src[0, bytes), 16-byte nontemporal loads and stores; the
 * ranges must not overlap. bytes: a positive multiple of 16; both pointers 16-byte aligned. */
int mxfp4_ceiling_copy(const void *src, void *dst, size_t bytes, void *stream);

/* Scaled FP4 matrix-core loop: `workgroups` workgroups of 8 wavefronts (at most one per
 * compute unit, two wavefronts per SIMD, as the GEMM runs); each wavefront issues `iters`
 * rounds of 8 independent v_mfma_scale_f32_32x32x64_f8f6f4 (E2M1 x E2M1 with E8M0 scales) on
 * register-resident operands whose bits change every round (random patterns seeded by `seed`,
 * as a GEMM's operands change). FLOPs = workgroups * 8 * iters * 8 * (2 * 32 * 32 * 64).
 * sink: workgroups * 512 floats, each lane's sum of its accumulators (finite).
 * workgroups in [1, 65536], iters in [1, 1 << 20]. */
int mxfp4_ceiling_mfma(int workgroups, int iters, uint32_t seed, float *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_CEILING_H_ */
