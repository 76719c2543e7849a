/*
 * kda_probe.h -- C ABI of libkda_probe: measured ceilings of the machine that
 * libkda's kernels are compared against.
 *
 * The roofline of each kernel in libkda is priced twice: against the chip's
 * published peaks (HBM 8 TB/s, dense bf16 matrix 2.5 PFLOP/s) and against
 * what plain hand-written kernels reach on the same GPU in the same process.
 * This library holds those plain kernels: streaming HBM copies in the access
 * patterns of libkda's paths (read + write of separate buffers, in-place
 * read-modify-write as the decode pool update does, read-only, write-only)
 * and a loop of independent bf16 matrix-core products.  None of them is part
 * of the method; they exist only to be timed.
 *
 * Conventions: every pointer is a DEVICE pointer owned by the caller, 16-byte
 * aligned; `stream` is a hipStream_t passed as void* (NULL = null stream).
 * Nothing is allocated, nothing is synchronised, a return of 0 means
 * "enqueued".  Return codes: 0 OK, 1 invalid argument (nothing enqueued),
 * 3 launch refused by the HIP runtime.
 */
#ifndef KDA_PROBE_H_
#define KDA_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming access over `bytes` bytes (a multiple of 64).
 *   mode 0 (copy):  dst[i] = src[i]            -- bytes read + bytes written
 *   mode 1 (rmw):   dst[i] = 0.5f * dst[i] + 1 -- in place; src unused (may be NULL)
 *   mode 2 (read):  sums src as fp32, one partial sum per 16 KiB of src to
 *                   dst[0 .. ceil(bytes / 16384) - 1]; traffic = bytes read
 *   mode 3 (write): dst[i] = 1.0f              -- src unused (may be NULL)
 * src and dst must not overlap (mode 0).  One workgroup of 1024 threads per
 * 16 KiB, one non-temporal 16-byte access per thread and direction. */
int kda_probe_hbm(int mode, const void* src, void* dst, size_t bytes, void* stream);

/* Dense bf16 matrix-core loop: `blocks` workgroups of 256 threads (four
 * waves), each wave issuing `iters` rounds of eight independent products:
 *   shape 0: eight v_mfma_f32_32x32x16_bf16 (32768 flops each) per round,
 *            262144 flops per wave and round;
 *   shape 1: eight v_mfma_f32_16x16x32_bf16 (16384 flops each) per round,
 *            131072 flops per wave and round.
 * The total work is blocks * 4 * iters times that.  One fp32 per wave (the
 * sum over its lanes of every accumulator entry) goes to out[0 .. 4 * blocks
 * - 1], so that no product is dead code.  blocks in [1, 65536], iters in [1, 1 << 24]. */
int kda_probe_mfma_bf16(int shape, int32_t blocks, int32_t iters, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_PROBE_H_ */
