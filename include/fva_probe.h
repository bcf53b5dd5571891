/*
 * fva_probe.h - measurement kernels of libfva_probe.so, used by bench.py to
 * read the attention kernel's rate against what the matrix cores of this
 * MI355X sustain on their own.  Not part of the attention path or its ABI
 * (include/fva.h).
 */
#ifndef FVA_PROBE_H
#define FVA_PROBE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Threads the MFMA probe launches per workgroup and workgroups per CU. */
#define FVA_PROBE_THREADS 512
#define FVA_PROBE_BLOCKS_PER_CU 1

/* Bytes of the operand buffer and of the output buffer fva_probe_mfma needs
 * for `blocks` workgroups.                                                  */
size_t fva_probe_operand_bytes(int32_t blocks);
size_t fva_probe_output_bytes(int32_t blocks);

/* Matrix-core-only steady state: `blocks` workgroups of FVA_PROBE_THREADS
 * threads (two waves per SIMD when blocks = one per CU), each wave issuing
 * `iters` rounds of four independent v_mfma_f32_32x32x16_bf16 products on
 * operands read once from `operands` (DEVICE, fva_probe_operand_bytes bytes:
 * per lane eight 32-bit words, A then B, as bf16 pairs).  No other memory
 * traffic; each thread writes one float of its accumulators to `out`
 * (DEVICE, fva_probe_output_bytes bytes) so the products are kept.  Work:
 * blocks * FVA_PROBE_THREADS / 64 * iters * 4 * 32768 flop.  Returns 0, or
 * -1 for bad arguments (nothing launched), -4 when the launch fails.       */
int32_t fva_probe_mfma(const void* operands, void* out, int32_t blocks, int32_t iters,
                       hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* FVA_PROBE_H */
