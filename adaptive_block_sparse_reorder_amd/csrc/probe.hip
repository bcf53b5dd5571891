// Matrix-core-only probe for the benchmark (declared in fva_probe.h): how
// many bf16 MFMA FLOP/s this card sustains when nothing else runs, on given
// operand bits.  Data-dependent switching power, not the issue rate, sets the
// clock the matrix cores hold, so the rate on random operands is the
// practical ceiling the attention kernel is read against.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fva_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(FVA_PROBE_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void probe_mfma_kernel(const u32x4* __restrict__ operands, float* __restrict__ out, int iters) {
  const int64_t g = (int64_t)blockIdx.x * FVA_PROBE_THREADS + threadIdx.x;
  const bf16x8 a = __builtin_bit_cast(bf16x8, operands[2 * g]);
  const bf16x8 b = __builtin_bit_cast(bf16x8, operands[2 * g + 1]);
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += (c0[r] + c1[r]) + (c2[r] + c3[r]);
  out[g] = s;
}

}  // namespace

extern "C" {

size_t fva_probe_operand_bytes(int32_t blocks) {
  return blocks > 0 ? (size_t)blocks * FVA_PROBE_THREADS * 32 : 0;
}

size_t fva_probe_output_bytes(int32_t blocks) {
  return blocks > 0 ? (size_t)blocks * FVA_PROBE_THREADS * 4 : 0;
}

int32_t fva_probe_mfma(const void* operands, void* out, int32_t blocks, int32_t iters,
                       hipStream_t stream) {
  if (!operands || !out || blocks <= 0 || iters <= 0) return -1;
  if (((uintptr_t)operands & 15u) != 0 || ((uintptr_t)out & 3u) != 0) return -1;
  hipLaunchKernelGGL(probe_mfma_kernel, dim3((unsigned)blocks), dim3(FVA_PROBE_THREADS), 0, stream,
                     (const u32x4*)operands, (float*)out, iters);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
