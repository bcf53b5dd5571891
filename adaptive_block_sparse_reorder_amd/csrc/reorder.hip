// Video-aware block organization (FVAttn page, section 3.1): token-major
// [B, N, Hh, d] <-> block order.  Pure data movement, bound by HBM bandwidth.
//
// Forward rows: each workgroup owns kRows consecutive reordered positions of
// one batch for every head.  The source token index of each position is
// computed once into LDS; the copy then walks (position, head, 16-byte chunk)
// with the chunk fastest, so that a wave reads whole contiguous token rows
// (all heads of a token are adjacent in the source) and writes whole 2*d-byte
// destination rows.
//
// Forward vt64: each workgroup owns one 64-token chunk of one head; rows are
// staged in LDS and written transposed (d-major, 128 contiguous bytes per
// channel), with the token slot's bits 2 and 3 swapped.
#include "fva_internal.hpp"

namespace fva {
namespace {

constexpr int kRows = 8;
constexpr int kThreads = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void reorder_rows_fwd(
    const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, BlockOrder bo, int64_t N,
    int64_t Npad, int Hh, int d, int64_t sb, int64_t sn, int64_t sh) {
  __shared__ int64_t tok[kRows];
  const int64_t r0 = (int64_t)blockIdx.x * kRows;
  const int b = blockIdx.y;
  if (threadIdx.x < kRows) {
    const int64_t r = r0 + threadIdx.x;
    tok[threadIdx.x] = r < N ? bo.src_token(r) : -1;
  }
  __syncthreads();
  const int cpr = d >> 3;  // 16-byte chunks per row
  const int total = kRows * Hh * cpr;
  for (int L = threadIdx.x; L < total; L += kThreads) {
    const int c = L % cpr;
    const int rh = L / cpr;
    const int h = rh % Hh;
    const int rl = rh / Hh;
    const int64_t r = r0 + rl;
    if (r >= Npad) continue;
    const int64_t n = tok[rl];
    u32x4 v = {0u, 0u, 0u, 0u};
    if (n >= 0) v = *(const u32x4*)(src + b * sb + n * sn + h * sh + c * 8);
    *(u32x4*)(dst + (((int64_t)b * Hh + h) * Npad + r) * d + c * 8) = v;
  }
}

__global__ __launch_bounds__(kThreads) void reorder_rows_inv(
    const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, BlockOrder bo, int64_t N,
    int64_t Npad, int Hh, int d, int64_t sb, int64_t sn, int64_t sh) {
  __shared__ int64_t tok[kRows];
  const int64_t r0 = (int64_t)blockIdx.x * kRows;
  const int b = blockIdx.y;
  if (threadIdx.x < kRows) {
    const int64_t r = r0 + threadIdx.x;
    tok[threadIdx.x] = r < N ? bo.src_token(r) : -1;
  }
  __syncthreads();
  const int cpr = d >> 3;
  const int total = kRows * Hh * cpr;
  for (int L = threadIdx.x; L < total; L += kThreads) {
    const int c = L % cpr;
    const int rh = L / cpr;
    const int h = rh % Hh;
    const int rl = rh / Hh;
    const int64_t n = tok[rl];
    if (n < 0) continue;
    const int64_t r = r0 + rl;
    const u32x4 v = *(const u32x4*)(src + (((int64_t)b * Hh + h) * Npad + r) * d + c * 8);
    *(u32x4*)(dst + b * sb + n * sn + h * sh + c * 8) = v;
  }
}

// slot of token offset k inside a 64-token vt64 chunk: bits 2 and 3 swapped
__device__ __forceinline__ int vt_slot(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

template <int D>
__global__ __launch_bounds__(kThreads) void reorder_vt64_fwd(
    const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, BlockOrder bo, int64_t N,
    int64_t Npad, int Hh, int64_t sb, int64_t sn, int64_t sh) {
  // stage[k][c], row padded by one 16-byte chunk against bank conflicts
  constexpr int kPitch = D + 8;
  __shared__ uint16_t stage[64 * kPitch];
  __shared__ int64_t tok[64];
  const int64_t chunk = blockIdx.x;  // 64-token chunk index within the head
  const int bh = blockIdx.y;
  const int b = bh / Hh, h = bh % Hh;
  const int64_t r0 = chunk * 64;
  if (threadIdx.x < 64) {
    const int64_t r = r0 + threadIdx.x;
    tok[threadIdx.x] = r < N ? bo.src_token(r) : -1;
  }
  __syncthreads();
  constexpr int cpr = D / 8;
  for (int L = threadIdx.x; L < 64 * cpr; L += kThreads) {
    const int c = L % cpr, k = L / cpr;
    const int64_t n = tok[k];
    u32x4 v = {0u, 0u, 0u, 0u};
    if (n >= 0) v = *(const u32x4*)(src + b * sb + n * sn + h * sh + c * 8);
    *(u32x4*)(&stage[k * kPitch + c * 8]) = v;
  }
  __syncthreads();
  // output: D rows (channels) x 64 slots; each thread writes 8 slots (16 B)
  uint16_t* out = dst + ((int64_t)bh * (Npad / 64) + chunk) * (int64_t)D * 64;
  for (int L = threadIdx.x; L < D * 8; L += kThreads) {
    const int sg = L % 8;    // slot group of 8
    const int c = L / 8;     // channel
    uint16_t vals[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int slot = sg * 8 + e;
      const int k = vt_slot(slot);  // the swap is an involution
      vals[e] = stage[k * kPitch + c];
    }
    u32x4 v;
    v.x = vals[0] | ((uint32_t)vals[1] << 16);
    v.y = vals[2] | ((uint32_t)vals[3] << 16);
    v.z = vals[4] | ((uint32_t)vals[5] << 16);
    v.w = vals[6] | ((uint32_t)vals[7] << 16);
    *(u32x4*)(out + c * 64 + sg * 8) = v;
  }
}

}  // namespace

fva_status launch_reorder(const Problem& p, const void* src, void* dst, const int64_t st[3],
                          int direction, int layout, hipStream_t s) {
  BlockOrder bo{p.T, p.H, p.W, p.bt, p.bh, p.bw};
  const uint16_t* in = (const uint16_t*)src;
  uint16_t* out = (uint16_t*)dst;
  if (direction == FVA_FORWARD && layout == FVA_LAYOUT_ROWS) {
    dim3 grid((unsigned)((p.Npad + kRows - 1) / kRows), (unsigned)p.B);
    hipLaunchKernelGGL(reorder_rows_fwd, grid, dim3(kThreads), 0, s, in, out, bo, p.N, p.Npad,
                       p.Hh, p.d, st[0], st[1], st[2]);
  } else if (direction == FVA_INVERSE) {
    dim3 grid((unsigned)((p.Npad + kRows - 1) / kRows), (unsigned)p.B);
    hipLaunchKernelGGL(reorder_rows_inv, grid, dim3(kThreads), 0, s, in, out, bo, p.N, p.Npad,
                       p.Hh, p.d, st[0], st[1], st[2]);
  } else {
    dim3 grid((unsigned)(p.Npad / 64), (unsigned)(p.B * p.Hh));
    if (p.d == 128)
      hipLaunchKernelGGL(reorder_vt64_fwd<128>, grid, dim3(kThreads), 0, s, in, out, bo, p.N,
                         p.Npad, p.Hh, st[0], st[1], st[2]);
    else
      hipLaunchKernelGGL(reorder_vt64_fwd<64>, grid, dim3(kThreads), 0, s, in, out, bo, p.N,
                         p.Npad, p.Hh, st[0], st[1], st[2]);
  }
  return hip_fail(hipGetLastError(), "reorder launch");
}

}  // namespace fva
