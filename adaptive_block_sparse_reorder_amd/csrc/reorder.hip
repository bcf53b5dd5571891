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
// Forward k64 / v64: each workgroup owns one 64-token chunk of one head and
// writes it in the tile layout the attention kernel stages into LDS verbatim.
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
  // four independent 16-byte loads in flight per thread; the inputs are read
  // once, so they are loaded non-temporally
  for (int L0 = threadIdx.x; L0 < total; L0 += 4 * kThreads) {
    u32x4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int L = L0 + j * kThreads;
      v[j] = u32x4{0u, 0u, 0u, 0u};
      if (L < total) {
        const int c = L % cpr, rh = L / cpr, h = rh % Hh, rl = rh / Hh;
        const int64_t n = tok[rl];
        if (n >= 0) v[j] = __builtin_nontemporal_load((const u32x4*)(src + b * sb + n * sn + h * sh + c * 8));
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int L = L0 + j * kThreads;
      if (L >= total) continue;
      const int c = L % cpr, rh = L / cpr, h = rh % Hh, rl = rh / Hh;
      const int64_t r = r0 + rl;
      if (r >= Npad) continue;
      *(u32x4*)(dst + (((int64_t)b * Hh + h) * Npad + r) * d + c * 8) = v[j];
    }
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
  // four loads in flight per thread, read non-temporally (read once)
  for (int L0 = threadIdx.x; L0 < total; L0 += 4 * kThreads) {
    u32x4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int L = min(L0 + j * kThreads, total - 1);
      const int c = L % cpr, rh = L / cpr, h = rh % Hh, rl = rh / Hh;
      v[j] = __builtin_nontemporal_load(
          (const u32x4*)(src + (((int64_t)b * Hh + h) * Npad + r0 + rl) * d + c * 8));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int L = L0 + j * kThreads;
      if (L >= total) continue;
      const int c = L % cpr, rh = L / cpr, h = rh % Hh, rl = rh / Hh;
      const int64_t n = tok[rl];
      if (n < 0) continue;
      *(u32x4*)(dst + b * sb + n * sn + h * sh + c * 8) = v[j];
    }
  }
}

// slot of token offset k inside a 64-token V chunk: bits 2 and 3 swapped
__device__ __forceinline__ int v_slot(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// Forward into one of the 64-token tile layouts.  The workgroup stages the
// chunk's 64 token rows of one head in LDS (rows padded by 16 bytes so the
// 16-byte column reads below are free of bank conflicts), then writes the
// 16 KB (d=128) tile in one contiguous, coalesced sweep.
//   K64: unit (c, r) = channels 8c..8c+7 of token r, at unit index c*64 + r
//   V64: unit (g, e) = channel e of the tokens in slots 8g..8g+7, at g*D + e
template <int D, bool IS_V>
__global__ __launch_bounds__(kThreads) void reorder_tile64_fwd(
    const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, BlockOrder bo, int64_t N,
    int64_t Npad, int Hh, int64_t sb, int64_t sn, int64_t sh) {
  constexpr int kPitch = D + 8;
  __shared__ __attribute__((aligned(16))) uint16_t stage[64 * kPitch];
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
  constexpr int kPer = 64 * cpr / kThreads;  // 16-byte loads per thread (4 at d=128)
  static_assert(kPer * kThreads == 64 * cpr, "chunk size");
  u32x4 lv[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int L = threadIdx.x + j * kThreads;
    const int c = L % cpr, k = L / cpr;
    const int64_t n = tok[k];
    lv[j] = u32x4{0u, 0u, 0u, 0u};
    if (n >= 0) lv[j] = __builtin_nontemporal_load((const u32x4*)(src + b * sb + n * sn + h * sh + c * 8));
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int L = threadIdx.x + j * kThreads;
    const int c = L % cpr, k = L / cpr;
    *(u32x4*)(&stage[k * kPitch + c * 8]) = lv[j];
  }
  __syncthreads();
  u32x4* out = (u32x4*)(dst + ((int64_t)bh * (Npad / 64) + chunk) * (int64_t)D * 64);
  for (int u = threadIdx.x; u < 64 * cpr; u += kThreads) {
    u32x4 v;
    if (!IS_V) {
      const int c = u / 64, r = u % 64;
      v = *(const u32x4*)(&stage[r * kPitch + c * 8]);
    } else {
      const int g = u / D, e = u % D;
      uint16_t vals[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) vals[q] = stage[v_slot(8 * g + q) * kPitch + e];
      v.x = vals[0] | ((uint32_t)vals[1] << 16);
      v.y = vals[2] | ((uint32_t)vals[3] << 16);
      v.z = vals[4] | ((uint32_t)vals[5] << 16);
      v.w = vals[6] | ((uint32_t)vals[7] << 16);
    }
    out[u] = v;
  }
}

// 3-D Hilbert index of cell (x0, x1, x2) on a 2^bits cube, by Skilling's
// transpose method ("Programming the Hilbert curve", AIP Conf. Proc. 707,
// 2004): undo excess work from the top bit down, Gray-encode, then read the
// index off the transposed form by interleaving bits (x0 most significant).
__device__ uint64_t hilbert3(uint32_t x0, uint32_t x1, uint32_t x2, int bits) {
  uint32_t X[3] = {x0, x1, x2};
  const uint32_t M = 1u << (bits - 1);
  for (uint32_t Q = M; Q > 1; Q >>= 1) {
    const uint32_t P = Q - 1;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      if (X[i] & Q) {
        X[0] ^= P;
      } else {
        const uint32_t t = (X[0] ^ X[i]) & P;
        X[0] ^= t;
        X[i] ^= t;
      }
    }
  }
  X[1] ^= X[0];
  X[2] ^= X[1];
  uint32_t t = 0;
  for (uint32_t Q = M; Q > 1; Q >>= 1)
    if (X[2] & Q) t ^= Q - 1;
  X[0] ^= t;
  X[1] ^= t;
  X[2] ^= t;
  uint64_t h = 0;
  for (int j = bits - 1; j >= 0; --j)
#pragma unroll
    for (int i = 0; i < 3; ++i) h = (h << 1) | ((X[i] >> j) & 1u);
  return h;
}

// One workgroup: order the tiles (raster or Hilbert over tile coordinates
// (tile-frame, tile-row, tile-column) on the bounding 2^m cube, out-of-grid
// cells skipped), then prefix-sum the clipped tile sizes into start[].
constexpr int kOrderThreads = 1024;

__global__ __launch_bounds__(kOrderThreads) void tile_order_kernel(BlockOrder g, int order,
                                                                   int64_t N, int32_t* table) {
  __shared__ uint64_t keys[kMaxTiles];
  __shared__ int32_t wsum[kOrderThreads / 64];
  const int nt = (g.T + g.bt - 1) / g.bt, ny = (g.H + g.bh - 1) / g.bh, nx = (g.W + g.bw - 1) / g.bw;
  const int ntiles = nt * ny * nx;
  int P = 1;
  while (P < ntiles) P <<= 1;
  int bits = 1;
  while ((1 << bits) < max(nt, max(ny, nx))) ++bits;
  for (int i = threadIdx.x; i < P; i += kOrderThreads) {
    uint64_t key = ~0ull;
    if (i < ntiles) {
      const uint32_t tt = i / (ny * nx), ty = (i / nx) % ny, tx = i % nx;
      const uint64_t h = order == FVA_ORDER_HILBERT ? hilbert3(tt, ty, tx, bits) : (uint64_t)i;
      key = (h << 13) | (uint64_t)i;
    }
    keys[i] = key;
  }
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int q = threadIdx.x; q < P / 2; q += kOrderThreads) {
        const int i = 2 * j * (q / j) + (q % j), l = i + j;
        const uint64_t a = keys[i], b = keys[l];
        if ((a > b) == ((i & k) == 0)) { keys[i] = b; keys[l] = a; }
      }
      __syncthreads();
    }
  int32_t* tile_id = table + 4;
  int32_t* start = tile_id + ntiles;
  // each thread owns a contiguous run of tiles; exclusive scan of their sizes
  const int per = (ntiles + kOrderThreads - 1) / kOrderThreads;
  const int k0 = threadIdx.x * per;
  int local = 0;
  for (int k = k0; k < min(ntiles, k0 + per); ++k) {
    const int id = (int)(keys[k] & 8191u);
    tile_id[k] = id;
    const int tt = id / (ny * nx), ty = (id / nx) % ny, tx = id % nx;
    local += min(g.bt, g.T - tt * g.bt) * min(g.bh, g.H - ty * g.bh) * min(g.bw, g.W - tx * g.bw);
  }
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  int x = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int run = x - local;
  for (int w = 0; w < wave; ++w) run += wsum[w];
  for (int k = k0; k < min(ntiles, k0 + per); ++k) {
    start[k] = run;
    const int id = tile_id[k];
    const int tt = id / (ny * nx), ty = (id / nx) % ny, tx = id % nx;
    run += min(g.bt, g.T - tt * g.bt) * min(g.bh, g.H - ty * g.bh) * min(g.bw, g.W - tx * g.bw);
  }
  if (threadIdx.x == 0) {
    start[ntiles] = (int32_t)N;
    table[0] = ntiles;
    table[1] = order;
    table[2] = 0;
    table[3] = 0;
  }
}

}  // namespace

int64_t tile_count(const Problem& p) {
  return (int64_t)((p.T + p.bt - 1) / p.bt) * ((p.H + p.bh - 1) / p.bh) * ((p.W + p.bw - 1) / p.bw);
}

fva_status launch_tile_order(const Problem& p, int order, int32_t* table, hipStream_t s) {
  BlockOrder g{p.T, p.H, p.W, p.bt, p.bh, p.bw, nullptr, nullptr, 0};
  hipLaunchKernelGGL(tile_order_kernel, dim3(1), dim3(kOrderThreads), 0, s, g, order, p.N, table);
  return hip_fail(hipGetLastError(), "tile order launch");
}

fva_status launch_reorder(const Problem& p, const void* src, void* dst, const int64_t st[3],
                          int direction, int layout, const int32_t* table, hipStream_t s) {
  BlockOrder bo{p.T, p.H, p.W, p.bt, p.bh, p.bw, nullptr, nullptr, 0};
  if (table) {
    const int64_t nt = tile_count(p);
    bo.tile_id = table + 4;
    bo.start = table + 4 + nt;
    bo.ntiles = (int32_t)nt;
  }
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
    const bool v = layout == FVA_LAYOUT_V64;
#define FVA_TILE_LAUNCH(DD, VV)                                                               \
  hipLaunchKernelGGL((reorder_tile64_fwd<DD, VV>), grid, dim3(kThreads), 0, s, in, out, bo, p.N, \
                     p.Npad, p.Hh, st[0], st[1], st[2])
    if (p.d == 128) {
      if (v) FVA_TILE_LAUNCH(128, true);
      else FVA_TILE_LAUNCH(128, false);
    } else {
      if (v) FVA_TILE_LAUNCH(64, true);
      else FVA_TILE_LAUNCH(64, false);
    }
#undef FVA_TILE_LAUNCH
  }
  return hip_fail(hipGetLastError(), "reorder launch");
}

}  // namespace fva
