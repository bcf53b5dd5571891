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

// Reordered position r (< N) -> source token index.  Tokens inside a tile
// are always visited in raster order (t, y, x).  Tiles are visited either in
// raster order (closed form: every tile-frame slab covers whole frames and
// every tile row inside a slab covers whole rows, so the tile containing r
// follows from three divisions) or in the order of a tile table (tile_id[k],
// start[k] = first reordered position of the k-th tile), found by binary
// search.  A table lookup is bounded: it returns -1 (and raises the table's
// status word) when the table's header names another grid or an entry does
// not describe a tile of this grid, and it never indexes past the table.
struct BlockOrder {
  int32_t T, H, W, bt, bh, bw;
  int32_t* table;          // null: raster tile order
  int32_t ntiles;          // tiles of this grid
  __device__ __forceinline__ int64_t src_token(int64_t r) const {
    if (table) return src_token_table(r);
    const int64_t HW = (int64_t)H * W;
    const int64_t slab = (int64_t)bt * HW;
    const int32_t tt = (int32_t)(r / slab);
    int64_t r1 = r - (int64_t)tt * slab;
    const int32_t st = min(bt, T - tt * bt);
    const int64_t rowband = (int64_t)st * bh * W;
    const int32_t ty = (int32_t)(r1 / rowband);
    int64_t r2 = r1 - (int64_t)ty * rowband;
    const int32_t sy = min(bh, H - ty * bh);
    const int32_t tilesz = st * sy * bw;
    const int32_t tx = (int32_t)(r2 / tilesz);
    const int32_t r3 = (int32_t)(r2 - (int64_t)tx * tilesz);
    const int32_t sx = min(bw, W - tx * bw);
    const int32_t t = r3 / (sy * sx);
    const int32_t rem = r3 - t * (sy * sx);
    const int32_t y = rem / sx;
    const int32_t x = rem - y * sx;
    return ((int64_t)(tt * bt + t) * H + (ty * bh + y)) * W + (tx * bw + x);
  }
  __device__ __forceinline__ bool header_matches() const {
    const int32_t* h = table;
    return h[0] == ntiles && h[3] == T && h[4] == H && h[5] == W && h[6] == bt && h[7] == bh &&
           h[8] == bw;
  }
  __device__ int64_t src_token_table(int64_t r) const {
    if (!header_matches()) return bad();
    const int32_t* tile_id = table + kTableHeaderWords;
    const int32_t* start = tile_id + ntiles;
    int lo = 0, hi = ntiles;  // start[lo] <= r < start[hi] for a well-formed table
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)start[mid] <= r) lo = mid;
      else hi = mid;
    }
    const int32_t nty = (H + bh - 1) / bh, ntx = (W + bw - 1) / bw;
    const int32_t id = tile_id[lo];
    if (id < 0 || id >= ntiles) return bad();
    const int32_t tt = id / (nty * ntx), ty = (id / ntx) % nty, tx = id % ntx;
    const int32_t st = min(bt, T - tt * bt), sy = min(bh, H - ty * bh), sx = min(bw, W - tx * bw);
    const int64_t o64 = r - (int64_t)start[lo];
    if (o64 < 0 || o64 >= (int64_t)st * sy * sx) return bad();
    const int32_t o = (int32_t)o64;
    const int32_t t = o / (sy * sx);
    const int32_t rem = o - t * (sy * sx);
    const int32_t y = rem / sx;
    const int32_t x = rem - y * sx;
    return ((int64_t)(tt * bt + t) * H + (ty * bh + y)) * W + (tx * bw + x);
  }
  __device__ int64_t bad() const {
    atomicOr(table + 2, 1);
    return -1;
  }
};

constexpr int kRows = 8;
constexpr int kThreads = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

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

// Forward rows that also write each block's mean over its real tokens (the
// pooled block representative of section 3.1's routing, in float32).  One
// workgroup per (block, group of kPoolHeads heads, batch): the block's source
// token indices go to LDS once; thread (position class, head, 16-byte chunk)
// copies positions p = class, class + PP, ... with the chunk fastest (a wave
// reads whole 2*d-byte source rows and writes whole 2*d-byte rows) and sums
// the real ones into eight float32 lanes; the PP position classes are then
// added in class order.  One head per workgroup (many small workgroups, all
// of a thread's rows loaded at once) measured 10 % faster at 720p than eight.
constexpr int kPoolHeads = 1;

template <int D>
__global__ __launch_bounds__(kThreads) void reorder_rows_pool_fwd(
    const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, float* __restrict__ pooled,
    BlockOrder bo, int64_t N, int64_t Npad, int Hh, int BLK, int nB, int64_t sb, int64_t sn,
    int64_t sh) {
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int UNITS = kPoolHeads * CPR;    // (head, chunk) units per position
  constexpr int PP = kThreads / UNITS;       // position classes: 2 (d=128) or 4 (d=64)
  constexpr int U = 16;                      // loads in flight per thread (at most)
  __shared__ int64_t tok[128];
  __shared__ float part[PP][kPoolHeads * D];
  const int blk = blockIdx.x, h0 = blockIdx.y * kPoolHeads, b = blockIdx.z;
  const int64_t r0 = (int64_t)blk * BLK;
  const int nreal = (int)min((int64_t)BLK, N - r0);
  for (int i = threadIdx.x; i < BLK; i += kThreads) tok[i] = i < nreal ? bo.src_token(r0 + i) : -1;
  __syncthreads();
  const int u = threadIdx.x % UNITS, cls = threadIdx.x / UNITS;
  const int hl = u / CPR, c = u % CPR, h = h0 + hl;
  const bool live = h < Hh;
  const uint16_t* sp = src + b * sb + (int64_t)min(h, Hh - 1) * sh + c * 8;
  uint16_t* dp = dst + (((int64_t)b * Hh + min(h, Hh - 1)) * Npad + r0) * D + c * 8;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int p0 = cls; p0 < BLK; p0 += PP * U) {
    u32x4 v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int pos = p0 + j * PP;
      v[j] = u32x4{0u, 0u, 0u, 0u};
      if (live && pos < BLK) {
        const int64_t n = tok[pos];
        if (n >= 0) v[j] = __builtin_nontemporal_load((const u32x4*)(sp + n * sn));
      }
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int pos = p0 + j * PP;
      if (!live || pos >= BLK) continue;
      *(u32x4*)(dp + (int64_t)pos * D) = v[j];
      if (pos < nreal) {
        acc[0] += bf16_lo(v[j].x); acc[1] += bf16_hi(v[j].x);
        acc[2] += bf16_lo(v[j].y); acc[3] += bf16_hi(v[j].y);
        acc[4] += bf16_lo(v[j].z); acc[5] += bf16_hi(v[j].z);
        acc[6] += bf16_lo(v[j].w); acc[7] += bf16_hi(v[j].w);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[cls][u * 8 + e] = acc[e];
  __syncthreads();
  for (int o = threadIdx.x; o < kPoolHeads * D; o += kThreads) {
    const int hh = h0 + o / D;
    if (hh >= Hh) continue;
    float sum = part[0][o];
#pragma unroll
    for (int q = 1; q < PP; ++q) sum += part[q][o];
    pooled[(((int64_t)b * Hh + hh) * nB + blk) * D + (o % D)] = sum / (float)nreal;
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
// With POOL the workgroup owns a whole block (BLK/64 chunks, one after the
// other) and also writes the block's mean over its real tokens: each thread
// sums the rows it loaded (pad rows load as zero and are not added), then the
// threads of one chunk column are added by shuffles and the four waves
// through LDS, in a fixed order.
template <int D, bool IS_V, bool POOL>
__global__ __launch_bounds__(kThreads) void reorder_tile64_fwd(
    const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, float* __restrict__ pooled,
    BlockOrder bo, int64_t N, int64_t Npad, int Hh, int BLK, int nB, int64_t sb, int64_t sn,
    int64_t sh) {
  static_assert(!(IS_V && POOL), "pooling is for the K layout");
  constexpr int kPitch = D + 8;
  __shared__ __attribute__((aligned(16))) uint16_t stage[64 * kPitch];
  __shared__ int64_t tok[64];
  __shared__ float part[POOL ? 4 : 1][POOL ? D : 1];
  const int bh = blockIdx.y;
  const int b = bh / Hh, h = bh % Hh;
  const int chunks = POOL ? BLK / 64 : 1;
  constexpr int cpr = D / 8;
  constexpr int kPer = 64 * cpr / kThreads;  // 16-byte loads per thread (4 at d=128)
  static_assert(kPer * kThreads == 64 * cpr, "chunk size");
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int q = 0; q < chunks; ++q) {
    const int64_t chunk = (int64_t)blockIdx.x * chunks + q;  // 64-token chunk within the head
    const int64_t r0 = chunk * 64;
    if (q > 0) __syncthreads();  // the previous chunk's LDS reads are done
    if (threadIdx.x < 64) {
      const int64_t r = r0 + threadIdx.x;
      tok[threadIdx.x] = r < N ? bo.src_token(r) : -1;
    }
    __syncthreads();
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
      if (POOL && r0 + k < N) {
        acc[0] += bf16_lo(lv[j].x); acc[1] += bf16_hi(lv[j].x);
        acc[2] += bf16_lo(lv[j].y); acc[3] += bf16_hi(lv[j].y);
        acc[4] += bf16_lo(lv[j].z); acc[5] += bf16_hi(lv[j].z);
        acc[6] += bf16_lo(lv[j].w); acc[7] += bf16_hi(lv[j].w);
      }
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
        for (int qq = 0; qq < 8; ++qq) vals[qq] = stage[v_slot(8 * g + qq) * kPitch + e];
        v.x = vals[0] | ((uint32_t)vals[1] << 16);
        v.y = vals[2] | ((uint32_t)vals[3] << 16);
        v.z = vals[4] | ((uint32_t)vals[5] << 16);
        v.w = vals[6] | ((uint32_t)vals[7] << 16);
      }
      out[u] = v;
    }
  }
  if (POOL) {
    // lanes l, l ^ cpr, l ^ 2cpr, ... of a wave hold the same channel chunk
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
#pragma unroll
    for (int off = cpr; off < 64; off <<= 1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], off, 64);
    }
    if (lane < cpr) {
#pragma unroll
      for (int e = 0; e < 8; ++e) part[wave][lane * 8 + e] = acc[e];
    }
    __syncthreads();
    if (threadIdx.x < D) {
      const int64_t rb = (int64_t)blockIdx.x * BLK;
      const int nreal = (int)min((int64_t)BLK, N - rb);
      const float sum = (part[0][threadIdx.x] + part[1][threadIdx.x]) +
                        (part[2][threadIdx.x] + part[3][threadIdx.x]);
      pooled[((int64_t)bh * nB + blockIdx.x) * D + threadIdx.x] = sum / (float)nreal;
    }
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
  int32_t* tile_id = table + kTableHeaderWords;
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
    const int32_t hdr[kTableHeaderWords] = {ntiles, order, 0, g.T, g.H, g.W, g.bt, g.bh, g.bw,
                                            0, 0, 0};
    for (int w = 0; w < kTableHeaderWords; ++w) table[w] = hdr[w];
  }
}

}  // namespace

int64_t tile_count(const Problem& p) {
  return (int64_t)((p.T + p.bt - 1) / p.bt) * ((p.H + p.bh - 1) / p.bh) * ((p.W + p.bw - 1) / p.bw);
}

fva_status launch_tile_order(const Problem& p, int order, int32_t* table, hipStream_t s) {
  BlockOrder g{p.T, p.H, p.W, p.bt, p.bh, p.bw, nullptr, 0};
  hipLaunchKernelGGL(tile_order_kernel, dim3(1), dim3(kOrderThreads), 0, s, g, order, p.N, table);
  return hip_fail(hipGetLastError(), "tile order launch");
}

fva_status launch_reorder(const Problem& p, const void* src, void* dst, const int64_t st[3],
                          int direction, int layout, int32_t* table, hipStream_t s) {
  BlockOrder bo{p.T, p.H, p.W, p.bt, p.bh, p.bw, table, (int32_t)tile_count(p)};
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
#define FVA_TILE_LAUNCH(DD, VV)                                                                 \
  hipLaunchKernelGGL((reorder_tile64_fwd<DD, VV, false>), grid, dim3(kThreads), 0, s, in, out,  \
                     nullptr, bo, p.N, p.Npad, p.Hh, p.BLK, p.nB, st[0], st[1], st[2])
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

fva_status launch_reorder_pool(const Problem& p, const void* src, void* dst, float* pooled,
                               const int64_t st[3], int layout, int32_t* table, hipStream_t s) {
  BlockOrder bo{p.T, p.H, p.W, p.bt, p.bh, p.bw, table, (int32_t)tile_count(p)};
  const uint16_t* in = (const uint16_t*)src;
  uint16_t* out = (uint16_t*)dst;
  if (layout == FVA_LAYOUT_ROWS) {
    dim3 grid((unsigned)p.nB, (unsigned)((p.Hh + kPoolHeads - 1) / kPoolHeads), (unsigned)p.B);
    if (p.d == 128)
      hipLaunchKernelGGL(reorder_rows_pool_fwd<128>, grid, dim3(kThreads), 0, s, in, out, pooled,
                         bo, p.N, p.Npad, p.Hh, p.BLK, p.nB, st[0], st[1], st[2]);
    else
      hipLaunchKernelGGL(reorder_rows_pool_fwd<64>, grid, dim3(kThreads), 0, s, in, out, pooled,
                         bo, p.N, p.Npad, p.Hh, p.BLK, p.nB, st[0], st[1], st[2]);
  } else {
    dim3 grid((unsigned)p.nB, (unsigned)(p.B * p.Hh));
    if (p.d == 128)
      hipLaunchKernelGGL((reorder_tile64_fwd<128, false, true>), grid, dim3(kThreads), 0, s, in,
                         out, pooled, bo, p.N, p.Npad, p.Hh, p.BLK, p.nB, st[0], st[1], st[2]);
    else
      hipLaunchKernelGGL((reorder_tile64_fwd<64, false, true>), grid, dim3(kThreads), 0, s, in,
                         out, pooled, bo, p.N, p.Npad, p.Hh, p.BLK, p.nB, st[0], st[1], st[2]);
  }
  return hip_fail(hipGetLastError(), "reorder with pooling launch");
}

}  // namespace fva
