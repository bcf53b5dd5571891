// Sparse-routing frontend (FVAttn page, sections 2 and 3.1; top-up: section
// 3.3): block mean-pooling of Q and K, pooled block scores, the Top-p CDF cut
// with a Top-k floor, mask materialization (bitmask, per-row counts, ascending
// column lists, per-head workload), the optional per-head top-up, and the
// heaviest-first work queue.
#include "fva_internal.hpp"

namespace fva {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Monotone map float32 -> uint32 (larger float -> larger key); -0 == +0.
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u & 0x7fffffffu) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float order_key_inv(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

__global__ void zero_route_state(int32_t* head_count, int nheads, uint32_t* flags) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nheads) head_count[i] = 0;
  if (i == 0) *flags = 0u;
}

// ------------------------------------------------------------------ pooling
// grid (nB, B*Hh, 2 [q|k]); 256 threads.  Thread = (row group, 16-byte channel
// chunk) for both Q (rows layout) and K (k64 tile layout, where a wave's four
// row groups read four consecutive 16-byte units of each chunk); the row
// groups of a wave are reduced with two (d=128) or three (d=64) shuffles, the
// four waves through LDS.
template <int D>
__global__ __launch_bounds__(256) void pool_kernel(const uint16_t* __restrict__ qr,
                                                   const uint16_t* __restrict__ kr,
                                                   float* __restrict__ qbar,
                                                   float* __restrict__ kbar, int64_t N,
                                                   int64_t Npad, int BLK, int nB) {
  constexpr int CPR = D / 8;           // chunks per row
  constexpr int RG = 256 / CPR;        // row groups
  __shared__ float part[4][D];
  const int blk = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int nreal = (int)min((int64_t)BLK, N - (int64_t)blk * BLK);
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  // thread -> 16-byte chunk c of rows rg, rg+RG, ...; Q rows are token-major,
  // K is in k64 tiles (unit (c, r) of a 64-token tile at (c*64 + r)*16 bytes)
  const bool is_k = blockIdx.z != 0;
  const uint16_t* x = (is_k ? kr : qr) + (bh * Npad + (int64_t)blk * BLK) * D;
  const int c = threadIdx.x % CPR;
  const int rg = threadIdx.x / CPR;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  // all of a thread's rows (at most 128 / RG) are loaded before any is summed,
  // so the loads are in flight together.  Rows past the block's real tokens
  // load the last real row (always in bounds) and are not summed, so the sums
  // are those of the real rows in row order.
  constexpr int MAXR = 128 / RG;
  u32x4 v[MAXR];
#pragma unroll
  for (int i = 0; i < MAXR; ++i) {
    const int r = min(rg + i * RG, nreal - 1);
    const int64_t unit = is_k ? (int64_t)(r >> 6) * 64 * CPR + c * 64 + (r & 63)
                              : (int64_t)r * CPR + c;
    v[i] = __builtin_nontemporal_load((const u32x4*)(x + unit * 8));
  }
#pragma unroll
  for (int i = 0; i < MAXR; ++i) {
    if (rg + i * RG < nreal) {
      acc[0] += bf16_lo(v[i].x); acc[1] += bf16_hi(v[i].x);
      acc[2] += bf16_lo(v[i].y); acc[3] += bf16_hi(v[i].y);
      acc[4] += bf16_lo(v[i].z); acc[5] += bf16_hi(v[i].z);
      acc[6] += bf16_lo(v[i].w); acc[7] += bf16_hi(v[i].w);
    }
  }
  // reduce the row groups of this wave (lanes that share a chunk), then across waves
#pragma unroll
  for (int off = CPR; off < 64; off <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], off, 64);
  }
  if (lane < CPR) {
#pragma unroll
    for (int e = 0; e < 8; ++e) part[wave][c * 8 + e] = acc[e];
  }
  __syncthreads();
  if (threadIdx.x < D) {
    const float sum = (part[0][threadIdx.x] + part[1][threadIdx.x]) +
                      (part[2][threadIdx.x] + part[3][threadIdx.x]);
    (is_k ? kbar : qbar)[(bh * nB + blk) * D + threadIdx.x] = sum / (float)nreal;
  }
}

// ------------------------------------------------------------------ scores
// S[bh, i, j] = scale * sum_c qbar[bh, i, c] * kbar[bh, j, c]; 64x64 tiles.
template <int D>
__global__ __launch_bounds__(256) void score_kernel(const float* __restrict__ qbar,
                                                    const float* __restrict__ kbar,
                                                    float* __restrict__ S, int nB, float scale) {
  constexpr int KC = 32;
  __shared__ float qs[64][KC + 1];
  __shared__ float ks[64][KC + 1];
  const int64_t bh = blockIdx.z;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  const float* qb = qbar + bh * nB * D;
  const float* kb = kbar + bh * nB * D;
  float acc[4][4] = {};
  for (int c0 = 0; c0 < D; c0 += KC) {
    for (int L = threadIdx.x; L < 64 * KC; L += 256) {
      const int r = L / KC, c = L % KC;
      qs[r][c] = (i0 + r < nB) ? qb[(int64_t)(i0 + r) * D + c0 + c] : 0.f;
      ks[r][c] = (j0 + r < nB) ? kb[(int64_t)(j0 + r) * D + c0 + c] : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int c = 0; c < KC; ++c) {
      float a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) { a[u] = qs[ty + 16 * u][c]; b[u] = ks[tx + 16 * u][c]; }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fmaf(a[u], b[v], acc[u][v]);
    }
    __syncthreads();
  }
  float* Sb = S + bh * (int64_t)nB * nB;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = i0 + ty + 16 * u, j = j0 + tx + 16 * v;
      if (i < nB && j < nB) Sb[(int64_t)i * nB + j] = acc[u][v] * scale;
    }
}

// ------------------------------------------------------------------ block helpers

template <int NT>
__device__ int block_sum_i32(int v, int* red) {
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  int t = 0;
  for (int w = 0; w < NT / 64; ++w) t += red[w];
  __syncthreads();
  return t;
}

// Bitonic sort (ascending) of P keys in LDS by NT threads.
template <typename K, int NT>
__device__ void bitonic_sort(K* keys, int P) {
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int q = threadIdx.x; q < P / 2; q += NT) {
        const int i = 2 * j * (q / j) + (q % j);
        const int l = i + j;
        const K a = keys[i], b = keys[l];
        const bool up = (i & k) == 0;
        if ((a > b) == up) { keys[i] = b; keys[l] = a; }
      }
      __syncthreads();
    }
  }
}

// Writes bitmask words, and the ascending column list, of one row from the
// LDS bitmask `bits` (words entries).  Returns nothing; col_idx gets popcount
// entries.  Must be called by all threads of the block.
template <int NT>
__device__ void emit_row(const uint32_t* bits, int words, uint32_t* bm_out, int16_t* col_out,
                         int* wpre) {
  for (int w = threadIdx.x; w < words; w += NT) {
    bm_out[w] = bits[w];
    int pre = 0;
    for (int v = 0; v < w; ++v) pre += __popc(bits[v]);
    wpre[w] = pre;
  }
  __syncthreads();
  for (int w = threadIdx.x; w < words; w += NT) {
    uint32_t m = bits[w];
    int pos = wpre[w];
    while (m) {
      const int bit = __ffs(m) - 1;
      m &= m - 1u;
      col_out[pos++] = (int16_t)(w * 32 + bit);
    }
  }
}

// ------------------------------------------------------------------ route
// One wave per row, E = ceil(nB/64) scores per lane (lane l holds key blocks
// l, l+64, l+128, ...).  No sort: the selected set is a prefix of the
// importance order (score descending, key block ascending), so it is the set
// of keys at or above a threshold key.  The 43-bit priority key is
// order_key(score) << 11 | (2047 - j): larger means earlier in the order, and
// it is unique within a row.
//   Top-p: with e_j = exp(s_j - max) in float64, Z = sum e_j and target
//   p*Z, the cut key is the largest key x whose tail mass S(x) = sum of e_j
//   over keys >= x reaches the target; it is found bit by bit from the top
//   (43 steps), each S(x) a wave sum in a fixed butterfly order.  Adding
//   terms never lowers a rounded sum, so S is monotone in x exactly as
//   computed and the search is exact for it.
//   Top-k floor: the largest key with at least k keys at or above it, by the
//   same search on ballot counts.
// The kept set is every key at or above the lower of the two thresholds.
// Each lane's 64-bit ballot per stride is two bitmask words directly, and
// ballot prefix counts place the ascending column list.
constexpr int kRouteThreads = 256;
constexpr int kRouteRowsPerBlock = kRouteThreads / 64;
constexpr int kMaxWaveNB = 2048;  // rows up to this many blocks: one wave per row
constexpr int kKeyBits = 43;
constexpr int kMaxNB = 32767;     // int16 column indices

// Sum of a double over the wave, the same bits in every lane.  Each step adds
// a partner lane's value with DPP or a lane swap (no LDS traffic): mirror
// inside 8 lanes, swap pairs of 2, swap neighbours, mirror inside 16, swap
// rows of 16, swap halves of 32.  Every step pairs lanes symmetrically and
// addition commutes, so all lanes hold identical partial sums after each step.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)u, CTRL, 0xF, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double swap_add_f64(double v, bool rows32) {
  const uint64_t u = __double_as_longlong(v);
  uint32_t lo0, lo1, hi0, hi1;
  if (rows32) {
    const auto l = __builtin_amdgcn_permlane32_swap((uint32_t)u, (uint32_t)u, false, false);
    const auto h = __builtin_amdgcn_permlane32_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
    lo0 = l[0]; lo1 = l[1]; hi0 = h[0]; hi1 = h[1];
  } else {
    const auto l = __builtin_amdgcn_permlane16_swap((uint32_t)u, (uint32_t)u, false, false);
    const auto h = __builtin_amdgcn_permlane16_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
    lo0 = l[0]; lo1 = l[1]; hi0 = h[0]; hi1 = h[1];
  }
  return __longlong_as_double((long long)(((uint64_t)hi0 << 32) | lo0)) +
         __longlong_as_double((long long)(((uint64_t)hi1 << 32) | lo1));
}
constexpr int kDppHalfMirror = 0x141, kDppRowMirror = 0x140;
constexpr int kDppQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<kDppHalfMirror>(v);
  v += dpp_f64<kDppQuadSwap2>(v);
  v += dpp_f64<kDppQuadSwap1>(v);
  v += dpp_f64<kDppRowMirror>(v);
  v = swap_add_f64(v, false);
  return swap_add_f64(v, true);
}

template <int E>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const float* __restrict__ S, int nB, int words, int64_t rows, float top_p, int topk,
    uint32_t* __restrict__ bitmask, int32_t* __restrict__ row_count,
    int16_t* __restrict__ col_idx, int32_t* __restrict__ head_count, uint32_t* flags) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRouteRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole wave: no barriers below
  const int64_t bh = row / nB;
  const float* s = S + row * nB;
  uint64_t key[E];
  float sv[E];
  bool nan_seen = false;
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = lane + 64 * e;
    key[e] = 0;
    sv[e] = -INFINITY;
    if (j < nB) {
      const float x = s[j];
      nan_seen |= (x != x);
      sv[e] = x;
      key[e] = ((uint64_t)order_key(x) << 11) | (uint64_t)(2047 - j);
      mx = fmaxf(mx, x);
    }
  }
  if (__builtin_amdgcn_ballot_w64(nan_seen) && lane == 0) atomicOr(flags, 1u);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));

  // count of keys >= x over the row (wave-uniform)
  auto count_ge = [&](uint64_t x) -> int {
    int c = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) c += __builtin_popcountll(__builtin_amdgcn_ballot_w64(key[e] >= x));
    return c;
  };

  // Top-p threshold (all keys when p >= 1, none when p <= 0)
  uint64_t thr;
  if (top_p >= 1.0f) {
    thr = 1;
  } else if (top_p <= 0.0f) {
    thr = ~0ull;
  } else {
    const double m = (double)mx;
    double ev[E];
    double part = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      ev[e] = key[e] != 0 ? exp((double)sv[e] - m) : 0.0;
      part += ev[e];
    }
    const double target = (double)top_p * wave_sum_f64(part);
    auto search = [&](uint64_t x, int hi_bit, int lo_bit) {
      for (int b = hi_bit; b >= lo_bit; --b) {
        const uint64_t c = x | (1ull << b);
        double t = 0.0;
#pragma unroll
        for (int e = 0; e < E; ++e) t += key[e] >= c ? ev[e] : 0.0;
        if (wave_sum_f64(t) >= target) x = c;
      }
      return x;
    };
    // the score bits first; the index bits only matter when several keys
    // share the boundary score, otherwise the cut key is that one key
    uint64_t x = search(0, kKeyBits - 1, 11);
    int ties = 0;
    uint64_t only = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint64_t bal = __builtin_amdgcn_ballot_w64(key[e] != 0 && (key[e] >> 11) == (x >> 11));
      ties += __builtin_popcountll(bal);
      if (bal) {
        const int l = __builtin_ctzll(bal);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(key[e] >> 32), l);
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)key[e], l);
        only = ((uint64_t)hi << 32) | lo;
      }
    }
    thr = ties == 1 ? only : search(x, 10, 0);
  }
  // Top-k floor: lower the threshold to the k-th key when the cut kept fewer
  if (topk > 0 && count_ge(thr) < topk) {
    if (topk >= nB) {
      thr = 1;
    } else {
      uint64_t x = 0;
      for (int b = kKeyBits - 1; b >= 0; --b) {
        const uint64_t c = x | (1ull << b);
        if (count_ge(c) >= topk) x = c;
      }
      thr = x;
    }
  }

  // bitmask words, ascending column list, counts
  uint32_t* bm = bitmask + row * words;
  int16_t* ci = col_idx + row * nB;
  const uint64_t below = (1ull << lane) - 1ull;
  int n = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (64 * e >= nB) break;
    const bool sel = key[e] != 0 && key[e] >= thr;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(sel);
    if (lane < 2 && 2 * e + lane < words) bm[2 * e + lane] = (uint32_t)(bal >> (32 * lane));
    if (sel) ci[n + __builtin_popcountll(bal & below)] = (int16_t)(lane + 64 * e);
    n += __builtin_popcountll(bal);
  }
  if (lane == 0) {
    row_count[row] = n;
    atomicAdd(&head_count[bh], n);
  }
}

// Rows of more than kMaxWaveNB blocks: one 1024-thread workgroup per row, the
// same threshold searches over 47-bit keys (order_key(s) << 15 | (32767 - j)),
// with every wave total combined across the 16 waves through LDS in wave
// order, so the sums stay deterministic.  Thread t holds blocks t + 1024e; it
// keeps the 32-bit order keys and the float64 exponentials in registers and
// forms the full key when it compares (past 8 blocks per thread, E = 16 and
// 32, part of them lives in scratch memory: slower, same results).
constexpr int kWideThreads = 1024;
constexpr int kWideWaves = kWideThreads / 64;
constexpr int kWideKeyBits = 47;

template <int E>
__global__ __launch_bounds__(kWideThreads) void route_wide_kernel(
    const float* __restrict__ S, int nB, int words, float top_p, int topk,
    uint32_t* __restrict__ bitmask, int32_t* __restrict__ row_count,
    int16_t* __restrict__ col_idx, int32_t* __restrict__ head_count, uint32_t* flags) {
  __shared__ double dred[2][kWideWaves];
  __shared__ int ired[2][kWideWaves];
  __shared__ float fred[kWideWaves];
  __shared__ uint64_t s_only;
  __shared__ int wbase[32 * kWideWaves];  // selected counts per (e, wave), then their exclusive prefix
  __shared__ int wtot[kWideWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = blockIdx.x;
  const int64_t bh = row / nB;
  const float* s = S + row * nB;
  uint32_t ok[E];  // order keys; slots past nB are not keys (key_of gives 0)
  bool nan_seen = false;
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = threadIdx.x + kWideThreads * e;
    ok[e] = 0u;
    if (j < nB) {
      const float x = s[j];
      nan_seen |= (x != x);
      ok[e] = order_key(x);
      mx = fmaxf(mx, x);
    }
  }
  auto key_of = [&](int e) -> uint64_t {
    const int j = threadIdx.x + kWideThreads * e;
    return j < nB ? ((uint64_t)ok[e] << 15) | (uint64_t)(32767 - j) : 0ull;
  };
  if (__builtin_amdgcn_ballot_w64(nan_seen) && lane == 0) atomicOr(flags, 1u);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if (lane == 0) fred[wave] = mx;
  __syncthreads();
  mx = fred[0];
  for (int w = 1; w < kWideWaves; ++w) mx = fmaxf(mx, fred[w]);

  // block totals: each wave's total (identical in its lanes) is combined in
  // wave order; two alternating buffers let one barrier serve each total
  int ph = 0;
  auto block_sum_f64 = [&](double wave_total) -> double {
    if (lane == 0) dred[ph][wave] = wave_total;
    __syncthreads();
    double t = 0.0;
    for (int w = 0; w < kWideWaves; ++w) t += dred[ph][w];
    ph ^= 1;
    return t;
  };
  auto block_sum_i32 = [&](int wave_total) -> int {
    if (lane == 0) ired[ph][wave] = wave_total;
    __syncthreads();
    int t = 0;
    for (int w = 0; w < kWideWaves; ++w) t += ired[ph][w];
    ph ^= 1;
    return t;
  };
  auto count_ge = [&](uint64_t x) -> int {
    int c = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) c += __builtin_popcountll(__builtin_amdgcn_ballot_w64(key_of(e) >= x));
    return block_sum_i32(c);
  };

  uint64_t thr;
  if (top_p >= 1.0f) {
    thr = 1;
  } else if (top_p <= 0.0f) {
    thr = ~0ull;
  } else {
    const double m = (double)mx;
    double ev[E];
    double part = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      ev[e] = key_of(e) != 0 ? exp((double)order_key_inv(ok[e]) - m) : 0.0;
      part += ev[e];
    }
    const double target = (double)top_p * block_sum_f64(wave_sum_f64(part));
    auto search = [&](uint64_t x, int hi_bit, int lo_bit) {
      for (int b = hi_bit; b >= lo_bit; --b) {
        const uint64_t c = x | (1ull << b);
        double t = 0.0;
#pragma unroll
        for (int e = 0; e < E; ++e) t += key_of(e) >= c ? ev[e] : 0.0;
        if (block_sum_f64(wave_sum_f64(t)) >= target) x = c;
      }
      return x;
    };
    uint64_t x = search(0, kWideKeyBits - 1, 15);
    int ties = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint64_t k = key_of(e);
      const bool tie = k != 0 && (k >> 15) == (x >> 15);
      if (tie) s_only = k;  // read only when exactly one key ties
      ties += __builtin_popcountll(__builtin_amdgcn_ballot_w64(tie));
    }
    ties = block_sum_i32(ties);  // its barrier also publishes s_only
    thr = ties == 1 ? s_only : search(x, 14, 0);
  }
  if (topk > 0 && count_ge(thr) < topk) {
    if (topk >= nB) {
      thr = 1;
    } else {
      uint64_t x = 0;
      for (int b = kWideKeyBits - 1; b >= 0; --b) {
        const uint64_t c = x | (1ull << b);
        if (count_ge(c) >= topk) x = c;
      }
      thr = x;
    }
  }

  // bitmask words straight from the ballots; the column list from an
  // exclusive scan of the per-(e, wave) counts in block order (e major)
  uint32_t* bm = bitmask + row * words;
  int16_t* ci = col_idx + row * nB;
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint64_t k = key_of(e);
    const uint64_t bal = __builtin_amdgcn_ballot_w64(k != 0 && k >= thr);
    const int w0 = 32 * e + 2 * wave;
    if (lane < 2 && w0 + lane < words) bm[w0 + lane] = (uint32_t)(bal >> (32 * lane));
    if (lane == 0) wbase[e * kWideWaves + wave] = __builtin_popcountll(bal);
  }
  __syncthreads();
  const int f = threadIdx.x;  // E*16 <= 512 entries: waves 0..7 hold them
  const int v = f < E * kWideWaves ? wbase[f] : 0;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();  // also: every thread has read its wbase entry
  int before = 0, mine = 0;
  for (int w = 0; w < kWideWaves; ++w) {
    if (w < wave) before += wtot[w];
    mine += wtot[w];
  }
  if (f < E * kWideWaves) wbase[f] = before + incl - v;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint64_t k = key_of(e);
    const bool sel = k != 0 && k >= thr;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(sel);
    if (sel)
      ci[wbase[e * kWideWaves + wave] + __builtin_popcountll(bal & below)] =
          (int16_t)(threadIdx.x + kWideThreads * e);
  }
  if (threadIdx.x == 0) {
    row_count[row] = mine;
    atomicAdd(&head_count[bh], mine);
  }
}

// ------------------------------------------------------------------ top-up
// Priority key of pair (i, j) with score s: smaller = higher priority
// (score descending, then i ascending, then j ascending).  62 bits.
__device__ __forceinline__ uint64_t pair_key(float s, int i, int j) {
  return ((uint64_t)(~order_key(s)) << 30) | ((uint64_t)i << 15) | (uint64_t)j;
}

// Exact selection of the need-th smallest priority key among a head's
// unselected pairs (need = budget - W_h), by an 8-pass radix select over the
// 62-bit keys (digits of 8 bits from the top, the last of 6).  Each pass is
// a sliced histogram (many workgroups per head, LDS histograms merged with
// global atomics) and a per-head pick of the digit where the running count
// reaches need.  thresh[bh] is an exclusive bound: pairs with key < thresh
// are added; 0 means none, ~0 means every unselected pair.
struct TopupState {
  uint64_t prefix;
  int64_t need;
  int32_t mode;  // 0 none, 1 select, 2 all
  int32_t pad;
};
constexpr int kSelSlices = 32;

__global__ void topup_init_kernel(const int32_t* __restrict__ head_count, int nB, int64_t budget,
                                  const int64_t* __restrict__ budgets, int nheads,
                                  TopupState* __restrict__ st, uint32_t* __restrict__ ghist,
                                  uint64_t* __restrict__ thresh) {
  const int bh = blockIdx.x;
  for (int b = threadIdx.x; b < 256; b += blockDim.x) ghist[bh * 256 + b] = 0u;
  if (threadIdx.x != 0) return;
  const int64_t pairs = (int64_t)nB * nB;
  const int64_t W = head_count[bh];
  const int64_t need = (budgets ? budgets[bh] : budget) - W;
  TopupState s{0ull, need, 1, 0};
  if (need <= 0) { s.mode = 0; thresh[bh] = 0ull; }
  else if (need >= pairs - W) { s.mode = 2; thresh[bh] = ~0ull; }
  st[bh] = s;
}

__global__ __launch_bounds__(256) void topup_hist_kernel(
    const float* __restrict__ S, const uint32_t* __restrict__ bitmask, int nB, int words,
    const TopupState* __restrict__ st, uint32_t* __restrict__ ghist, int pass) {
  __shared__ uint32_t hist[256];
  const int64_t bh = blockIdx.x;
  const TopupState s = st[bh];
  if (s.mode != 1) return;
  for (int b = threadIdx.x; b < 256; b += 256) hist[b] = 0u;
  __syncthreads();
  const int64_t pairs = (int64_t)nB * nB;
  const int64_t q0 = pairs * blockIdx.y / kSelSlices, q1 = pairs * (blockIdx.y + 1) / kSelSlices;
  const int sh = pass == 7 ? 0 : 54 - 8 * pass;
  const int hishift = pass == 0 ? 64 : sh + (pass == 7 ? 6 : 8);
  const uint32_t dmask = pass == 7 ? 63u : 255u;
  const float* Sh = S + bh * pairs;
  const uint32_t* Bh = bitmask + bh * (int64_t)nB * words;
  for (int64_t q = q0 + threadIdx.x; q < q1; q += 256) {
    const int i = (int)(q / nB), j = (int)(q - (int64_t)i * nB);
    if ((Bh[(int64_t)i * words + (j >> 5)] >> (j & 31)) & 1u) continue;
    const uint64_t key = pair_key(Sh[q], i, j);
    if (hishift < 64 && (key >> hishift) != s.prefix) continue;
    atomicAdd(&hist[(uint32_t)(key >> sh) & dmask], 1u);
  }
  __syncthreads();
  for (int b = threadIdx.x; b < 256; b += 256)
    if (hist[b]) atomicAdd(&ghist[bh * 256 + b], hist[b]);
}

__global__ void topup_pick_kernel(TopupState* __restrict__ st, uint32_t* __restrict__ ghist,
                                  uint64_t* __restrict__ thresh, int pass) {
  const int bh = blockIdx.x;
  if (threadIdx.x != 0) return;
  TopupState s = st[bh];
  if (s.mode != 1) return;
  uint32_t* h = ghist + bh * 256;
  int64_t nd = s.need;
  uint32_t d = 0;
  for (; d < 256; ++d) {
    if ((int64_t)h[d] >= nd) break;
    nd -= h[d];
  }
  // when digit d's bucket holds exactly the pairs still needed, every key
  // with this prefix is taken and the lower digits cannot change the set:
  // the bound is the first key past the bucket (with distinct scores this
  // ends the select after the four score digits)
  const bool whole = d < 256 && (int64_t)h[d] == nd;
  for (int b = 0; b < 256; ++b) h[b] = 0u;
  const int sh = pass == 7 ? 0 : 54 - 8 * pass;
  s.need = nd;
  s.prefix = (s.prefix << (pass == 7 ? 6 : 8)) | d;
  if (pass == 7 || whole) {
    thresh[bh] = (s.prefix + 1ull) << sh;
    s.mode = 0;
  }
  st[bh] = s;
}

// One workgroup per row of a topped-up head: add pairs below the threshold,
// rewrite the row's bitmask, count and column list, and the head workload.
__global__ __launch_bounds__(kRouteThreads) void topup_apply_kernel(
    const float* __restrict__ S, int nB, int words, const uint64_t* __restrict__ thresh,
    uint32_t* __restrict__ bitmask, int32_t* __restrict__ row_count,
    int16_t* __restrict__ col_idx, int32_t* __restrict__ head_count) {
  __shared__ uint32_t bits[(kMaxNB + 31) / 32];
  __shared__ int red[4];
  __shared__ int wpre[(kMaxNB + 31) / 32];
  const int64_t row = blockIdx.x;
  const int64_t bh = row / nB;
  const int i = (int)(row - bh * nB);
  const uint64_t th = thresh[bh];
  if (th == 0ull) return;
  uint32_t* bm = bitmask + row * words;
  for (int w = threadIdx.x; w < words; w += kRouteThreads) bits[w] = bm[w];
  __syncthreads();
  int added = 0;
  const float* s = S + row * nB;
  for (int j = threadIdx.x; j < nB; j += kRouteThreads) {
    const bool sel = (bits[j >> 5] >> (j & 31)) & 1u;
    if (!sel && pair_key(s[j], i, j) < th) {
      atomicOr(&bits[j >> 5], 1u << (j & 31));
      ++added;
    }
  }
  __syncthreads();
  const int tot = block_sum_i32<kRouteThreads>(added, red);
  if (tot == 0) return;
  emit_row<kRouteThreads>(bits, words, bm, col_idx + row * nB, wpre);
  if (threadIdx.x == 0) {
    row_count[row] += tot;
    atomicAdd(&head_count[bh], tot);
  }
}

// ------------------------------------------------------------------ queue
// Stable counting sort of rows by count, descending, in three launches:
//   1. per chunk of 1024 rows: sort (count desc, row) in LDS, record each
//      row's rank inside its run of equal counts, and the chunk's run lengths;
//   2. one exclusive scan over (count descending, chunk ascending) turns the
//      run lengths into output offsets;
//   3. scatter: queue[offset(chunk, count) + rank] = row.
constexpr int kQThreads = 1024;

__global__ __launch_bounds__(kQThreads) void queue_chunk_kernel(
    const int32_t* __restrict__ row_count, int64_t rows, int nB, int32_t* __restrict__ tmp_row,
    int32_t* __restrict__ tmp_rank, int32_t* __restrict__ hist) {
  __shared__ uint32_t keys[kQThreads];
  __shared__ int32_t wtot[kQThreads / 64];
  const int64_t base = (int64_t)blockIdx.x * kQThreads;
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  // this chunk's run lengths by count (nB + 1 entries), zero where no row has it
  int32_t* h = hist + (int64_t)blockIdx.x * (nB + 1);
  for (int c = threadIdx.x; c <= nB; c += kQThreads) h[c] = 0;
  const int64_t item = base + threadIdx.x;
  keys[threadIdx.x] = item < rows
                          ? ((uint32_t)(nB - row_count[item]) << 10) | (uint32_t)threadIdx.x
                          : 0xffffffffu;
  __syncthreads();
  // only the chunk's real rows need sorting: the first power of two that
  // holds them (the rest are all-ones keys, already in place at the end)
  const int64_t nreal = min((int64_t)kQThreads, rows - base);
  int P = 2;
  while (P < nreal) P <<= 1;
  bitonic_sort<uint32_t, kQThreads>(keys, P);
  const uint32_t k = keys[threadIdx.x];
  const bool valid = k != 0xffffffffu;
  const uint32_t grp = k >> 10;
  const bool head = threadIdx.x == 0 || (keys[threadIdx.x - 1] >> 10) != grp;
  int st = head ? (int)threadIdx.x : 0;  // inclusive max-scan of run starts
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(st, o, 64);
    if (lane >= o) st = max(st, v);
  }
  if (lane == 63) wtot[wave] = st;
  __syncthreads();
  int carry = 0;
  for (int w = 0; w < wave; ++w) carry = max(carry, wtot[w]);
  st = max(st, carry);
  if (valid) {
    tmp_row[base + threadIdx.x] = (int32_t)(base + (k & 1023u));
    tmp_rank[base + threadIdx.x] = (int)threadIdx.x - st;
    const bool tail = threadIdx.x == kQThreads - 1 || (keys[threadIdx.x + 1] >> 10) != grp;
    if (tail) h[nB - (int)grp] = (int)threadIdx.x - st + 1;
  }
}

// In-place exclusive scan of hist[chunk][c] in the order (c descending,
// chunk ascending): one workgroup, tiles of 1024 with a running carry.
__global__ __launch_bounds__(kQThreads) void queue_scan_kernel(int32_t* __restrict__ hist,
                                                               int64_t nchunks, int nB) {
  __shared__ int32_t wtot[kQThreads / 64];
  __shared__ int32_t s_carry;
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int64_t E = (int64_t)(nB + 1) * nchunks;
  if (threadIdx.x == 0) s_carry = 0;
  __syncthreads();
  for (int64_t e0 = 0; e0 < E; e0 += kQThreads) {
    const int64_t e = e0 + threadIdx.x;
    int64_t idx = -1;
    int v = 0;
    if (e < E) {
      const int c = nB - (int)(e / nchunks);
      const int64_t ch = e % nchunks;
      idx = ch * (nB + 1) + c;
      v = hist[idx];
    }
    int x = v;  // inclusive wave scan
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wtot[wave] = x;
    __syncthreads();
    int before = s_carry;
    for (int w = 0; w < wave; ++w) before += wtot[w];
    if (idx >= 0) hist[idx] = before + x - v;
    __syncthreads();
    if (threadIdx.x == kQThreads - 1) s_carry = before + x;
    __syncthreads();
  }
}

__global__ void queue_scatter_kernel(const int32_t* __restrict__ tmp_row,
                                     const int32_t* __restrict__ tmp_rank,
                                     const int32_t* __restrict__ hist,
                                     const int32_t* __restrict__ row_count, int64_t rows, int nB,
                                     int32_t* __restrict__ queue) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= rows) return;
  const int32_t row = tmp_row[t];
  const int64_t chunk = t / kQThreads;
  queue[hist[chunk * (nB + 1) + row_count[row]] + tmp_rank[t]] = row;
}

}  // namespace

namespace {

void launch_topup_kernels(const Problem& p, const fva_mask& m, char* ws, int64_t budget,
                          const int64_t* budgets, hipStream_t s) {
  const RouteWs L = route_ws_layout(p);
  uint64_t* thresh = (uint64_t*)(ws + L.thresh_off);
  TopupState* st = (TopupState*)(ws + L.tstate_off);
  uint32_t* ghist = (uint32_t*)(ws + L.thist_off);
  const int nheads = p.B * p.Hh;
  hipLaunchKernelGGL(topup_init_kernel, dim3(nheads), dim3(256), 0, s, m.head_count, p.nB,
                     budget, budgets, nheads, st, ghist, thresh);
  for (int pass = 0; pass < 8; ++pass) {
    hipLaunchKernelGGL(topup_hist_kernel, dim3(nheads, kSelSlices), dim3(256), 0, s, m.scores,
                       m.bitmask, p.nB, p.words, st, ghist, pass);
    hipLaunchKernelGGL(topup_pick_kernel, dim3(nheads), dim3(64), 0, s, st, ghist, thresh, pass);
  }
  hipLaunchKernelGGL(topup_apply_kernel, dim3((unsigned)p.rows), dim3(kRouteThreads), 0, s,
                     m.scores, p.nB, p.words, thresh, m.bitmask, m.row_count, m.col_idx,
                     m.head_count);
}

void launch_queue(const Problem& p, const fva_mask& m, char* ws, hipStream_t s) {
  const RouteWs L = route_ws_layout(p);
  const int64_t nchunks = (p.rows + kQThreads - 1) / kQThreads;
  int32_t* tmp_row = (int32_t*)(ws + L.qtmp_row_off);
  int32_t* tmp_rank = (int32_t*)(ws + L.qtmp_rank_off);
  int32_t* hist = (int32_t*)(ws + L.qhist_off);
  hipLaunchKernelGGL(queue_chunk_kernel, dim3((unsigned)nchunks), dim3(kQThreads), 0, s,
                     m.row_count, p.rows, p.nB, tmp_row, tmp_rank, hist);
  hipLaunchKernelGGL(queue_scan_kernel, dim3(1), dim3(kQThreads), 0, s, hist, nchunks, p.nB);
  hipLaunchKernelGGL(queue_scatter_kernel, dim3((unsigned)((p.rows + 255) / 256)), dim3(256), 0,
                     s, tmp_row, tmp_rank, hist, m.row_count, p.rows, p.nB, m.queue);
}

}  // namespace

fva_status launch_route(const Problem& p, const void* qr, const void* kr,
                        const fva_route_params& prm, float scale, const fva_mask& m,
                        char* ws, int flags, hipStream_t s) {
  const RouteWs L = route_ws_layout(p);
  uint32_t* wflags = (uint32_t*)(ws + L.flags_off);
  const bool pooled_in = (flags & FVA_ROUTE_POOLED_IN) != 0;
  // block means: the workspace's, or the caller's (written by fva_reorder_pool)
  const float* qbar = pooled_in ? (const float*)qr : (const float*)(ws + L.qbar_off);
  const float* kbar = pooled_in ? (const float*)kr : (const float*)(ws + L.kbar_off);
  const int nheads = p.B * p.Hh;
  hipLaunchKernelGGL(zero_route_state, dim3((nheads + 255) / 256), dim3(256), 0, s,
                     m.head_count, nheads, wflags);
  if (!(flags & FVA_ROUTE_SCORES_IN)) {
    dim3 pg(p.nB, nheads, 2);
    float* qw = (float*)(ws + L.qbar_off);
    float* kw = (float*)(ws + L.kbar_off);
    if (pooled_in) {
      // nothing to pool
    } else if (p.d == 128)
      hipLaunchKernelGGL(pool_kernel<128>, pg, dim3(256), 0, s, (const uint16_t*)qr,
                         (const uint16_t*)kr, qw, kw, p.N, p.Npad, p.BLK, p.nB);
    else
      hipLaunchKernelGGL(pool_kernel<64>, pg, dim3(256), 0, s, (const uint16_t*)qr,
                         (const uint16_t*)kr, qw, kw, p.N, p.Npad, p.BLK, p.nB);
    dim3 sg((p.nB + 63) / 64, (p.nB + 63) / 64, nheads);
    if (p.d == 128)
      hipLaunchKernelGGL(score_kernel<128>, sg, dim3(256), 0, s, qbar, kbar, m.scores, p.nB,
                         scale);
    else
      hipLaunchKernelGGL(score_kernel<64>, sg, dim3(256), 0, s, qbar, kbar, m.scores, p.nB,
                         scale);
  }
  // scores per lane: ceil(nB / 64), rounded up to an instantiated width
#define FVA_ROUTE(E)                                                                           \
  hipLaunchKernelGGL(route_kernel<E>, dim3((unsigned)((p.rows + kRouteRowsPerBlock - 1) /      \
                                                      kRouteRowsPerBlock)),                    \
                     dim3(kRouteThreads), 0, s, m.scores, p.nB, p.words, p.rows, prm.top_p,     \
                     prm.topk_floor, m.bitmask, m.row_count, m.col_idx, m.head_count, wflags)
#define FVA_ROUTE_WIDE(E)                                                                      \
  hipLaunchKernelGGL(route_wide_kernel<E>, dim3((unsigned)p.rows), dim3(kWideThreads), 0, s,   \
                     m.scores, p.nB, p.words, prm.top_p, prm.topk_floor, m.bitmask,          \
                     m.row_count, m.col_idx, m.head_count, wflags)
  const int per_lane = (p.nB + 63) / 64;
  const int per_thread = (p.nB + kWideThreads - 1) / kWideThreads;
  if (p.nB > kMaxWaveNB) {
    if (per_thread <= 4) FVA_ROUTE_WIDE(4);
    else if (per_thread <= 8) FVA_ROUTE_WIDE(8);
    else if (per_thread <= 16) FVA_ROUTE_WIDE(16);
    else FVA_ROUTE_WIDE(32);
  } else if (per_lane <= 2) FVA_ROUTE(2);
  else if (per_lane <= 4) FVA_ROUTE(4);
  else if (per_lane <= 8) FVA_ROUTE(8);
  else if (per_lane <= 10) FVA_ROUTE(10);
  else if (per_lane <= 12) FVA_ROUTE(12);
  else if (per_lane <= 16) FVA_ROUTE(16);
  else if (per_lane <= 24) FVA_ROUTE(24);
  else FVA_ROUTE(32);
#undef FVA_ROUTE
#undef FVA_ROUTE_WIDE
  if (prm.aug_budget > 0) launch_topup_kernels(p, m, ws, (int64_t)prm.aug_budget, nullptr, s);
  launch_queue(p, m, ws, s);
  return hip_fail(hipGetLastError(), "route launch");
}

fva_status launch_topup(const Problem& p, const int64_t* budgets, const fva_mask& m, char* ws,
                        hipStream_t s) {
  launch_topup_kernels(p, m, ws, 0, budgets, s);
  launch_queue(p, m, ws, s);
  return hip_fail(hipGetLastError(), "top-up launch");
}

}  // namespace fva
