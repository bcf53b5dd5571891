// Block-sparse flash attention for gfx950 (FVAttn page, section 2: the block
// mask decides which query-block/key-block pairs are computed; section 3.2:
// work is balanced on the realized per-row workload, here by persistent work
// queues).
//
// Work item = one query block (BLK rows) of one head, processed by one
// workgroup of BLK/32 waves; each wave owns 32 queries and walks every
// selected key block of the row in 64-key sub-tiles.  A sub-tile of K and V
// (32 KB at d=128) is staged in LDS by direct HBM->LDS buffer loads
// (buffer_load_dwordx4 with the LDS destination), double-buffered, so a
// workgroup uses 64 KB and two independent workgroups share a CU: while one
// is in its softmax the other keeps the matrix cores busy.
//
// Products use v_mfma_f32_32x32x16_bf16 in transposed form:
//   S^T (keys x queries) = K * Q^T     A = K from LDS, B = Q^T in registers
//   O^T (d x queries)   += V^T * P^T   A = V^T from LDS, B = P^T in registers
// With queries on the MFMA column axis every lane holds one query's column,
// so the running max, sum and the rescale of O are lane-local (one cross-half
// exchange per tile for the max).  P^T leaves the S accumulator in exactly the
// B-operand order the PV product needs once the V^T chunk stores key slots
// with bits 2 and 3 swapped (done by the reorder kernel).
//
// Online softmax in the log2 domain with the scale folded into one FMA per
// score, and a lazy rescale: the running reference max only moves (and O and
// the running sum are rescaled) when a tile's max exceeds it by more than
// 2^8, so exponentials stay <= 256 and most tiles skip the rescale.
//
// Schedules: static contiguous split (fixed placement), hardware grid over the
// heaviest-first queue, a persistent atomic heaviest-first queue, and an
// XCD-aware persistent schedule: heads are placed on the 8 XCDs heaviest
// first by longest-processing-time on their realized workload W_h, each XCD
// walks its heads' rows in query-block order (neighbouring query blocks share
// most key blocks, so their K/V stream through that XCD's L2 once), and a
// workgroup whose XCD runs dry steals from the other XCDs' lists.
#include <algorithm>
#include <mutex>

#include "fva_internal.hpp"

namespace fva {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int KT = 64;           // keys per sub-tile
constexpr int kColChunk = 2048;  // column-list entries staged in LDS at a time
constexpr int NXCD = 8;          // XCDs; workgroups are dealt to them round robin
constexpr float kLazy = 8.0f;    // log2-domain slack before the reference max moves

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Raw byte buffer over [base, base + bytes): the resource lives in SGPRs, so a
// copy needs only a 32-bit per-lane offset (data format 32, as gfx9 raw
// buffers use; accesses past `bytes` read zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_buffer(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// 16 bytes per lane from buffer rs at voff + soff (soff wave-uniform) into LDS
// at lds_uniform + 16*lane.  HBM->LDS copies issued as buffer loads leave the
// matrix cores' issue rate nearly untouched; the same copies with a 64-bit
// per-lane address cost a sixth of it when one is issued per four MFMAs.
__device__ __forceinline__ void buf2lds16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff,
                                          char* lds_uniform) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rs, (__attribute__((address_space(3))) void*)lds_uniform, 16, voff, soff, 0, 0);
}

// LDS tiles are verbatim copies of the k64 / v64 HBM tiles:
//   K tile: 16-byte unit (c, r) = channels 8c..8c+7 of key r at byte (c*64 + r)*16
//   V tile: 16-byte unit (g, e) = channel e of key slots 8g..8g+7 at byte (g*D + e)*16
// A wave's MFMA operand read touches 64 consecutive units (one lane each), so
// every read is conflict-free and its address is one per-lane base plus an
// immediate offset.

// Attention workspace: [0,256) counters and per-XCD offsets, then the
// XCD-ordered row list.
struct AttnWs {
  static constexpr int kQueueCtr = 0;      // int: global queue counter
  static constexpr int kXcdCtr = 16;       // int[8]: per-XCD counters
  static constexpr int kXcdOff = 32;       // int[9]: per-XCD offsets into xq
  __host__ __device__ static size_t xq_off() { return 256; }
  __host__ __device__ static size_t bytes(int64_t rows) {
    return xq_off() + ((rows * 4 + 255) & ~(int64_t)255);
  }
};

struct AttnArgs {
  const uint16_t* qr;
  const uint16_t* kr;
  const uint16_t* vt;
  uint16_t* out;
  const int32_t* row_count;
  const int32_t* head_count;
  const int16_t* col_idx;
  const int32_t* queue;    // heaviest-first queue, or the XCD-ordered list
  int32_t* ws;             // attention workspace (int view)
  uint32_t* trace;
  float* lse;              // optional: per-query log-sum-exp, [B*Hh, N]
  int64_t N, Npad;
  int64_t rows;
  int nB;
  float sl2;   // scale * log2(e)
  float isl2;  // 1 / sl2: the lazy threshold is kept in raw-score units
  int direct;  // 1: queue entry i is row i (every item is resident at once, so
               // the order of the queue buys nothing and its read is skipped)
};

// QT = 32-query tiles per wave (1: 4 waves of 32 queries per 128-row block,
// two waves per SIMD; 2: 2 waves of 64 queries, one wave per SIMD).
template <int QT>
constexpr int attn_threads(int blk) { return blk / (32 * QT) * 64; }

// Teams per workgroup when a launch has no more rows than CUs: each team
// (BLK/32 waves, its own K/V double buffers) walks every TEAMS-th key
// sub-tile of the row and the teams' softmax states are merged in LDS at the
// end, so a row's critical path is shared.  At most two waves per SIMD and
// 128 KB of tile buffers per workgroup.
template <int D, int BLK>
constexpr int attn_teams() { return (D == 64 && BLK == 64) ? 4 : 2; }

// CHUNKED: rows may select more than kColChunk blocks, so the column list
// is walked in LDS chunks (launched only when nB > kColChunk; otherwise the
// walk is one straight pass over a list read whole).
// TEAMS: 1, or attn_teams<D, BLK>() for launches with rows <= CUs (never
// together with CHUNKED).
template <int D, int BLK, int QT, int SCHED, bool DENSE, bool TRACE, bool CHUNKED, int TEAMS>
__global__ __launch_bounds__(attn_threads<QT>(BLK) * TEAMS) __attribute__((amdgpu_waves_per_eu(
    QT == 1 ? 2 : 1, QT == 1 ? 2 : 1))) void attn_kernel(AttnArgs a) {
  static_assert(TEAMS == 1 || !CHUNKED, "teams serve short launches only");
  constexpr int NT = attn_threads<QT>(BLK);  // threads of one team: BLK/(32*QT) waves
  constexpr int NW = NT / 64;
  constexpr int NTALL = NT * TEAMS;          // threads of the workgroup
  constexpr int TILE = KT * D * 2;       // bytes of one K or V^T sub-tile
  constexpr int NSUB = BLK / KT;         // sub-tiles per key block
  constexpr int KSTEPS = D / 16;         // MFMA k-steps over the head dim
  constexpr int DT = D / 32;             // 32-row tiles of the head dim
  constexpr int CPR = D / 8;             // 16-byte chunks per K row
  constexpr int LOADS = TILE / 16 / NT;  // 16-byte loads per thread per K (or V) tile
  static_assert(LOADS * 16 * NT == TILE, "tile size");
  // LDS per team: K tiles at [0, 2*TILE), V^T tiles at [2*TILE, 4*TILE)
  __shared__ __attribute__((aligned(16))) char lds_all[4 * TILE * TEAMS];
  __shared__ int16_t s_cols[kColChunk];
  __shared__ int s_item;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int team = TEAMS == 1 ? 0 : __builtin_amdgcn_readfirstlane((tid >> 6) / NW);
  const int wave = TEAMS == 1 ? __builtin_amdgcn_readfirstlane(tid >> 6)
                              : __builtin_amdgcn_readfirstlane((tid >> 6) % NW);  // in its team
  char* const lds = lds_all + team * 4 * TILE;
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  // byte offset of this thread's first 16-byte load inside a tile; load k of
  // the wave adds k*NW*1024 (each wave instruction moves 1 KB contiguously)
  const uint32_t loff = (uint32_t)(wave * 64 + lane) * 16u;

  // the XCD this workgroup runs on, read from the hardware (XCC_ID): the
  // dispatcher deals workgroups round robin over the XCDs, but the XCD of
  // workgroup 0 is not fixed (it moved when other queues had work), and the
  // lists only pay off when the XCD that takes a list is the one it runs on
  const int xcd = (int)(__builtin_amdgcn_s_getreg((31 << 11) | 20) & (NXCD - 1));
  int victim = 0;  // XCD schedule: how far thread 0 has moved from its own XCD

  // fetch the next item (position in the schedule's row list); -1 when done
  auto fetch = [&]() -> int64_t {
    if (SCHED == FVA_SCHED_QUEUE) {
      if (tid == 0) s_item = atomicAdd(a.ws + AttnWs::kQueueCtr, 1);
      __syncthreads();
      const int64_t it = s_item;
      return it < a.rows ? it : -1;
    } else {  // FVA_SCHED_XCD
      if (tid == 0) {
        int got = -1;
        while (victim < NXCD) {
          const int y = (xcd + victim) % NXCD;
          const int beg = a.ws[AttnWs::kXcdOff + y], end = a.ws[AttnWs::kXcdOff + y + 1];
          if (end > beg) {
            const int it = atomicAdd(a.ws + AttnWs::kXcdCtr + y, 1);
            if (it < end - beg) { got = beg + it; break; }
          }
          ++victim;
        }
        s_item = got;
      }
      __syncthreads();
      return s_item;
    }
  };

  int64_t item, item_end = 0;
  if (SCHED == FVA_SCHED_STATIC) {
    const int64_t G = gridDim.x;
    item = (int64_t)blockIdx.x * a.rows / G;
    item_end = ((int64_t)blockIdx.x + 1) * a.rows / G;
  } else if (SCHED == FVA_SCHED_QUEUE || SCHED == FVA_SCHED_XCD) {
    item = fetch();
  } else if (DENSE) {
    // XCD-aware remap: the workgroups b with one residue b mod 8 share an XCD
    // (round-robin dealing), so each XCD walks a contiguous range of rows
    // (whole heads); a bijection of b whichever XCD the dealing starts on
    const int64_t b = blockIdx.x;
    item = (a.rows % NXCD == 0) ? (b % NXCD) * (a.rows / NXCD) + b / NXCD : b;
  } else {
    item = blockIdx.x;
  }

  while (true) {
    if (SCHED == FVA_SCHED_STATIC) {
      if (item >= item_end) break;
    } else if (item < 0 || item >= a.rows) {
      break;
    }
    uint64_t t_start = 0;
    if (TRACE && tid == 0) t_start = __builtin_amdgcn_s_memrealtime();
    int64_t row;
    if (DENSE || SCHED == FVA_SCHED_STATIC || a.direct) row = item;
    else row = a.queue[item];
    row = __builtin_amdgcn_readfirstlane((int)row);
    const int64_t bh = row / a.nB;
    const int qb = (int)(row - bh * a.nB);
    // Q^T operands: q-tile j of this wave = 32 queries; lane holds query l32,
    // d chunk 2kk+hl (issued first: their latency overlaps the column list's)
    const int64_t q0 = (int64_t)qb * BLK + wave * 32 * QT;
    bf16x8 qop[QT][KSTEPS];
#pragma unroll
    for (int j = 0; j < QT; ++j) {
      const uint16_t* qp = a.qr + (bh * a.Npad + q0 + 32 * j + l32) * D + hl * 8;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) qop[j][kk] = as_bf16x8(*(const u32x4*)(qp + kk * 16));
    }
    int cnt = a.nB;
    const int16_t* cols = DENSE ? nullptr : a.col_idx + row * a.nB;
    if (!DENSE) {
      // the count and the first chunk of the column row are read together
      // (entries past the count are in bounds and never used), not one after
      // the other
      const int cnt_ld = a.row_count[row];
      const int n0 = CHUNKED ? min(a.nB, kColChunk) : a.nB;
      for (int t = tid; t < n0; t += NTALL) s_cols[t] = cols[t];
      cnt = __builtin_amdgcn_readfirstlane(cnt_ld);
      __syncthreads();
    }
    const int64_t nlast = a.N - (int64_t)(a.nB - 1) * BLK;  // real keys of the last block
    // the column list is walked in chunks of kColChunk held in s_cols (one
    // chunk unless a row selects more blocks); U = sub-tiles of this chunk
    int c0 = 0;
    int ccnt = (DENSE || !CHUNKED) ? cnt : min(cnt, kColChunk);
    int U = 0;

    // this head's K and V tiles (the tile of key0 starts at element key0*D)
    const __amdgpu_buffer_rsrc_t kbuf = byte_buffer(a.kr + bh * a.Npad * D, (int)(a.Npad * D * 2));
    const __amdgpu_buffer_rsrc_t vbuf = byte_buffer(a.vt + bh * a.Npad * D, (int)(a.Npad * D * 2));

    auto key0_of = [&](int u) -> int64_t {
      const int t = u / NSUB, half = u % NSUB;
      const int kb = DENSE ? t : __builtin_amdgcn_readfirstlane((int)s_cols[t]);
      return (int64_t)kb * BLK + half * KT;
    };
    auto load_tile = [&](__amdgpu_buffer_rsrc_t rs, int u, char* buf) {
      const uint32_t soff = (uint32_t)(key0_of(u) * D * 2);
#pragma unroll
      for (int k = 0; k < LOADS; ++k)
        buf2lds16(rs, loff, soff + k * NW * 1024, buf + (k * NW + wave) * 1024);
    };
    // team-local sub-tile v is the row's sub-tile team + v*TEAMS; the local
    // index picks the buffer, the row's index the keys
    auto gsub = [&](int v) { return TEAMS == 1 ? v : team + v * TEAMS; };
    auto load_k = [&](int u) { load_tile(kbuf, gsub(u), lds + (u & 1) * TILE); };
    auto load_v = [&](int u) { load_tile(vbuf, gsub(u), lds + (2 + (u & 1)) * TILE); };

    f32x16 oacc[DT][QT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int j = 0; j < QT; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][j][r] = 0.f;
    // m_use: reference max (log2 domain); m_thr: the raw score above which a
    // tile moves it, (m_use + kLazy) / sl2, so a tile's test is one compare
    float m_use[QT], l_run[QT], m_thr[QT];
#pragma unroll
    for (int j = 0; j < QT; ++j) { m_use[j] = -INFINITY; l_run[j] = 0.f; m_thr[j] = -INFINITY; }

    // S^T of sub-tile u: keys 32m + (acc row) x queries 32j + l32
    auto qk = [&](int u, f32x16 (&s)[2][QT]) {
      const char* kt = lds + (u & 1) * TILE;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int j = 0; j < QT; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[m][j][r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
          const bf16x8 kop = as_bf16x8(
              *(const u32x4*)(kt + (2 * kk + hl) * 1024 + (32 * m + l32) * 16));
#pragma unroll
          for (int j = 0; j < QT; ++j)
            s[m][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[j][kk], s[m][j], 0, 0, 0);
        }
      }
    };
    // masking of padded keys, tile max and lazy rescale for sub-tile u
    auto prep = [&](int u, f32x16 (&s)[2][QT]) {
      const int kvalid = (int)min((int64_t)KT, a.N - key0_of(gsub(u)));
      if (kvalid < KT) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int j = 0; j < QT; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = 32 * m + 8 * (r >> 2) + 4 * hl + (r & 3);
              if (key >= kvalid) s[m][j][r] = -INFINITY;
            }
      }
      float mx[QT];
      bool grow = false;
#pragma unroll
      for (int j = 0; j < QT; ++j) {
        float v = fmaxf(s[0][j][0], s[0][j][1]);
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int r = (m == 0 ? 2 : 0); r < 16; ++r) v = fmaxf(v, s[m][j][r]);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                         false, false);
        mx[j] = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        grow = grow || (mx[j] > m_thr[j]);
      }
      // move the reference max only when a tile exceeds it by 2^8
      if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
        for (int j = 0; j < QT; ++j) {
          const float m_new = fmaxf(m_use[j], mx[j] * a.sl2);
          const float alpha = __builtin_amdgcn_exp2f(m_use[j] - m_new);
          l_run[j] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[dt][j][r] *= alpha;
          m_use[j] = m_new;
          m_thr[j] = (m_new + kLazy) * a.isl2;
        }
      }
    };
    // probabilities of sub-tile u as PV B-operands, and their bf16 sum
    auto probs = [&](const f32x16 (&s)[2][QT], bf16x8 (&pop)[2][2][QT]) {
      const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int j = 0; j < QT; ++j) {
        const float nm = -m_use[j];
        float ls = l_run[j];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            u32x4 pk;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float p0 = __builtin_amdgcn_exp2f(fmaf(s[m][j][8 * b + 2 * e], a.sl2, nm));
              const float p1 = __builtin_amdgcn_exp2f(fmaf(s[m][j][8 * b + 2 * e + 1], a.sl2, nm));
              const uint32_t w = pack_bf16(p0, p1);
              ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one2, ls, false);
              pk[e] = w;
            }
            pop[m][b][j] = as_bf16x8(pk);
          }
        l_run[j] = ls;
      }
    };
    auto pv = [&](int u, const bf16x8 (&pop)[2][2][QT]) {
      const char* vtile = lds + (2 + (u & 1)) * TILE;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            const bf16x8 vop = as_bf16x8(*(const u32x4*)(
                vtile + (4 * m + 2 * b + hl) * (D * 16) + (32 * dt + l32) * 16));
#pragma unroll
            for (int j = 0; j < QT; ++j)
              oacc[dt][j] =
                  __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[m][b][j], oacc[dt][j], 0, 0, 0);
          }
      }
    };

    while (true) {
      U = ccnt * NSUB;
      if (ccnt > 0 && c0 + ccnt == cnt) {
        const int lastcol = DENSE ? a.nB - 1 : (int)s_cols[ccnt - 1];
        if (lastcol == a.nB - 1) U -= NSUB - (int)((nlast + KT - 1) / KT);
      }
      U = __builtin_amdgcn_readfirstlane(U);
      // this team's sub-tiles, and the steps every team takes (the teams
      // share the per-step barrier; a team past its last sub-tile idles)
      const int Ut = TEAMS == 1 ? U : (U > team ? (U - 1 - team) / TEAMS + 1 : 0);
      const int S = TEAMS == 1 ? U : (U + TEAMS - 1) / TEAMS;
      if (S > 0) {
        // prologue: K(0), V(0), K(1) in flight; S(0) once K(0) has landed
        if (TEAMS == 1 || Ut > 0) {
          load_k(0);
          load_v(0);
        }
        if (Ut > 1) load_k(1);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        f32x16 sa[2][QT], sb[2][QT];
        if (TEAMS == 1 || Ut > 0) qk(0, sa);
        // steady state: at iteration u, S(u) is in registers, K(u+1) and V(u)
        // are (being) loaded; K(u+2) and V(u+1) are issued here.  S(u+1) is
        // computed unconditionally (on a stale buffer after the last tile; the
        // result is then unused) so the products of the next tile and the
        // softmax of this one share one basic block.
        auto step = [&](int u, f32x16 (&sc)[2][QT], f32x16 (&sn)[2][QT]) {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          __syncthreads();
          if (u + 2 < Ut) load_k(u + 2);
          if (u + 1 < Ut) load_v(u + 1);
          if (TEAMS == 1 || u < Ut) {
            prep(u, sc);
            bf16x8 pop[2][2][QT];
            qk(u + 1, sn);
            probs(sc, pop);
            pv(u, pop);
          }
        };
        for (int u = 0; u < S; u += 2) {
          step(u, sa, sb);
          if (u + 1 >= S) break;
          step(u + 1, sb, sa);
        }
      }
      c0 += ccnt;
      if (DENSE || !CHUNKED || c0 >= cnt) break;
      // next chunk of the column list: every wave is done with the tile
      // buffers and the previous chunk before either is overwritten
      __syncthreads();
      ccnt = min(cnt - c0, kColChunk);
      for (int t = tid; t < ccnt; t += NTALL) s_cols[t] = cols[c0 + t];
      __syncthreads();
    }

    if (TEAMS > 1) {
      // merge the teams' softmax states into team 0, team by team in order:
      // with m = max of the references, O and l of each team scale by
      // 2^(m_t - m) (0 for a team that saw no key)
      static_assert(QT == 1, "teams merge one query tile per wave");
      constexpr int PER = 2 + DT * 16;  // floats per lane: reference, sum, O
      constexpr int SLOTS = NW * 64;    // lanes of one team
      static_assert((TEAMS - 1) * PER * SLOTS * 4 <= 4 * TILE * TEAMS, "merge buffer");
      float* const mb = reinterpret_cast<float*>(lds_all);
      const int slot = wave * 64 + lane;
      __syncthreads();  // every team is done with its tile buffers
      if (team > 0) {
        float* dst = mb + (team - 1) * PER * SLOTS + slot;
        dst[0] = m_use[0];
        dst[SLOTS] = l_run[0];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) dst[(2 + dt * 16 + r) * SLOTS] = oacc[dt][0][r];
      }
      __syncthreads();
      if (team == 0) {
        for (int t = 1; t < TEAMS; ++t) {
          const float* src = mb + (t - 1) * PER * SLOTS + slot;
          const float mt = src[0];
          const float mx = fmaxf(m_use[0], mt);
          const float a0 = m_use[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_use[0] - mx);
          const float at = mt == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mt - mx);
          l_run[0] = l_run[0] * a0 + src[SLOTS] * at;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              oacc[dt][0][r] = oacc[dt][0][r] * a0 + src[(2 + dt * 16 + r) * SLOTS] * at;
          m_use[0] = mx;
        }
      }
    }

    // finalize (team 0): total sum over both half-waves, normalize, write bf16
#pragma unroll
    for (int j = 0; j < QT; ++j) {
      if (TEAMS > 1 && team != 0) break;
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run[j]),
                                                       __float_as_uint(l_run[j]), false, false);
      const float l = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      const float inv = l > 0.f ? 1.f / l : 0.f;
      const int64_t q = q0 + 32 * j + l32;
      const float sc_ = q < a.N ? inv : 0.f;
      // natural log-sum-exp of the scaled scores over the keys used:
      // sum_k exp2(s_k * sl2) = 2^m_use * l
      if (a.lse && hl == 0 && q < a.N)
        a.lse[bh * a.N + q] = l > 0.f ? (m_use[j] + log2f(l)) * 0.69314718055994531f : -INFINITY;
      uint16_t* op = a.out + (bh * a.Npad + q) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u32x2 w;
          w.x = pack_bf16(oacc[dt][j][4 * i + 0] * sc_, oacc[dt][j][4 * i + 1] * sc_);
          w.y = pack_bf16(oacc[dt][j][4 * i + 2] * sc_, oacc[dt][j][4 * i + 3] * sc_);
          *(u32x2*)(op + 32 * dt + 8 * i + 4 * hl) = w;
        }
    }
    if (TRACE && tid == 0) {
      const uint64_t t_end = __builtin_amdgcn_s_memrealtime();
      uint32_t* tr = a.trace + item * 8;
      tr[0] = (uint32_t)row;
      tr[1] = __builtin_amdgcn_s_getreg((31 << 11) | 20);  // XCC_ID
      tr[2] = __builtin_amdgcn_s_getreg((31 << 11) | 4);   // HW_ID
      tr[3] = blockIdx.x;
      tr[4] = (uint32_t)t_start;
      tr[5] = (uint32_t)(t_start >> 32);
      tr[6] = (uint32_t)t_end;
      tr[7] = (uint32_t)(t_end >> 32);
    }
    // all waves are done with the LDS buffers and the column list
    __syncthreads();
    if (SCHED == FVA_SCHED_STATIC) {
      ++item;
    } else if (SCHED == FVA_SCHED_QUEUE || SCHED == FVA_SCHED_XCD) {
      item = fetch();
    } else {
      break;
    }
  }
}

__global__ void zero_counter(int32_t* ws) { ws[AttnWs::kQueueCtr] = 0; }

// XCD plan (one workgroup): order heads by W_h descending (ties by head id),
// assign them greedily to the least-loaded XCD (longest processing time
// first), lay the XCD row lists out contiguously (XCD x owns [off[x],
// off[x+1]) and its heads follow in assignment order, nB rows each), and
// write every head's rows in query-block order at its place.  Neighbouring
// query blocks select mostly the same key blocks, so the workgroups resident
// on one XCD stream shared K/V tiles through that XCD's L2; balance comes
// from the head placement and stealing.
constexpr int kPlanThreads = 256;

__global__ __launch_bounds__(kPlanThreads) void xcd_plan_kernel(const int32_t* head_count,
                                                                int nheads, int nB, int32_t* ws) {
  __shared__ uint64_t keys[kMaxXcdHeads];
  __shared__ int32_t hbase[kMaxXcdHeads];
  __shared__ int32_t s_off[NXCD];
  int P = 1;
  while (P < nheads) P <<= 1;
  for (int h = threadIdx.x; h < P; h += kPlanThreads)
    keys[h] = h < nheads ? ((uint64_t)(~(uint32_t)head_count[h]) << 32) | (uint32_t)h : ~0ull;
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int q = threadIdx.x; q < P / 2; q += kPlanThreads) {
        const int i = 2 * j * (q / j) + (q % j), l = i + j;
        const uint64_t x = keys[i], y = keys[l];
        if ((x > y) == ((i & k) == 0)) { keys[i] = y; keys[l] = x; }
      }
      __syncthreads();
    }
  if (threadIdx.x == 0) {
    int64_t load[NXCD] = {0, 0, 0, 0, 0, 0, 0, 0};
    int nh[NXCD] = {0, 0, 0, 0, 0, 0, 0, 0};
    // hbase[h] <- (xcd, position within the xcd), then the row offset
    for (int r = 0; r < nheads; ++r) {
      const int h = (int)(uint32_t)keys[r];
      int best = 0;
      for (int x = 1; x < NXCD; ++x)
        if (load[x] < load[best]) best = x;
      load[best] += head_count[h];
      hbase[h] = best | (nh[best]++ << 3);
    }
    int off = 0;
    for (int x = 0; x < NXCD; ++x) {
      s_off[x] = off;
      ws[AttnWs::kXcdOff + x] = off;
      ws[AttnWs::kXcdCtr + x] = 0;
      off += nh[x] * nB;
    }
    ws[AttnWs::kXcdOff + NXCD] = off;
  }
  __syncthreads();
  for (int h = threadIdx.x; h < nheads; h += kPlanThreads)
    hbase[h] = s_off[hbase[h] & 7] + (hbase[h] >> 3) * nB;
  __syncthreads();
  int32_t* xq = ws + AttnWs::xq_off() / 4;
  const int64_t rows = (int64_t)nheads * nB;
  for (int64_t t = threadIdx.x; t < rows; t += kPlanThreads) {
    const int h = (int)(t / nB);
    xq[hbase[h] + (t - (int64_t)h * nB)] = (int32_t)t;
  }
}

constexpr int kQT = 1;  // 32-query tiles per wave in the launched kernels

template <int D, int BLK, bool CH>
fva_status launch_sparse(const Problem& p, AttnArgs a, int flags, hipStream_t s) {
  const int sched = flags & 0x3;
  const bool trace = (flags & FVA_TRACE) != 0;
  constexpr int NT = attn_threads<kQT>(BLK);
  // persistent grid: as many workgroups as can be resident at once (the
  // occupancy query costs microseconds of host time, so it is asked once per
  // device and kept)
  const int cus = device_cu_count();
  static int occ_cache[64] = {0};  // 0 = not asked yet; two racing callers store the same value
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "current device");
  int per_cu = (dev >= 0 && dev < 64) ? __atomic_load_n(&occ_cache[dev], __ATOMIC_ACQUIRE) : 0;
  if (per_cu == 0) {
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &per_cu, reinterpret_cast<const void*>(&attn_kernel<D, BLK, kQT, FVA_SCHED_QUEUE, false, false, CH, 1>),
        NT, 0);
    if (e != hipSuccess) return hip_fail(e, "occupancy query");
    if (per_cu < 1) per_cu = 1;
    if (dev >= 0 && dev < 64) __atomic_store_n(&occ_cache[dev], per_cu, __ATOMIC_RELEASE);
  }
  const int64_t slots = (int64_t)cus * per_cu;
  const int64_t persist = std::min<int64_t>(p.rows, slots);
#define FVA_LAUNCH(SCH, TR, GRIDN)                                                         \
  hipLaunchKernelGGL((attn_kernel<D, BLK, kQT, SCH, false, TR, CH, 1>), dim3((unsigned)(GRIDN)), dim3(NT), \
                     0, s, a)
  // No more rows than CUs, under every schedule: one workgroup per row, with
  // teams of waves sharing each row's key sub-tiles (a launch this short is
  // bound by its longest row, not by the total work).
  if constexpr (!CH) {
    if (p.rows <= cus) {
      constexpr int T = attn_teams<D, BLK>();
      a.direct = 1;
      if (trace)
        hipLaunchKernelGGL((attn_kernel<D, BLK, kQT, FVA_SCHED_GRID, false, true, false, T>),
                           dim3((unsigned)p.rows), dim3(NT * T), 0, s, a);
      else
        hipLaunchKernelGGL((attn_kernel<D, BLK, kQT, FVA_SCHED_GRID, false, false, false, T>),
                           dim3((unsigned)p.rows), dim3(NT * T), 0, s, a);
      return hip_fail(hipGetLastError(), "sparse attention launch");
    }
  }
  // When every item fits in one wave of resident workgroups, each persistent
  // workgroup of the queue and XCD schedules would run exactly one item: one
  // plain launch with workgroup i on row i does the same work without the
  // counter reset, the XCD plan or the queue read (all items start at once,
  // so their order does not matter).
  if (sched != FVA_SCHED_STATIC && p.rows <= slots) {
    a.direct = 1;
    if (trace) FVA_LAUNCH(FVA_SCHED_GRID, true, p.rows);
    else FVA_LAUNCH(FVA_SCHED_GRID, false, p.rows);
  } else if (sched == FVA_SCHED_QUEUE) {
    hipLaunchKernelGGL(zero_counter, dim3(1), dim3(1), 0, s, a.ws);
    if (trace) FVA_LAUNCH(FVA_SCHED_QUEUE, true, persist);
    else FVA_LAUNCH(FVA_SCHED_QUEUE, false, persist);
  } else if (sched == FVA_SCHED_XCD) {
    const int nheads = p.B * p.Hh;
    hipLaunchKernelGGL(xcd_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, a.head_count, nheads,
                       p.nB, a.ws);
    a.queue = a.ws + AttnWs::xq_off() / 4;
    if (trace) FVA_LAUNCH(FVA_SCHED_XCD, true, persist);
    else FVA_LAUNCH(FVA_SCHED_XCD, false, persist);
  } else if (sched == FVA_SCHED_STATIC) {
    if (trace) FVA_LAUNCH(FVA_SCHED_STATIC, true, persist);
    else FVA_LAUNCH(FVA_SCHED_STATIC, false, persist);
  } else {
    if (trace) FVA_LAUNCH(FVA_SCHED_GRID, true, p.rows);
    else FVA_LAUNCH(FVA_SCHED_GRID, false, p.rows);
  }
#undef FVA_LAUNCH
  return hip_fail(hipGetLastError(), "sparse attention launch");
}

template <int D, int BLK>
fva_status launch_t(const Problem& p, AttnArgs a, int flags, bool dense, hipStream_t s) {
  if (dense) {
    constexpr int NT = attn_threads<kQT>(BLK);
    constexpr int T = attn_teams<D, BLK>();
    if (p.rows <= device_cu_count())  // as for the sparse kernel
      hipLaunchKernelGGL((attn_kernel<D, BLK, kQT, FVA_SCHED_GRID, true, false, false, T>),
                         dim3((unsigned)p.rows), dim3(NT * T), 0, s, a);
    else
      hipLaunchKernelGGL((attn_kernel<D, BLK, kQT, FVA_SCHED_GRID, true, false, false, 1>),
                         dim3((unsigned)p.rows), dim3(NT), 0, s, a);
    return hip_fail(hipGetLastError(), "dense attention launch");
  }
  return p.nB > kColChunk ? launch_sparse<D, BLK, true>(p, a, flags, s)
                          : launch_sparse<D, BLK, false>(p, a, flags, s);
}

// Attention workspace for callers that cannot allocate: every device that
// loads the library holds its own copy of this array until the process ends.
// Host code uses only the device address that hipGetSymbolAddress returns
// for it (per device), never the array's name.
static __device__ __align__(256) char scratch[FVA_NOALLOC_ATTN_WS_MAX];

}  // namespace

size_t attn_ws_bytes(const Problem& p) { return AttnWs::bytes(p.rows); }

fva_status noalloc_attn_ws(void** out) {
  static std::mutex mu;
  static void* ptrs[64] = {nullptr};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "current device");
  if (dev < 0 || dev >= 64) return fail(FVA_ERR_UNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lk(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "scratch symbol address");
    if (!p) return fail(FVA_ERR_HIP, "scratch symbol address is null");
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return FVA_OK;
}

fva_status launch_attn(const Problem& p, const void* qr, const void* kr, const void* vt,
                       void* out, const fva_mask* m, float scale, int flags, void* ws,
                       void* trace, void* lse, bool dense, hipStream_t s) {
  AttnArgs a;
  a.qr = (const uint16_t*)qr;
  a.kr = (const uint16_t*)kr;
  a.vt = (const uint16_t*)vt;
  a.out = (uint16_t*)out;
  a.row_count = m ? m->row_count : nullptr;
  a.head_count = m ? m->head_count : nullptr;
  a.col_idx = m ? m->col_idx : nullptr;
  a.queue = m ? m->queue : nullptr;
  a.ws = (int32_t*)ws;
  a.trace = (uint32_t*)trace;
  a.lse = (float*)lse;
  a.N = p.N;
  a.Npad = p.Npad;
  a.rows = p.rows;
  a.nB = p.nB;
  a.sl2 = scale * 1.4426950408889634f;
  a.isl2 = 1.0f / a.sl2;
  a.direct = 0;
  if (p.d == 128 && p.BLK == 128) return launch_t<128, 128>(p, a, flags, dense, s);
  if (p.d == 128 && p.BLK == 64) return launch_t<128, 64>(p, a, flags, dense, s);
  if (p.d == 64 && p.BLK == 128) return launch_t<64, 128>(p, a, flags, dense, s);
  return launch_t<64, 64>(p, a, flags, dense, s);
}

}  // namespace fva
