// Block-sparse flash attention for gfx950 (FVAttn page, section 2: only the
// selected query-key block pairs are evaluated; section 3.2: work is balanced
// on the realized per-row workload, here by a persistent heaviest-first queue).
//
// Work item = one query block (BLK rows) of one head.  A workgroup has two
// groups of BLK/32 waves; each wave owns 32 queries.  The selected key blocks
// of the row are cut into 64-key sub-tiles; a pipeline stage holds two
// sub-tiles (one per group) of K and V in LDS, double-buffered and filled by
// direct HBM->LDS loads (global_load_lds_dwordx4), so each group runs its own
// online softmax over half of the sub-tiles and the two partial results are
// merged through LDS at the end of the item.
//
// Products use v_mfma_f32_32x32x16_bf16 in transposed form:
//   S^T (keys x queries) = K * Q^T     A = K from LDS, B = Q^T in registers
//   O^T (d x queries)   += V^T * P^T   A = V^T from LDS, B = P^T in registers
// With queries on the MFMA column axis every lane holds one query's column,
// so the running max, sum and the rescale of O are lane-local (one cross-half
// exchange per tile for the max).  P^T leaves the S accumulator in exactly the
// B-operand order the PV product needs once the V^T chunk stores key slots
// with bits 2 and 3 swapped (done by the reorder kernel).
#include <algorithm>

#include "fva_internal.hpp"

namespace fva {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int KT = 64;  // keys per sub-tile

__device__ __forceinline__ uint32_t f2bf_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ void g2lds16(const void* g, char* lds_uniform) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_uniform, 16, 0,
                                   0);
}

// K sub-tile: 64 rows (keys) x D bf16; 16-byte chunk c of row r lives at
// physical chunk c ^ swz(r).  V^T sub-tile: D rows (channels) x 64 slots.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
__device__ __forceinline__ int swz_v(int r) { return (r >> 1) & 7; }

struct AttnArgs {
  const uint16_t* qr;
  const uint16_t* kr;
  const uint16_t* vt;
  uint16_t* out;
  const int32_t* row_count;
  const int16_t* col_idx;
  const int32_t* queue;
  int32_t* counter;
  uint32_t* trace;
  int64_t N, Npad;
  int64_t rows;
  int nB;
  float sl2;  // scale * log2(e)
};

template <int D, int BLK, int SCHED, bool DENSE, bool TRACE>
__global__ __launch_bounds__(BLK * 4) void attn_kernel(AttnArgs a) {
  constexpr int NT = BLK * 4;            // threads
  constexpr int NW = NT / 64;            // waves
  constexpr int GW = NW / 2;             // waves per group
  constexpr int TILE = KT * D * 2;       // bytes of one K or V^T sub-tile
  constexpr int STAGE = 4 * TILE;        // K0, V0, K1, V1
  constexpr int NSUB = BLK / KT;         // sub-tiles per key block
  constexpr int KSTEPS = D / 16;         // MFMA k-steps over the head dim
  constexpr int DT = D / 32;             // 32-row tiles of the head dim
  constexpr int CPR = D / 8;             // 16-byte chunks per K row
  constexpr int LOADS = STAGE / 16 / NT; // 16-byte loads per thread per stage
  static_assert(LOADS * 16 * NT == STAGE, "stage size");
  __shared__ __attribute__((aligned(16))) char lds[2 * STAGE];
  __shared__ int s_item;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave / GW;             // 0 or 1
  const int wq = wave % GW;              // query sub-block of this wave
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  int64_t item, item_end = 0;
  if (SCHED == FVA_SCHED_STATIC) {
    const int64_t G = gridDim.x;
    item = (int64_t)blockIdx.x * a.rows / G;
    item_end = ((int64_t)blockIdx.x + 1) * a.rows / G;
  } else if (SCHED == FVA_SCHED_QUEUE) {
    if (tid == 0) s_item = atomicAdd(a.counter, 1);
    __syncthreads();
    item = s_item;
  } else {
    item = blockIdx.x;
  }

  while (true) {
    if (SCHED == FVA_SCHED_STATIC) {
      if (item >= item_end) break;
    } else if (item >= a.rows) {
      break;
    }
    uint64_t t_start = 0;
    if (TRACE && tid == 0) t_start = __builtin_amdgcn_s_memrealtime();
    int64_t row;
    if (DENSE || SCHED == FVA_SCHED_STATIC) row = item;
    else row = a.queue[item];
    row = __builtin_amdgcn_readfirstlane((int)row);
    const int64_t bh = row / a.nB;
    const int qb = (int)(row - bh * a.nB);
    const int cnt = DENSE ? a.nB : __builtin_amdgcn_readfirstlane(a.row_count[row]);
    const int16_t* cols = a.col_idx + row * a.nB;
    const int64_t nlast = a.N - (int64_t)(a.nB - 1) * BLK;  // real keys of the last block
    int U = cnt * NSUB;
    if (cnt > 0) {
      const int lastcol = DENSE ? a.nB - 1 : (int)cols[cnt - 1];
      if (lastcol == a.nB - 1) U -= NSUB - (int)((nlast + KT - 1) / KT);
    }
    const int nstage = (U + 1) >> 1;

    const uint16_t* kbase = a.kr + bh * a.Npad * D;
    const uint16_t* vbase = a.vt + bh * a.Npad * D;  // vt64: chunk c at c*64*D

    // issue the loads of stage s into buffer s&1
    auto load_stage = [&](int s) {
      char* buf = lds + (s & 1) * STAGE;
#pragma unroll
      for (int k = 0; k < LOADS; ++k) {
        const int L0 = (k * NW + wave) * 64;        // first chunk of this wave's group
        const int part = L0 / (TILE / 16);          // 0:K0 1:V0 2:K1 3:V1
        const int g = part >> 1;
        const int u = 2 * s + g;
        if (u >= U) continue;                       // wave-uniform
        const int t = u / NSUB, half = u % NSUB;
        const int kb = DENSE ? t : (int)cols[t];
        const int64_t key0 = (int64_t)kb * BLK + half * KT;
        const int slot = (L0 % (TILE / 16)) + lane;
        const void* src;
        if ((part & 1) == 0) {
          const int r = slot / CPR, p = slot % CPR;
          const int c = p ^ swz_k<D>(r);
          src = kbase + (key0 + r) * D + c * 8;
        } else {
          const int r = slot / 8, p = slot % 8;
          const int c = p ^ swz_v(r);
          src = vbase + (key0 / KT) * (int64_t)(KT * D) + r * KT + c * 8;
        }
        g2lds16(src, buf + L0 * 16);
      }
    };

    // Q^T operand: this wave's 32 queries, lane holds query l32, d chunk 2kk+hl
    const int64_t q0 = (int64_t)qb * BLK + wq * 32;
    bf16x8 qop[KSTEPS];
    {
      const uint16_t* qp = a.qr + (bh * a.Npad + q0 + l32) * D + hl * 8;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) qop[kk] = as_bf16x8(*(const u32x4*)(qp + kk * 16));
    }

    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    if (nstage > 0) load_stage(0);
    for (int s = 0; s < nstage; ++s) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (s + 1 < nstage) load_stage(s + 1);
      const int u = 2 * s + grp;
      if (u < U) {
        const char* kt = lds + (s & 1) * STAGE + (2 * grp) * TILE;
        const char* vtile = kt + TILE;
        // S^T = K Q^T for keys 32m + (row) of this sub-tile
        f32x16 sacc[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[m][r] = 0.f;
          const int kr_ = 32 * m + l32;
#pragma unroll
          for (int kk = 0; kk < KSTEPS; ++kk) {
            const int c = (2 * kk + hl) ^ swz_k<D>(kr_);
            const bf16x8 kop = as_bf16x8(*(const u32x4*)(kt + kr_ * (D * 2) + c * 16));
            sacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[kk], sacc[m], 0, 0, 0);
          }
        }
        // keys of this sub-tile that are real
        const int t = u / NSUB, half = u % NSUB;
        const int kb = DENSE ? t : (int)cols[t];
        const int64_t key0 = (int64_t)kb * BLK + half * KT;
        const int kvalid = (int)min((int64_t)KT, a.N - key0);
        float mx = -INFINITY;
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float x = sacc[m][r] * a.sl2;
            if (kvalid < KT) {
              const int key = 32 * m + 8 * (r >> 2) + 4 * hl + (r & 3);
              if (key >= kvalid) x = -INFINITY;
            }
            sacc[m][r] = x;
            mx = fmaxf(mx, x);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        float psum = 0.f;
        bf16x8 pop[2][2];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            u32x4 pk;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float p0 = __builtin_amdgcn_exp2f(sacc[m][8 * b + 2 * e] - m_use);
              const float p1 = __builtin_amdgcn_exp2f(sacc[m][8 * b + 2 * e + 1] - m_use);
              psum += p0 + p1;
              pk[e] = f2bf_rne(p0) | (f2bf_rne(p1) << 16);
            }
            pop[m][b] = as_bf16x8(pk);
          }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
        // O^T += V^T P^T
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int vr = 32 * dt + l32;
#pragma unroll
          for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
              const int c = (4 * m + 2 * b + hl) ^ swz_v(vr);
              const bf16x8 vop = as_bf16x8(*(const u32x4*)(vtile + vr * (KT * 2) + c * 16));
              oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[m][b], oacc[dt], 0, 0, 0);
            }
        }
      }
    }
    // merge the two groups' partial results through LDS
    __syncthreads();
    float* mrg = (float*)lds + wq * (2 + 16 * DT) * 64;
    if (grp == 1) {
      mrg[0 * 64 + lane] = m_run;
      mrg[1 * 64 + lane] = l_run;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mrg[(2 + dt * 16 + r) * 64 + lane] = oacc[dt][r];
    }
    __syncthreads();
    if (grp == 0) {
      const float m1 = mrg[lane], l1 = mrg[64 + lane];
      const float mm = fmaxf(m_run, m1);
      const float mu = mm == -INFINITY ? 0.f : mm;
      const float a0 = __builtin_amdgcn_exp2f(m_run - mu);
      const float a1 = __builtin_amdgcn_exp2f(m1 - mu);
      float l = l_run * a0 + l1 * a1;
      l += __shfl_xor(l, 32, 64);
      const float inv = l > 0.f ? 1.f / l : 0.f;
      const int64_t q = q0 + l32;
      const bool real = q < a.N;
      uint16_t* op = a.out + (bh * a.Npad + q) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u32x2 w;
          float v[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = 4 * i + j;
            const float o = oacc[dt][r] * a0 + mrg[(2 + dt * 16 + r) * 64 + lane] * a1;
            v[j] = real ? o * inv : 0.f;
          }
          w.x = f2bf_rne(v[0]) | (f2bf_rne(v[1]) << 16);
          w.y = f2bf_rne(v[2]) | (f2bf_rne(v[3]) << 16);
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
    // next item
    if (SCHED == FVA_SCHED_STATIC) {
      ++item;
      __syncthreads();
    } else if (SCHED == FVA_SCHED_QUEUE) {
      if (tid == 0) s_item = atomicAdd(a.counter, 1);
      __syncthreads();
      item = s_item;
    } else {
      break;
    }
  }
}

__global__ void zero_counter(int32_t* c) { c[0] = 0; }

template <int D, int BLK>
fva_status launch_t(const Problem& p, const AttnArgs& a, int flags, bool dense, hipStream_t s) {
  const int sched = flags & 0x3;
  const bool trace = (flags & FVA_TRACE) != 0;
  constexpr int NT = BLK * 4;
  if (dense) {
    hipLaunchKernelGGL((attn_kernel<D, BLK, FVA_SCHED_GRID, true, false>), dim3((unsigned)p.rows),
                       dim3(NT), 0, s, a);
    return hip_fail(hipGetLastError(), "dense attention launch");
  }
  // persistent grid: as many workgroups as can be resident at once
  const int cus = device_cu_count();
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &per_cu, reinterpret_cast<const void*>(&attn_kernel<D, BLK, FVA_SCHED_QUEUE, false, false>),
      NT, 0);
  if (e != hipSuccess) return hip_fail(e, "occupancy query");
  if (per_cu < 1) per_cu = 1;
  const int64_t persist = std::min<int64_t>(p.rows, (int64_t)cus * per_cu);
#define FVA_LAUNCH(SCH, TR, GRIDN)                                                         \
  hipLaunchKernelGGL((attn_kernel<D, BLK, SCH, false, TR>), dim3((unsigned)(GRIDN)), dim3(NT), \
                     0, s, a)
  if (sched == FVA_SCHED_QUEUE) {
    hipLaunchKernelGGL(zero_counter, dim3(1), dim3(1), 0, s, a.counter);
    if (trace) FVA_LAUNCH(FVA_SCHED_QUEUE, true, persist);
    else FVA_LAUNCH(FVA_SCHED_QUEUE, false, persist);
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

}  // namespace

fva_status launch_attn(const Problem& p, const void* qr, const void* kr, const void* vt,
                       void* out, const fva_mask* m, float scale, int flags, void* ws,
                       void* trace, bool dense, hipStream_t s) {
  AttnArgs a;
  a.qr = (const uint16_t*)qr;
  a.kr = (const uint16_t*)kr;
  a.vt = (const uint16_t*)vt;
  a.out = (uint16_t*)out;
  a.row_count = m ? m->row_count : nullptr;
  a.col_idx = m ? m->col_idx : nullptr;
  a.queue = m ? m->queue : nullptr;
  a.counter = (int32_t*)ws;
  a.trace = (uint32_t*)trace;
  a.N = p.N;
  a.Npad = p.Npad;
  a.rows = p.rows;
  a.nB = p.nB;
  a.sl2 = scale * 1.4426950408889634f;
  if (p.d == 128 && p.BLK == 128) return launch_t<128, 128>(p, a, flags, dense, s);
  if (p.d == 128 && p.BLK == 64) return launch_t<128, 64>(p, a, flags, dense, s);
  if (p.d == 64 && p.BLK == 128) return launch_t<64, 128>(p, a, flags, dense, s);
  return launch_t<64, 64>(p, a, flags, dense, s);
}

}  // namespace fva
