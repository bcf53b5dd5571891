// Host side of the libfva C ABI: argument validation, derived sizes,
// workspace layouts and kernel dispatch.  Declarations: include/fva.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "fva_internal.hpp"

namespace fva {

static thread_local char g_err[512] = "";

fva_status fail(fva_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

fva_status hip_fail(hipError_t e, const char* what) {
  if (e == hipSuccess) return FVA_OK;
  return fail(FVA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

fva_status make_problem(const fva_grid* g, int32_t B, int32_t Hh, int32_t d, Problem* p) {
  if (!g) return fail(FVA_ERR_INVALID_ARG, "grid is null");
  if (g->T <= 0 || g->H <= 0 || g->W <= 0 || g->bt <= 0 || g->bh <= 0 || g->bw <= 0)
    return fail(FVA_ERR_INVALID_ARG, "grid and block sizes must be positive");
  if (B <= 0 || Hh <= 0 || d <= 0) return fail(FVA_ERR_INVALID_ARG, "B, Hh, d must be positive");
  if (d != 64 && d != 128) return fail(FVA_ERR_UNSUPPORTED, "head dim %d not in {64,128}", d);
  const int64_t BLK = (int64_t)g->bt * g->bh * g->bw;
  if (BLK != 64 && BLK != 128)
    return fail(FVA_ERR_UNSUPPORTED, "block size %lld not in {64,128}", (long long)BLK);
  const int64_t N = (int64_t)g->T * g->H * g->W;
  const int64_t nB = (N + BLK - 1) / BLK;
  if (nB > 32767)
    return fail(FVA_ERR_UNSUPPORTED, "%lld blocks exceed 32767 (int16 column indices)",
                (long long)nB);
  const int64_t rows = (int64_t)B * Hh * nB;
  if (rows >= (1ll << 31)) return fail(FVA_ERR_UNSUPPORTED, "too many rows");
  p->B = B;
  p->Hh = Hh;
  p->d = d;
  p->T = g->T; p->H = g->H; p->W = g->W;
  p->bt = g->bt; p->bh = g->bh; p->bw = g->bw;
  p->N = N;
  p->BLK = (int32_t)BLK;
  p->nB = (int32_t)nB;
  p->Npad = nB * BLK;
  p->words = (int32_t)((nB + 31) / 32);
  p->rows = rows;
  return FVA_OK;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

RouteWs route_ws_layout(const Problem& p) {
  RouteWs L;
  size_t off = 0;
  L.flags_off = off;
  off += 256;
  L.qbar_off = off;
  off = align256(off + (size_t)p.rows * p.d * sizeof(float));
  L.kbar_off = off;
  off = align256(off + (size_t)p.rows * p.d * sizeof(float));
  L.thresh_off = off;
  off = align256(off + (size_t)p.B * p.Hh * sizeof(uint64_t));
  L.tstate_off = off;
  off = align256(off + (size_t)p.B * p.Hh * 24);
  L.thist_off = off;
  off = align256(off + (size_t)p.B * p.Hh * 256 * sizeof(uint32_t));
  L.qtmp_row_off = off;
  off = align256(off + (size_t)p.rows * sizeof(int32_t));
  L.qtmp_rank_off = off;
  off = align256(off + (size_t)p.rows * sizeof(int32_t));
  L.qhist_off = off;
  off = align256(off + (size_t)((p.rows + 1023) / 1024) * (p.nB + 1) * sizeof(int32_t));
  L.total = off;
  return L;
}

int device_cu_count() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lk(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static fva_status check_mask(const fva_mask* m, bool need_scores) {
  if (!m) return fail(FVA_ERR_INVALID_ARG, "mask is null");
  if ((need_scores && !m->scores) || !m->bitmask || !m->row_count || !m->col_idx ||
      !m->head_count || !m->queue)
    return fail(FVA_ERR_INVALID_ARG, "a mask buffer is null");
  return FVA_OK;
}

}  // namespace fva

using namespace fva;

extern "C" {

fva_status fva_sizes(const fva_grid* grid, int32_t B, int32_t Hh, int32_t d, fva_sizes_t* out) {
  if (!out) return fail(FVA_ERR_INVALID_ARG, "out is null");
  Problem p;
  fva_status st = make_problem(grid, B, Hh, d, &p);
  if (st != FVA_OK) return st;
  memset(out, 0, sizeof(*out));
  out->N = p.N;
  out->Npad = p.Npad;
  out->BLK = p.BLK;
  out->nB = p.nB;
  out->words = p.words;
  out->rows = p.rows;
  out->route_ws_bytes = route_ws_layout(p).total;
  out->attn_ws_bytes = attn_ws_bytes(p);
  out->trace_bytes = (size_t)p.rows * 32;
  return FVA_OK;
}

fva_status fva_reorder_ex(const void* src, void* dst, int32_t B, int32_t Hh, int32_t d,
                          const fva_grid* grid, void* table, const int64_t strides[3],
                          int32_t direction, int32_t layout, hipStream_t stream) {
  Problem p;
  fva_status st = make_problem(grid, B, Hh, d, &p);
  if (st != FVA_OK) return st;
  if (!src || !dst || !strides) return fail(FVA_ERR_INVALID_ARG, "null pointer");
  if (direction != FVA_FORWARD && direction != FVA_INVERSE)
    return fail(FVA_ERR_INVALID_ARG, "direction %d", direction);
  if (layout != FVA_LAYOUT_ROWS && layout != FVA_LAYOUT_V64 && layout != FVA_LAYOUT_K64)
    return fail(FVA_ERR_INVALID_ARG, "layout %d", layout);
  if (direction == FVA_INVERSE && layout != FVA_LAYOUT_ROWS)
    return fail(FVA_ERR_INVALID_ARG, "inverse reorder writes the token-major layout only");
  for (int i = 0; i < 3; ++i)
    if (strides[i] <= 0 || (strides[i] & 7))
      return fail(FVA_ERR_INVALID_ARG, "stride %d = %lld must be a positive multiple of 8", i,
                  (long long)strides[i]);
  if (!aligned16(src) || !aligned16(dst)) return fail(FVA_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  if (strides[2] < d) return fail(FVA_ERR_INVALID_ARG, "head stride smaller than d");
  if (table && tile_count(p) > kMaxTiles)
    return fail(FVA_ERR_UNSUPPORTED, "%lld tiles exceed %d", (long long)tile_count(p), kMaxTiles);
  if (table && !aligned16(table)) return fail(FVA_ERR_INVALID_ARG, "table must be 16-byte aligned");
  return launch_reorder(p, src, dst, strides, direction, layout, (int32_t*)table, stream);
}

fva_status fva_reorder_pool(const void* src, void* dst, void* pooled, int32_t B, int32_t Hh,
                            int32_t d, const fva_grid* grid, void* table,
                            const int64_t strides[3], int32_t layout, hipStream_t stream) {
  Problem p;
  fva_status st = make_problem(grid, B, Hh, d, &p);
  if (st != FVA_OK) return st;
  if (!src || !dst || !pooled || !strides) return fail(FVA_ERR_INVALID_ARG, "null pointer");
  if (layout != FVA_LAYOUT_ROWS && layout != FVA_LAYOUT_K64)
    return fail(FVA_ERR_INVALID_ARG, "pooling reorder writes the rows or k64 layout, not %d",
                layout);
  for (int i = 0; i < 3; ++i)
    if (strides[i] <= 0 || (strides[i] & 7))
      return fail(FVA_ERR_INVALID_ARG, "stride %d = %lld must be a positive multiple of 8", i,
                  (long long)strides[i]);
  if (!aligned16(src) || !aligned16(dst) || !aligned16(pooled))
    return fail(FVA_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  if (strides[2] < d) return fail(FVA_ERR_INVALID_ARG, "head stride smaller than d");
  if (table && tile_count(p) > kMaxTiles)
    return fail(FVA_ERR_UNSUPPORTED, "%lld tiles exceed %d", (long long)tile_count(p), kMaxTiles);
  if (table && !aligned16(table)) return fail(FVA_ERR_INVALID_ARG, "table must be 16-byte aligned");
  return launch_reorder_pool(p, src, dst, (float*)pooled, strides, layout, (int32_t*)table,
                             stream);
}

fva_status fva_reorder(const void* src, void* dst, int32_t B, int32_t Hh, int32_t d,
                       const fva_grid* grid, const int64_t strides[3], int32_t direction,
                       int32_t layout, hipStream_t stream) {
  return fva_reorder_ex(src, dst, B, Hh, d, grid, nullptr, strides, direction, layout, stream);
}

fva_status fva_tile_order_bytes(const fva_grid* grid, size_t* bytes) {
  Problem p;
  fva_status st = make_problem(grid, 1, 1, 64, &p);
  if (st != FVA_OK) return st;
  if (!bytes) return fail(FVA_ERR_INVALID_ARG, "bytes is null");
  if (tile_count(p) > kMaxTiles)
    return fail(FVA_ERR_UNSUPPORTED, "%lld tiles exceed %d", (long long)tile_count(p), kMaxTiles);
  *bytes = tile_table_bytes(tile_count(p));
  return FVA_OK;
}

fva_status fva_tile_order(const fva_grid* grid, int32_t order, void* table, size_t table_bytes,
                          hipStream_t stream) {
  size_t need = 0;
  fva_status st = fva_tile_order_bytes(grid, &need);
  if (st != FVA_OK) return st;
  if (order != FVA_ORDER_RASTER && order != FVA_ORDER_HILBERT)
    return fail(FVA_ERR_INVALID_ARG, "order %d", order);
  if (!table || table_bytes < need)
    return fail(FVA_ERR_WORKSPACE, "tile table needs %zu bytes", need);
  if (!aligned16(table)) return fail(FVA_ERR_INVALID_ARG, "table must be 16-byte aligned");
  Problem p;
  make_problem(grid, 1, 1, 64, &p);
  return launch_tile_order(p, order, (int32_t*)table, stream);
}

fva_status fva_tile_table_status(const void* table, int32_t* status_out, hipStream_t stream) {
  if (!table || !status_out) return fail(FVA_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(table)) return fail(FVA_ERR_INVALID_ARG, "table must be 16-byte aligned");
  hipError_t e = hipMemcpyAsync(status_out, (const int32_t*)table + 2, sizeof(int32_t),
                                hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  return hip_fail(e, "tile table status copy");
}

fva_status fva_route(const void* qr, const void* kr, int32_t B, int32_t Hh, int32_t d,
                     const fva_grid* grid, const fva_route_params* params, const fva_mask* mask,
                     void* ws, size_t ws_bytes, int32_t flags, hipStream_t stream) {
  Problem p;
  fva_status st = make_problem(grid, B, Hh, d, &p);
  if (st != FVA_OK) return st;
  if (!params) return fail(FVA_ERR_INVALID_ARG, "params is null");
  if (flags & ~(FVA_ROUTE_SCORES_IN | FVA_ROUTE_POOLED_IN))
    return fail(FVA_ERR_INVALID_ARG, "flags 0x%x", flags);
  if ((flags & FVA_ROUTE_SCORES_IN) && (flags & FVA_ROUTE_POOLED_IN))
    return fail(FVA_ERR_INVALID_ARG, "FVA_ROUTE_SCORES_IN and FVA_ROUTE_POOLED_IN exclude each other");
  const bool scores_in = (flags & FVA_ROUTE_SCORES_IN) != 0;
  if (!scores_in && (!qr || !kr)) return fail(FVA_ERR_INVALID_ARG, "qr/kr null");
  if (!scores_in && (!aligned16(qr) || !aligned16(kr)))
    return fail(FVA_ERR_INVALID_ARG, "qr/kr must be 16-byte aligned");
  st = check_mask(mask, true);
  if (st != FVA_OK) return st;
  if (!(params->top_p == params->top_p)) return fail(FVA_ERR_INVALID_ARG, "top_p is NaN");
  if (params->topk_floor < 0) return fail(FVA_ERR_INVALID_ARG, "topk_floor < 0");
  if (params->aug_budget < 0) return fail(FVA_ERR_INVALID_ARG, "aug_budget < 0");
  const size_t need = route_ws_layout(p).total;
  if (!ws || ws_bytes < need)
    return fail(FVA_ERR_WORKSPACE, "route workspace needs %zu bytes, got %zu", need,
                ws ? ws_bytes : (size_t)0);
  if (((uintptr_t)ws & 255u) != 0) return fail(FVA_ERR_WORKSPACE, "workspace not 256-byte aligned");
  const float scale = params->scale > 0.f ? params->scale : 1.0f / sqrtf((float)d);
  return launch_route(p, qr, kr, *params, scale, *mask, (char*)ws, flags, stream);
}

fva_status fva_topup(int32_t B, int32_t Hh, int32_t d, const fva_grid* grid,
                     const int64_t* head_budget, const fva_mask* mask, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  Problem p;
  fva_status st = make_problem(grid, B, Hh, d, &p);
  if (st != FVA_OK) return st;
  if (!head_budget) return fail(FVA_ERR_INVALID_ARG, "head_budget is null");
  st = check_mask(mask, true);
  if (st != FVA_OK) return st;
  const size_t need = route_ws_layout(p).total;
  if (!ws || ws_bytes < need)
    return fail(FVA_ERR_WORKSPACE, "route workspace needs %zu bytes, got %zu", need,
                ws ? ws_bytes : (size_t)0);
  if (((uintptr_t)ws & 255u) != 0) return fail(FVA_ERR_WORKSPACE, "workspace not 256-byte aligned");
  return launch_topup(p, head_budget, *mask, (char*)ws, stream);
}

fva_status fva_route_flags(const void* ws, uint32_t* flags_out, hipStream_t stream) {
  if (!ws || !flags_out) return fail(FVA_ERR_INVALID_ARG, "null pointer");
  hipError_t e = hipMemcpyAsync(flags_out, ws, sizeof(uint32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  return hip_fail(e, "route flags copy");
}

static fva_status attn_common(const void* qr, const void* kr, const void* vt, void* out,
                              int32_t B, int32_t Hh, int32_t d, const fva_grid* grid,
                              Problem* p) {
  fva_status st = make_problem(grid, B, Hh, d, p);
  if (st != FVA_OK) return st;
  if (!qr || !kr || !vt || !out) return fail(FVA_ERR_INVALID_ARG, "null tensor pointer");
  if (!aligned16(qr) || !aligned16(kr) || !aligned16(vt) || !aligned16(out))
    return fail(FVA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  return FVA_OK;
}

static fva_status sparse_attn_checked(const void* qr, const void* kr, const void* vt, void* out,
                                      int32_t B, int32_t Hh, int32_t d, const fva_grid* grid,
                                      const fva_mask* mask, float scale, int32_t flags,
                                      Problem* p) {
  fva_status st = attn_common(qr, kr, vt, out, B, Hh, d, grid, p);
  if (st != FVA_OK) return st;
  st = check_mask(mask, false);
  if (st != FVA_OK) return st;
  const int sched = flags & 0x3;
  if (flags & ~(0x3 | FVA_TRACE)) return fail(FVA_ERR_INVALID_ARG, "flags 0x%x", flags);
  if (sched == FVA_SCHED_XCD && (int64_t)B * Hh > kMaxXcdHeads)
    return fail(FVA_ERR_UNSUPPORTED, "FVA_SCHED_XCD supports at most %d heads", kMaxXcdHeads);
  return FVA_OK;
}

static fva_status sparse_attn_launch(const Problem& p, const void* qr, const void* kr,
                                     const void* vt, void* out, const fva_mask* mask, float scale,
                                     int32_t flags, void* ws, void* trace, void* lse,
                                     hipStream_t stream) {
  if ((flags & FVA_TRACE) && !trace) return fail(FVA_ERR_INVALID_ARG, "FVA_TRACE needs a trace buffer");
  if (!(flags & FVA_TRACE)) trace = nullptr;
  if (((uintptr_t)lse & 3u) != 0) return fail(FVA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if (!(scale > 0.f)) scale = 1.0f / sqrtf((float)p.d);
  return launch_attn(p, qr, kr, vt, out, mask, scale, flags, ws, trace, lse, false, stream);
}

fva_status fva_sparse_attn(const void* qr, const void* kr, const void* vt, void* out, int32_t B,
                           int32_t Hh, int32_t d, const fva_grid* grid, const fva_mask* mask,
                           float scale, int32_t flags, void* ws, size_t ws_bytes, void* trace,
                           void* lse, hipStream_t stream) {
  Problem p;
  fva_status st = sparse_attn_checked(qr, kr, vt, out, B, Hh, d, grid, mask, scale, flags, &p);
  if (st != FVA_OK) return st;
  const size_t need = attn_ws_bytes(p);
  if (!ws || ws_bytes < need)
    return fail(FVA_ERR_WORKSPACE, "attention workspace needs %zu bytes, got %zu", need,
                ws ? ws_bytes : (size_t)0);
  if (((uintptr_t)ws & 255u) != 0) return fail(FVA_ERR_WORKSPACE, "workspace not 256-byte aligned");
  return sparse_attn_launch(p, qr, kr, vt, out, mask, scale, flags, ws, trace, lse, stream);
}

fva_status fva_sparse_attn_noalloc(const void* qr, const void* kr, const void* vt, void* out,
                                   int32_t B, int32_t Hh, int32_t d, const fva_grid* grid,
                                   const fva_mask* mask, float scale, int32_t flags, void* trace,
                                   void* lse, hipStream_t stream) {
  Problem p;
  fva_status st = sparse_attn_checked(qr, kr, vt, out, B, Hh, d, grid, mask, scale, flags, &p);
  if (st != FVA_OK) return st;
  const size_t need = attn_ws_bytes(p);
  if (need > (size_t)FVA_NOALLOC_ATTN_WS_MAX)
    return fail(FVA_ERR_UNSUPPORTED,
                "%lld rows need %zu bytes of attention workspace; the library's own holds %d "
                "(pass a workspace to fva_sparse_attn instead)",
                (long long)p.rows, need, FVA_NOALLOC_ATTN_WS_MAX);
  void* ws = nullptr;
  st = noalloc_attn_ws(&ws);
  if (st != FVA_OK) return st;
  return sparse_attn_launch(p, qr, kr, vt, out, mask, scale, flags, ws, trace, lse, stream);
}

fva_status fva_dense_attn(const void* qr, const void* kr, const void* vt, void* out, int32_t B,
                          int32_t Hh, int32_t d, const fva_grid* grid, float scale,
                          void* lse, hipStream_t stream) {
  Problem p;
  fva_status st = attn_common(qr, kr, vt, out, B, Hh, d, grid, &p);
  if (st != FVA_OK) return st;
  if (((uintptr_t)lse & 3u) != 0) return fail(FVA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if (!(scale > 0.f)) scale = 1.0f / sqrtf((float)d);
  return launch_attn(p, qr, kr, vt, out, nullptr, scale, FVA_SCHED_GRID, nullptr, nullptr, lse,
                     true, stream);
}

const char* fva_status_string(fva_status s) {
  switch (s) {
    case FVA_OK: return "FVA_OK";
    case FVA_ERR_INVALID_ARG: return "FVA_ERR_INVALID_ARG";
    case FVA_ERR_UNSUPPORTED: return "FVA_ERR_UNSUPPORTED";
    case FVA_ERR_WORKSPACE: return "FVA_ERR_WORKSPACE";
    case FVA_ERR_HIP: return "FVA_ERR_HIP";
  }
  return "FVA_UNKNOWN_STATUS";
}

const char* fva_last_error(void) { return g_err; }

}  // extern "C"
