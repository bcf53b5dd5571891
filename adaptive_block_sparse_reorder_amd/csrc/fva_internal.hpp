// Internal declarations shared by the libfva translation units (HIP, gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fva.h"

namespace fva {

// ---------------------------------------------------------------- host side

// Records a thread-local error message and returns `s`.
fva_status fail(fva_status s, const char* fmt, ...);
// Maps a HIP error to FVA_ERR_HIP with a message naming `what`.
fva_status hip_fail(hipError_t e, const char* what);

struct Problem {
  int32_t B, Hh, d;
  int32_t T, H, W, bt, bh, bw;
  int64_t N, Npad;
  int32_t BLK, nB, words;
  int64_t rows;  // B*Hh*nB
};

// Validates grid/shape and fills `p`.  Returns FVA_OK or an error status.
fva_status make_problem(const fva_grid* g, int32_t B, int32_t Hh, int32_t d, Problem* p);

// Number of compute units of the current device (cached per device).
int device_cu_count();

// Route workspace layout (byte offsets, 256-aligned).
struct RouteWs {
  size_t flags_off;     // uint32 status word
  size_t qbar_off;      // float [rows, d]
  size_t kbar_off;      // float [rows, d]
  size_t thresh_off;    // uint64 [B*Hh] top-up threshold keys
  size_t tstate_off;    // [B*Hh] top-up radix-select state (16 bytes each)
  size_t thist_off;     // uint32 [B*Hh, 256] top-up radix-select histograms
  size_t qtmp_row_off;  // int32 [rows] queue sort: rows in chunk-sorted order
  size_t qtmp_rank_off; // int32 [rows] queue sort: rank inside a run of equal counts
  size_t qhist_off;     // int32 [ceil(rows/1024), nB+1] queue sort: run lengths -> offsets
  size_t total;
};
RouteWs route_ws_layout(const Problem& p);
// Bytes of the attention workspace (scheduler counters and XCD row lists).
size_t attn_ws_bytes(const Problem& p);
// Device address of the library's own attention workspace on the current
// device (FVA_NOALLOC_ATTN_WS_MAX bytes; looked up once per device).
fva_status noalloc_attn_ws(void** out);
constexpr int kMaxXcdHeads = 4096;

// Kernel launchers (each returns FVA_OK or FVA_ERR_HIP).
fva_status launch_reorder(const Problem& p, const void* src, void* dst, const int64_t st[3],
                          int direction, int layout, int32_t* table, hipStream_t s);
fva_status launch_reorder_pool(const Problem& p, const void* src, void* dst, float* pooled,
                               const int64_t st[3], int layout, int32_t* table, hipStream_t s);
fva_status launch_route(const Problem& p, const void* qr, const void* kr,
                        const fva_route_params& prm, float scale, const fva_mask& m,
                        char* ws, int flags, hipStream_t s);
fva_status launch_topup(const Problem& p, const int64_t* budgets, const fva_mask& m, char* ws,
                        hipStream_t s);
fva_status launch_attn(const Problem& p, const void* qr, const void* kr, const void* vt,
                       void* out, const fva_mask* m, float scale, int flags, void* ws,
                       void* trace, void* lse, bool dense, hipStream_t s);

// ---------------------------------------------------------------- tile tables

constexpr int kTableHeaderWords = 12;

// Tile table (device buffer written by fva_tile_order): a header of
// kTableHeaderWords int32 {ntiles, order, status, T, H, W, bt, bh, bw, 0, 0,
// 0}, then tile_id[ntiles], then start[ntiles + 1].
constexpr int kMaxTiles = 8192;
inline size_t tile_table_bytes(int64_t ntiles) {
  return 4 * kTableHeaderWords + 4 * ntiles + 4 * (ntiles + 1);
}
fva_status launch_tile_order(const Problem& p, int order, int32_t* table, hipStream_t s);
int64_t tile_count(const Problem& p);

}  // namespace fva
