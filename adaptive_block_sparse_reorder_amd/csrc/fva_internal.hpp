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
constexpr int kMaxXcdHeads = 4096;

// Kernel launchers (each returns FVA_OK or FVA_ERR_HIP).
fva_status launch_reorder(const Problem& p, const void* src, void* dst, const int64_t st[3],
                          int direction, int layout, const int32_t* table, hipStream_t s);
fva_status launch_route(const Problem& p, const void* qr, const void* kr,
                        const fva_route_params& prm, float scale, const fva_mask& m,
                        char* ws, int flags, hipStream_t s);
fva_status launch_topup(const Problem& p, const int64_t* budgets, const fva_mask& m, char* ws,
                        hipStream_t s);
fva_status launch_attn(const Problem& p, const void* qr, const void* kr, const void* vt,
                       void* out, const fva_mask* m, float scale, int flags, void* ws,
                       void* trace, void* lse, bool dense, hipStream_t s);

// ---------------------------------------------------------------- device side

// Reordered position r (< N) -> source token index.  Tokens inside a tile
// are always visited in raster order (t, y, x).  Tiles are visited either in
// raster order (closed form: every tile-frame slab covers whole frames and
// every tile row inside a slab covers whole rows, so the tile containing r
// follows from three divisions) or in the order of a tile table (tile_id[k],
// start[k] = first reordered position of the k-th tile), found by binary
// search.
struct BlockOrder {
  int32_t T, H, W, bt, bh, bw;
  const int32_t* tile_id;  // null: raster tile order
  const int32_t* start;    // [ntiles + 1]
  int32_t ntiles;
  __device__ __forceinline__ int64_t src_token(int64_t r) const {
    if (tile_id) return src_token_table(r);
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
  __device__ __forceinline__ int64_t src_token_table(int64_t r) const {
    int lo = 0, hi = ntiles;  // start[lo] <= r < start[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)start[mid] <= r) lo = mid;
      else hi = mid;
    }
    const int32_t nty = (H + bh - 1) / bh, ntx = (W + bw - 1) / bw;
    const int32_t id = tile_id[lo];
    const int32_t tt = id / (nty * ntx), ty = (id / ntx) % nty, tx = id % ntx;
    const int32_t st = min(bt, T - tt * bt), sy = min(bh, H - ty * bh), sx = min(bw, W - tx * bw);
    const int32_t o = (int32_t)(r - start[lo]);
    const int32_t t = o / (sy * sx);
    const int32_t rem = o - t * (sy * sx);
    const int32_t y = rem / sx;
    const int32_t x = rem - y * sx;
    return ((int64_t)(tt * bt + t) * H + (ty * bh + y)) * W + (tx * bw + x);
  }
};

// Tile table (device buffer written by fva_tile_order): header of 4 int32
// {ntiles, order, 0, 0}, then tile_id[ntiles], then start[ntiles + 1].
constexpr int kMaxTiles = 8192;
inline size_t tile_table_bytes(int64_t ntiles) { return 16 + 4 * ntiles + 4 * (ntiles + 1); }
fva_status launch_tile_order(const Problem& p, int order, int32_t* table, hipStream_t s);
int64_t tile_count(const Problem& p);

}  // namespace fva
