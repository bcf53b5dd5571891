/*
 * fva.h - C ABI of libfva, adaptive block-sparse self-attention for video
 * diffusion transformers on AMD Instinct MI355X (gfx950).
 *
 * The operations follow "FVAttn: Adaptive Sparse Attention with Runtime Load
 * Balancing for Video Generation" (papers.paperslantern.ai/papers/2607.16190):
 *   - video-aware block organization of the T x H x W latent token grid
 *     (section 3.1),
 *   - the sparse-routing frontend: block similarities from pooled Q/K, a Top-p
 *     CDF threshold with a Top-k safety floor, per-head workload and the
 *     key-block importance order (sections 2 and 3.1),
 *   - slack-aware augmentation, here a per-head top-up of further high-score
 *     blocks up to a pair budget (section 3.3),
 *   - block-sparse attention computed for the chosen (query block, key block)
 *     pairs alone (section 2), run as a persistent kernel over a heaviest-first
 *     work queue, the one-GPU counterpart of runtime load balancing
 *     (section 3.2).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates or frees device memory.
 *   - Work is enqueued on `stream`; no call synchronizes with the host.
 *   - Arguments are validated on the host before anything is launched.  A
 *     negative fva_status is returned on failure and fva_last_error() gives a
 *     thread-local message.  Nothing is launched when validation fails.
 *   - bf16 tensors are IEEE bfloat16 stored as uint16.
 *   - Supported: head dim d in {64, 128}; block size BLK = bt*bh*bw in
 *     {64, 128}; number of blocks nB <= 32767 (int16 column indices);
 *     B*Hh*nB < 2^31.  Other shapes return FVA_ERR_UNSUPPORTED.
 *   - Calls are reentrant (no global mutable state) apart from the per-thread
 *     error string.
 *
 * Shapes (N = T*H*W tokens, BLK tokens per block, nB = ceil(N/BLK) blocks,
 * Npad = nB*BLK):
 *   token-major   [B, N, Hh, d]  the DiT layout, element strides given by caller
 *   rows          [B, Hh, Npad, d] reordered, contiguous, pad rows zero
 *   k64           [B, Hh, Npad/64, d/8, 64, 8] reordered K in 64-token tiles:
 *                 element (c, r, e) of tile t is channel 8c+e of token 64t+r
 *   v64           [B, Hh, Npad/64, 8, d, 8] reordered V in 64-token tiles:
 *                 element (g, e, q) of tile t is channel e of token 64t+k
 *                 where k is slot 8g+q with bits 2 and 3 swapped
 *   (the tile layouts are the order in which the attention kernel's MFMA
 *   operands are read, so a tile is copied to LDS verbatim; pad tokens zero)
 */
#ifndef FVA_H
#define FVA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FVA_OK = 0,
  FVA_ERR_INVALID_ARG = -1,   /* null pointer, non-positive size, bad flag   */
  FVA_ERR_UNSUPPORTED = -2,   /* valid but outside the supported shapes      */
  FVA_ERR_WORKSPACE = -3,     /* workspace missing or too small              */
  FVA_ERR_HIP = -4            /* a HIP runtime call or launch failed         */
} fva_status;

/* Latent grid T x H x W and block shape bt x bh x bw (section 3.1). */
typedef struct {
  int32_t T, H, W;
  int32_t bt, bh, bw;
} fva_grid;

/* Derived sizes of a problem. */
typedef struct {
  int64_t N;                 /* tokens                                      */
  int64_t Npad;              /* nB * BLK                                    */
  int32_t BLK;               /* tokens per block                            */
  int32_t nB;                /* blocks per head                             */
  int32_t words;             /* 32-bit words per bitmask row = ceil(nB/32)   */
  int32_t reserved;
  int64_t rows;              /* B*Hh*nB routing rows = attention work items  */
  size_t route_ws_bytes;     /* workspace fva_route needs                    */
  size_t attn_ws_bytes;      /* workspace fva_sparse_attn needs              */
  size_t trace_bytes;        /* bytes of an FVA_TRACE buffer (32 per item)   */
} fva_sizes_t;

/* Routing parameters (sections 2 and 3.1; top-up: section 3.3). */
typedef struct {
  float top_p;               /* Top-p threshold, used at its float32 value.
                                p >= 1 keeps every block, p <= 0 none.       */
  int32_t topk_floor;        /* Top-k safety floor, absolute block count >= 0 */
  int64_t aug_budget;        /* per-head pair budget for the top-up; 0 = off  */
  float scale;               /* score scale; <= 0 selects 1/sqrt(d)          */
  int32_t reserved;
} fva_route_params;

/* The block mask and its derived metadata; all DEVICE pointers, caller-owned.
 * Row index r = (b*Hh + h)*nB + i for query block i of head h in batch b.   */
typedef struct {
  float* scores;             /* [rows, nB] float32 pooled block scores       */
  uint32_t* bitmask;         /* [rows, words]; bit j%32 of word j/32 = M(h,i,j) */
  int32_t* row_count;        /* [rows] selected key blocks per row            */
  int16_t* col_idx;          /* [rows, nB] selected key blocks, ascending;
                                entries past row_count are unspecified       */
  int32_t* head_count;       /* [B*Hh] W_h = selected pairs of the head       */
  int32_t* queue;            /* [rows] row ids, row_count descending, ties by
                                row id ascending (heaviest first)            */
} fva_mask;

/* fva_route flags */
#define FVA_ROUTE_SCORES_IN 0x1  /* skip pooling and scoring: route from
                                    mask->scores as given                    */
#define FVA_ROUTE_POOLED_IN 0x2  /* skip pooling: qr and kr point to the
                                    float32 block means [B*Hh, nB, d] of Q and
                                    K that fva_reorder_pool wrote            */

/* fva_sparse_attn flags: schedule of (head, query-block) work items */
#define FVA_SCHED_QUEUE  0x0  /* persistent workgroups pop the heaviest-first
                                 queue through an atomic counter (default)   */
#define FVA_SCHED_STATIC 0x1  /* persistent workgroups take contiguous runs of
                                 rows in row order (fixed placement)         */
#define FVA_SCHED_GRID   0x2  /* one workgroup per queue entry, hardware
                                 dispatch                                    */
#define FVA_SCHED_XCD    0x3  /* persistent, XCD-aware: heads placed on the
                                 8 XCDs heaviest first (longest-processing-
                                 time on W_h); each XCD pops its heads' rows
                                 in query-block order and steals from the
                                 others when it runs dry (at most 4096 heads) */
#define FVA_TRACE        0x10 /* write one trace record per item             */

/* fva_reorder directions and layouts */
#define FVA_FORWARD 0
#define FVA_INVERSE 1
#define FVA_LAYOUT_ROWS 0
#define FVA_LAYOUT_V64 1
#define FVA_LAYOUT_K64 2

/* Sizes of a problem and the workspaces it needs.  B, Hh > 0; d as above.
 * Returns FVA_ERR_UNSUPPORTED for shapes outside the supported set.        */
fva_status fva_sizes(const fva_grid* grid, int32_t B, int32_t Hh, int32_t d,
                     fva_sizes_t* out);

/* Video-aware block organization (section 3.1).  Reordered position r holds
 * the token visited r-th when tiles of bt x bh x bw are walked in raster
 * order (tile frame, tile row, tile column; edge tiles clipped) and tokens
 * inside a tile in raster order (t, y, x).  Positions N..Npad-1 are padding.
 *
 * FVA_FORWARD: src is token-major [B, N, Hh, d] with element strides
 *   strides[0..2] for (b, n, h) and unit channel stride; dst is `rows`
 *   (FVA_LAYOUT_ROWS), `k64` (FVA_LAYOUT_K64) or `v64` (FVA_LAYOUT_V64);
 *   pad tokens are written as zero.
 * FVA_INVERSE: src is `rows`; dst is token-major [B, N, Hh, d] with element
 *   strides strides[0..2]; pad rows are dropped.  Layout must be ROWS.
 * Pointers and strides must be 16-byte aligned (strides multiples of 8).
 * src and dst must not overlap.                                             */
fva_status fva_reorder(const void* src, void* dst, int32_t B, int32_t Hh, int32_t d,
                       const fva_grid* grid, const int64_t strides[3],
                       int32_t direction, int32_t layout, hipStream_t stream);

/* Tile orders for the block organization (section 3.1): tiles may be visited
 * along a 3-D Hilbert index, which keeps tiles that neighbour each other in
 * the video grid close together in the block sequence. */
#define FVA_ORDER_RASTER 0   /* tiles in raster order (what fva_reorder uses)   */
#define FVA_ORDER_HILBERT 1  /* tiles by their 3-D Hilbert index over (tile
                                frame, tile row, tile column) on the bounding
                                2^m cube, out-of-grid cells skipped          */

/* Bytes of the device tile table for `grid` (at most 8192 tiles). */
fva_status fva_tile_order_bytes(const fva_grid* grid, size_t* bytes);

/* Writes the tile table of `order` for `grid` into the DEVICE buffer `table`
 * (fva_tile_order_bytes() bytes, 16-byte aligned): a header of 12 int32
 * {ntiles, order, status = 0, T, H, W, bt, bh, bw, 0, 0, 0}, then the raster
 * id of the k-th tile (ntiles entries), then the first reordered position of
 * the k-th tile (ntiles + 1 entries, the last = N).  Tokens inside a tile stay
 * in raster order.                                                          */
fva_status fva_tile_order(const fva_grid* grid, int32_t order, void* table, size_t table_bytes,
                          hipStream_t stream);

/* fva_reorder with the tile order taken from a table written by
 * fva_tile_order for the SAME grid and block shape (DEVICE pointer, 16-byte
 * aligned); table = NULL is raster order.  All other arguments and layouts
 * are as for fva_reorder.  The kernels compare the table's header with
 * `grid` and check every entry they use before indexing with it: a table of
 * another grid, or a damaged one, never makes them read outside the table or
 * the source.  Positions they cannot place are written as zero (forward) or
 * not written (inverse), and the table's status word (header word 2) is set
 * to 1; read it with fva_tile_table_status.                                 */
fva_status fva_reorder_ex(const void* src, void* dst, int32_t B, int32_t Hh, int32_t d,
                          const fva_grid* grid, void* table, const int64_t strides[3],
                          int32_t direction, int32_t layout, hipStream_t stream);

/* Forward block organization (as fva_reorder_ex, FVA_FORWARD) that also
 * writes the block means the router pools (sections 2 and 3.1): pooled
 * (DEVICE, float32 [B*Hh, nB, d], 16-byte aligned, caller-owned) gets, for
 * every head (b, h) and block i, the mean over the block's real tokens of
 * their d channels (pad positions are not counted), summed in float32.
 * layout: FVA_LAYOUT_ROWS (for Q) or FVA_LAYOUT_K64 (for K); dst is written
 * exactly as fva_reorder_ex writes it.  table: NULL (raster tile order) or a
 * tile table of this grid, checked as for fva_reorder_ex (positions that
 * cannot be placed get zeros in dst and count as zero rows in their block's
 * mean).  Pass the two means to fva_route with FVA_ROUTE_POOLED_IN in
 * place of qr and kr; this saves the router's second read of Q and K.      */
fva_status fva_reorder_pool(const void* src, void* dst, void* pooled, int32_t B, int32_t Hh,
                            int32_t d, const fva_grid* grid, void* table,
                            const int64_t strides[3], int32_t layout, hipStream_t stream);

/* Copies a tile table's status word (0 = every lookup so far was consistent,
 * 1 = a reorder found the table does not belong to its grid) to *status_out
 * (host), synchronously on `stream`.                                        */
fva_status fva_tile_table_status(const void* table, int32_t* status_out, hipStream_t stream);

/* Sparse-routing frontend (sections 2 and 3.1; top-up section 3.3).
 * qr: `rows` bf16, kr: `k64` bf16 (with FVA_ROUTE_POOLED_IN: the float32
 * block means of Q and K from fva_reorder_pool).  For every row (b, h, i):
 *   1. unless FVA_ROUTE_SCORES_IN: qbar, kbar = mean of each block's real
 *      tokens (read from qr and kr with FVA_ROUTE_POOLED_IN);
 *      scores[r, j] = (qbar_i . kbar_j) * scale in float32;
 *   2. importance order = key blocks by score descending, ties by index
 *      ascending (-0 == +0);
 *   3. float64 softmax of the row accumulated along that order; the Top-p set
 *      is the shortest prefix whose cumulative share reaches top_p; the row
 *      keeps max(that length, topk_floor) blocks, at most nB;
 *   4. bitmask, row_count, col_idx and head_count are written;
 *   5. if aug_budget > 0, every head whose W_h is below the budget gains the
 *      (aug_budget - W_h) unselected pairs of highest score (ties: query block
 *      ascending, then key block ascending) and its rows are rewritten;
 *   6. queue = rows ordered heaviest first.
 * ws must hold fva_sizes().route_ws_bytes bytes, 256-byte aligned.  A NaN
 * score sets bit 0 of the first 32-bit word of ws (read it with
 * fva_route_flags after the stream completes); routing of that row is then
 * unspecified but stays in bounds.                                          */
fva_status fva_route(const void* qr, const void* kr, int32_t B, int32_t Hh, int32_t d,
                     const fva_grid* grid, const fva_route_params* params,
                     const fva_mask* mask, void* ws, size_t ws_bytes, int32_t flags,
                     hipStream_t stream);

/* Copies the routing status word from a route workspace to *flags_out (host)
 * synchronously on `stream`.  Bit 0: a NaN score was seen.                 */
fva_status fva_route_flags(const void* ws, uint32_t* flags_out, hipStream_t stream);

/* Block-sparse attention (section 2: the mask decides which (query block,
 * key block) pairs are computed).  For each real query token of block i of
 * head (b, h):
 *   out = sum over the real keys of the selected key blocks of
 *         softmax_k((q . k) * scale) * v_k,
 * computed with bf16 MFMA products, float32 accumulation and an online
 * softmax.  Rows with no selected block, and pad rows, are written as zero.
 * Inputs must be finite: the kernels are compiled without NaN semantics, so
 * a NaN or infinity in Q, K or V gives an unspecified result for its rows.
 * qr: `rows` bf16; kr: `k64` bf16; vt: `v64` bf16; out: `rows` bf16.
 * scale <= 0 selects 1/sqrt(d).  flags: one FVA_SCHED_* value, optionally
 * | FVA_TRACE.  The schedule changes where and when rows run, never their
 * bits: every schedule computes each row the same way.  (A launch with no
 * more rows than the device has CUs runs one workgroup per row under every
 * schedule, with teams of waves sharing the row's key blocks; fva_dense_attn
 * does the same for such problems.)  ws: fva_sizes().attn_ws_bytes bytes, 256-byte aligned
 * (scheduler counters and lists; contents need not be initialized).
 * trace (with FVA_TRACE): trace_bytes bytes; record k (8 x uint32) describes
 * the k-th processed queue entry: {row, XCC_ID, HW_ID, workgroup id,
 * t0 lo, t0 hi, t1 lo, t1 hi} with t = s_memrealtime ticks (100 MHz).
 * lse (optional, NULL to skip): float32 [B*Hh, N], 4-byte aligned, indexed
 * by reordered query position; entry i is the natural log-sum-exp of the
 * scaled scores over the keys that query used,
 *   lse_i = log sum_k exp((q_i . k) * scale)   (-inf with no selected block).
 * Against the dense kernel's lse, exp(lse_sparse - lse_dense) is the share of
 * the query's full softmax mass that the selected blocks hold (the recall of
 * the mask; block-sparse quality is framed this way on the DFSAttn abstract
 * listed at thelatestinai.com/papers/2607.16190).                          */
fva_status fva_sparse_attn(const void* qr, const void* kr, const void* vt, void* out,
                           int32_t B, int32_t Hh, int32_t d, const fva_grid* grid,
                           const fva_mask* mask, float scale, int32_t flags,
                           void* ws, size_t ws_bytes, void* trace, void* lse,
                           hipStream_t stream);

/* fva_sparse_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and results, with the attention workspace taken from a
 * static array of FVA_NOALLOC_ATTN_WS_MAX bytes that the library holds on
 * each device until the process ends, instead of a caller buffer.  The call
 * itself allocates nothing.  Problems whose workspace would exceed that
 * (more than about 262 000 rows, fva_sizes().attn_ws_bytes) return
 * FVA_ERR_UNSUPPORTED before any launch.  Every call on one device shares
 * that device's array: calls that overlap in time on one device (two streams,
 * two threads) race and must be serialized by the caller.  The kernels
 * initialize whatever they need in it, so no clearing is required.          */
#define FVA_NOALLOC_ATTN_WS_MAX (1 << 20)
fva_status fva_sparse_attn_noalloc(const void* qr, const void* kr, const void* vt, void* out,
                                   int32_t B, int32_t Hh, int32_t d, const fva_grid* grid,
                                   const fva_mask* mask, float scale, int32_t flags,
                                   void* trace, void* lse, hipStream_t stream);

/* Dense attention over every key block with the same core: the comparator
 * for the sparse kernel.  Same layouts, output and lse conventions as above
 * (lse then sums over all real keys).                                      */
fva_status fva_dense_attn(const void* qr, const void* kr, const void* vt, void* out,
                          int32_t B, int32_t Hh, int32_t d, const fva_grid* grid,
                          float scale, void* lse, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Load balancing and slack-aware augmentation on virtual ranks (FVAttn
 * sections 3.2 and 3.3).  Host functions: all pointers are HOST pointers.
 * ---------------------------------------------------------------------- */
#define FVA_RLB_PAIRS 0           /* plans are disjoint rank swaps (involutions)  */
#define FVA_RLB_RING 1            /* every rank sends one head to rank r+1 mod R */
#define FVA_RLB_MAX_PAIR_RANKS 12 /* the pair search enumerates every matching   */

typedef struct {
  int64_t max_before;        /* critical-path rank load before balancing      */
  int64_t max_after;         /* ... after                                     */
  double mean;               /* mean rank load                                */
  double lambda_before;      /* load-imbalance factor max/mean before         */
  double lambda_after;       /* ... after                                     */
  double solve_us;           /* planner wall time                             */
  int32_t migrations;        /* ranks that send a head                        */
  int32_t reserved;
} fva_rlb_stats;

/* Runtime load balancing (section 3.2) on R virtual ranks.  head_count[h] is
 * the realized workload W_h (selected block pairs, as fva_route writes it).
 * Heads start on ranks by contiguous Ulysses placement: head h on rank
 * floor(h*R/nheads).  A plan is a permutation of the ranks in which rank r
 * sends one local head to send_to[r] and receives one; fixed points send
 * nothing (send_to[r] = send_head[r] = -1).  The plan minimizes the largest
 * rank load first and the sum of squared rank loads second (equivalently the
 * variance), exactly over the chosen topology; when no plan shortens the
 * critical path, no head moves.  Outputs: send_to[ranks], send_head[ranks]
 * (global head ids), rank_of_head[nheads] after migration, stats.
 * FVA_RLB_PAIRS needs ranks <= FVA_RLB_MAX_PAIR_RANKS.                      */
fva_status fva_rlb_plan(const int32_t* head_count, int32_t nheads, int32_t ranks,
                        int32_t topology, int32_t* send_to, int32_t* send_head,
                        int32_t* rank_of_head, fva_rlb_stats* stats);

/* Slack-aware augmentation budgets (section 3.3).  With rank loads L_r from
 * rank_of_head, rank r's slack is max_r L_r - L_r and its extra budget is
 * floor(alpha * slack) pairs (alpha = augmentation coefficient in [0, 1]),
 * split evenly over the rank's heads in ascending head id (remainder to the
 * lowest ids).  head_budget[h] = W_h + extra share, capped at
 * max(head_cap, W_h) (head_cap = nB*nB: all pairs).  rank_load_after
 * (nullable, [ranks]) receives the budgeted rank loads.  Pass head_budget to
 * fva_topup on the device.                                                  */
fva_status fva_sasa_budget(const int32_t* head_count, int32_t nheads, int32_t ranks,
                           const int32_t* rank_of_head, float alpha, int64_t head_cap,
                           int64_t* head_budget, int64_t* rank_load_after);

/* Per-head top-up of an existing mask (section 3.3, device): every head whose
 * W_h (mask->head_count) is below head_budget[h] (DEVICE int64 [B*Hh]) gains
 * the head_budget[h] - W_h unselected pairs of highest score in mask->scores
 * (ties: query block ascending, then key block ascending); bitmask, row
 * counts, column lists, head_count and the heaviest-first queue are then
 * rewritten.  ws is a route workspace (fva_sizes().route_ws_bytes).         */
fva_status fva_topup(int32_t B, int32_t Hh, int32_t d, const fva_grid* grid,
                     const int64_t* head_budget, const fva_mask* mask, void* ws,
                     size_t ws_bytes, hipStream_t stream);

/* Human-readable status name, and the calling thread's last error detail. */
const char* fva_status_string(fva_status s);
const char* fva_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* FVA_H */
