// Host-only driver for the C-ABI validation layer (fva_api.hip), built with
// g++ under AddressSanitizer and UBSan by tests/test_host_sanitizers.py.
// The HIP runtime calls that file makes and the kernel launchers it hands
// valid calls to are replaced by stubs here: the stubs record each launch
// (so the driver can tell which calls got past validation) and never touch
// the pointers they are given.  The driver checks hand-picked argument
// errors, then throws seeded random arguments at every entry point; it exits
// non-zero on a wrong status, and the sanitizers abort on memory errors or
// undefined behaviour.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "fva_internal.hpp"

// ---------------------------------------------------------------- stubs

static int g_launches = 0;
static fva::Problem g_last;

extern "C" {
hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) {
  *v = 256;
  return hipSuccess;
}
hipError_t hipMemcpyAsync(void* dst, const void*, size_t n, hipMemcpyKind, hipStream_t) {
  memset(dst, 0, n);  // the "device" side is never read
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
const char* hipGetErrorString(hipError_t) { return "stub"; }
}

namespace fva {
static fva_status note(const Problem& p) {
  ++g_launches;
  g_last = p;
  return FVA_OK;
}
fva_status launch_reorder(const Problem& p, const void*, void*, const int64_t*, int, int,
                          int32_t*, hipStream_t) {
  return note(p);
}
fva_status launch_reorder_pool(const Problem& p, const void*, void*, float*, const int64_t*, int,
                               int32_t*, hipStream_t) {
  return note(p);
}
fva_status launch_route(const Problem& p, const void*, const void*, const fva_route_params&,
                        float, const fva_mask&, char*, int, hipStream_t) {
  return note(p);
}
fva_status launch_topup(const Problem& p, const int64_t*, const fva_mask&, char*, hipStream_t) {
  return note(p);
}
fva_status launch_attn(const Problem& p, const void*, const void*, const void*, void*,
                       const fva_mask*, float, int, void*, void*, void*, bool, hipStream_t) {
  return note(p);
}
fva_status launch_tile_order(const Problem& p, int, int32_t*, hipStream_t) { return note(p); }
int64_t tile_count(const Problem& p) {
  return (int64_t)((p.T + p.bt - 1) / p.bt) * ((p.H + p.bh - 1) / p.bh) *
         ((p.W + p.bw - 1) / p.bw);
}
size_t attn_ws_bytes(const Problem& p) { return 256 + 4 * (size_t)p.rows; }
static char g_static_ws[256] __attribute__((aligned(256)));
fva_status noalloc_attn_ws(void** out) {
  *out = g_static_ws;
  return FVA_OK;
}
}  // namespace fva

// ---------------------------------------------------------------- helpers

static int g_fail = 0;
#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "line %d: expectation failed: %s\n", __LINE__, #cond); \
      ++g_fail;                                                       \
    }                                                                 \
  } while (0)

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd() {  // 64-bit LCG (Knuth's MMIX constants), top bits
  g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(g_state >> 33);
}
static int pick(int n) { return (int)(rnd() % (uint32_t)n); }

// stand-ins for device buffers: aligned host memory the stubs never read
alignas(256) static char g_arena[1 << 16];
static void* aligned_ptr(int k) { return g_arena + 256 * (k % 200); }
static void* any_ptr() {
  switch (pick(4)) {
    case 0: return nullptr;
    case 1: return g_arena + 1 + pick(15);  // misaligned
    default: return aligned_ptr(pick(200));
  }
}

static fva_grid grid_of(int T, int H, int W, int bt, int bh, int bw) {
  fva_grid g;
  g.T = T; g.H = H; g.W = W; g.bt = bt; g.bh = bh; g.bw = bw;
  return g;
}

static fva_grid random_grid() {
  static const int blocks[][3] = {{1, 8, 8}, {1, 8, 16}, {2, 8, 8}, {4, 4, 4}, {2, 8, 4},
                                  {1, 4, 8}, {0, 8, 8}, {1, 1, 64}, {3, 5, 7}};
  const int* b = blocks[pick(9)];
  return grid_of(pick(6) - 1 + pick(40), pick(70), pick(90), b[0], b[1], b[2]);
}

static fva_mask mask_of(bool scores) {
  fva_mask m;
  m.scores = scores ? (float*)aligned_ptr(1) : nullptr;
  m.bitmask = (uint32_t*)aligned_ptr(2);
  m.row_count = (int32_t*)aligned_ptr(3);
  m.col_idx = (int16_t*)aligned_ptr(4);
  m.head_count = (int32_t*)aligned_ptr(5);
  m.queue = (int32_t*)aligned_ptr(6);
  return m;
}

// ---------------------------------------------------------------- cases

static void fixed_cases() {
  fva_sizes_t sz;
  const fva_grid g = grid_of(5, 16, 16, 1, 8, 8);  // 1280 tokens, 20 blocks of 64
  EXPECT(fva_sizes(&g, 1, 2, 64, &sz) == FVA_OK);
  EXPECT(sz.N == 1280 && sz.Npad == 1280 && sz.nB == 20 && sz.words == 1 && sz.rows == 40);
  EXPECT(fva_sizes(&g, 1, 2, 96, &sz) == FVA_ERR_UNSUPPORTED);
  EXPECT(strstr(fva_last_error(), "head dim") != nullptr);
  EXPECT(fva_sizes(nullptr, 1, 2, 64, &sz) == FVA_ERR_INVALID_ARG);
  EXPECT(fva_sizes(&g, 0, 2, 64, &sz) == FVA_ERR_INVALID_ARG);
  EXPECT(fva_sizes(&g, 1, 2, 64, nullptr) == FVA_ERR_INVALID_ARG);
  const fva_grid most = grid_of(1, 1, 32767 * 64, 1, 1, 64);
  EXPECT(fva_sizes(&most, 1, 1, 64, &sz) == FVA_OK && sz.nB == 32767);
  const fva_grid over = grid_of(1, 1, 32768 * 64, 1, 1, 64);
  EXPECT(fva_sizes(&over, 1, 1, 64, &sz) == FVA_ERR_UNSUPPORTED);
  const fva_grid rows = grid_of(1, 1, 32767 * 64, 1, 1, 64);  // 2 * 40000 * 32767 >= 2^31 rows
  EXPECT(fva_sizes(&rows, 2, 40000, 64, &sz) == FVA_ERR_UNSUPPORTED);
  EXPECT(fva_sizes(&rows, 1, 65536, 64, &sz) == FVA_OK);      // 2^31 - 65536 rows

  const int64_t st[3] = {1280 * 2 * 64, 2 * 64, 64};
  void* a = aligned_ptr(10);
  void* b = aligned_ptr(11);
  int before = g_launches;
  EXPECT(fva_reorder(a, b, 1, 2, 64, &g, st, FVA_FORWARD, FVA_LAYOUT_ROWS, nullptr) == FVA_OK);
  EXPECT(g_launches == before + 1 && g_last.nB == 20 && g_last.rows == 40);
  before = g_launches;
  EXPECT(fva_reorder(a, b, 1, 2, 64, &g, st, FVA_INVERSE, FVA_LAYOUT_K64, nullptr) ==
         FVA_ERR_INVALID_ARG);
  EXPECT(fva_reorder(a, b, 1, 2, 64, &g, st, 7, FVA_LAYOUT_ROWS, nullptr) == FVA_ERR_INVALID_ARG);
  EXPECT(fva_reorder(g_arena + 8, b, 1, 2, 64, &g, st, FVA_FORWARD, FVA_LAYOUT_ROWS, nullptr) ==
         FVA_ERR_INVALID_ARG);
  const int64_t bad_st[3] = {1280 * 2 * 64, 2 * 64, 4};
  EXPECT(fva_reorder(a, b, 1, 2, 64, &g, bad_st, FVA_FORWARD, FVA_LAYOUT_ROWS, nullptr) ==
         FVA_ERR_INVALID_ARG);
  EXPECT(fva_reorder_ex(a, b, 1, 2, 64, &g, g_arena + 4, st, FVA_FORWARD, FVA_LAYOUT_ROWS,
                        nullptr) == FVA_ERR_INVALID_ARG);
  EXPECT(fva_reorder_pool(a, b, nullptr, 1, 2, 64, &g, nullptr, st, FVA_LAYOUT_ROWS, nullptr) ==
         FVA_ERR_INVALID_ARG);
  EXPECT(fva_reorder_pool(a, b, aligned_ptr(12), 1, 2, 64, &g, nullptr, st, FVA_LAYOUT_V64,
                          nullptr) == FVA_ERR_INVALID_ARG);
  EXPECT(g_launches == before);
  EXPECT(fva_reorder_pool(a, b, aligned_ptr(12), 1, 2, 64, &g, nullptr, st, FVA_LAYOUT_K64,
                          nullptr) == FVA_OK);
  EXPECT(g_launches == before + 1);

  fva_route_params prm;
  memset(&prm, 0, sizeof(prm));
  prm.top_p = 0.9f;
  prm.topk_floor = 2;
  fva_mask m = mask_of(true);
  fva_sizes_t s2;
  EXPECT(fva_sizes(&g, 1, 2, 64, &s2) == FVA_OK);
  std::vector<char> ws(s2.route_ws_bytes + 256);
  char* wsp = (char*)(((uintptr_t)ws.data() + 255) & ~(uintptr_t)255);
  before = g_launches;
  EXPECT(fva_route(a, b, 1, 2, 64, &g, &prm, &m, wsp, s2.route_ws_bytes, 0, nullptr) == FVA_OK);
  EXPECT(fva_route(a, b, 1, 2, 64, &g, &prm, &m, wsp, s2.route_ws_bytes,
                   FVA_ROUTE_SCORES_IN | FVA_ROUTE_POOLED_IN, nullptr) == FVA_ERR_INVALID_ARG);
  EXPECT(fva_route(a, b, 1, 2, 64, &g, &prm, &m, wsp, s2.route_ws_bytes - 1, 0, nullptr) ==
         FVA_ERR_WORKSPACE);
  EXPECT(fva_route(a, b, 1, 2, 64, &g, &prm, &m, wsp + 8, s2.route_ws_bytes, 0, nullptr) ==
         FVA_ERR_WORKSPACE);
  prm.top_p = NAN;
  EXPECT(fva_route(a, b, 1, 2, 64, &g, &prm, &m, wsp, s2.route_ws_bytes, 0, nullptr) ==
         FVA_ERR_INVALID_ARG);
  prm.top_p = 0.9f;
  prm.topk_floor = -1;
  EXPECT(fva_route(a, b, 1, 2, 64, &g, &prm, &m, wsp, s2.route_ws_bytes, 0, nullptr) ==
         FVA_ERR_INVALID_ARG);
  prm.topk_floor = 2;
  fva_mask m0 = mask_of(false);
  EXPECT(fva_route(a, b, 1, 2, 64, &g, &prm, &m0, wsp, s2.route_ws_bytes, 0, nullptr) ==
         FVA_ERR_INVALID_ARG);
  EXPECT(g_launches == before + 1);
  uint32_t flags = 7;
  EXPECT(fva_route_flags(wsp, &flags, nullptr) == FVA_OK && flags == 0);
  EXPECT(fva_route_flags(nullptr, &flags, nullptr) == FVA_ERR_INVALID_ARG);

  std::vector<char> aws(s2.attn_ws_bytes + 256);
  char* awp = (char*)(((uintptr_t)aws.data() + 255) & ~(uintptr_t)255);
  before = g_launches;
  EXPECT(fva_sparse_attn(a, b, a, b, 1, 2, 64, &g, &m, 0.f, FVA_SCHED_XCD, awp, s2.attn_ws_bytes,
                         nullptr, nullptr, nullptr) == FVA_OK);
  EXPECT(fva_sparse_attn(a, b, a, b, 1, 2, 64, &g, &m, 0.f, FVA_TRACE, awp, s2.attn_ws_bytes,
                         nullptr, nullptr, nullptr) == FVA_ERR_INVALID_ARG);
  EXPECT(fva_sparse_attn(a, b, a, b, 1, 2, 64, &g, &m, 0.f, 0x40, awp, s2.attn_ws_bytes, nullptr,
                         nullptr, nullptr) == FVA_ERR_INVALID_ARG);
  EXPECT(fva_sparse_attn(a, b, a, b, 1, 2, 64, &g, &m, 0.f, 0, awp, s2.attn_ws_bytes - 1, nullptr,
                         nullptr, nullptr) == FVA_ERR_WORKSPACE);
  EXPECT(fva_sparse_attn(a, b, a, b, 1, 2, 64, &g, &m, 0.f, 0, awp, s2.attn_ws_bytes, nullptr,
                         g_arena + 2, nullptr) == FVA_ERR_INVALID_ARG);
  EXPECT(fva_sparse_attn_noalloc(a, b, a, b, 1, 2, 64, &g, &m, 0.f, 0, nullptr, nullptr,
                                 nullptr) == FVA_OK);
  EXPECT(fva_dense_attn(a, b, a, g_arena + 16 + 8, 1, 2, 64, &g, 0.f, nullptr, nullptr) ==
         FVA_ERR_INVALID_ARG);
  EXPECT(fva_dense_attn(a, b, a, b, 1, 2, 64, &g, 0.f, nullptr, nullptr) == FVA_OK);
  EXPECT(g_launches == before + 3);
  const fva_grid many = grid_of(1, 1, 64 * 64, 1, 1, 64);  // 4097 heads for the XCD limit
  EXPECT(fva_sparse_attn(a, b, a, b, 1, 4097, 64, &many, &m, 0.f, FVA_SCHED_XCD, awp, 1 << 30,
                         nullptr, nullptr, nullptr) == FVA_ERR_UNSUPPORTED);

  size_t tb = 0;
  EXPECT(fva_tile_order_bytes(&g, &tb) == FVA_OK && tb == 4 * 12 + 4 * 20 + 4 * 21);
  EXPECT(fva_tile_order(&g, 5, aligned_ptr(30), tb, nullptr) == FVA_ERR_INVALID_ARG);
  EXPECT(fva_tile_order(&g, FVA_ORDER_HILBERT, aligned_ptr(30), tb - 1, nullptr) ==
         FVA_ERR_WORKSPACE);
  const fva_grid tiles = grid_of(100, 100, 100, 1, 8, 8);  // past 8192 tiles
  EXPECT(fva_tile_order_bytes(&tiles, &tb) == FVA_ERR_UNSUPPORTED);
  int32_t status = 3;
  EXPECT(fva_tile_table_status(aligned_ptr(30), &status, nullptr) == FVA_OK && status == 0);
  EXPECT(fva_tile_table_status(g_arena + 4, &status, nullptr) == FVA_ERR_INVALID_ARG);

  const int64_t budgets[2] = {10, 20};
  EXPECT(fva_topup(1, 2, 64, &g, budgets, &m, wsp, s2.route_ws_bytes, nullptr) == FVA_OK);
  EXPECT(fva_topup(1, 2, 64, &g, nullptr, &m, wsp, s2.route_ws_bytes, nullptr) ==
         FVA_ERR_INVALID_ARG);
  for (int s = -5; s <= 1; ++s) EXPECT(fva_status_string((fva_status)s) != nullptr);
}

// Random arguments at every entry point: the status must be an fva_status
// value, and a call that reached a launcher must have passed validation of
// the pointers it was given.
static void random_cases(int n) {
  for (int it = 0; it < n; ++it) {
    const fva_grid g = random_grid();
    const int B = pick(4), Hh = pick(50) - 1;  // 0 and -1 are invalid
    const int d = pick(3) == 0 ? 96 : (pick(2) ? 64 : 128);
    fva_sizes_t sz;
    const fva_status ss = fva_sizes(pick(20) ? &g : nullptr, B, Hh, d, &sz);
    EXPECT(ss <= 0 && ss >= FVA_ERR_HIP);
    if (ss == FVA_OK) {
      EXPECT(sz.Npad == (int64_t)sz.nB * sz.BLK && sz.N <= sz.Npad && sz.N > sz.Npad - sz.BLK);
      EXPECT(sz.rows == (int64_t)B * Hh * sz.nB && sz.words == (sz.nB + 31) / 32);
    }
    int64_t st[3] = {pick(3) ? 8 * (1 + pick(4000)) : -8, 8 * pick(100), 8 * pick(40)};
    const int before = g_launches;
    void* s0 = any_ptr();
    void* d0 = any_ptr();
    fva_status r = FVA_OK;
    switch (pick(9)) {
      case 0:
        r = fva_reorder(s0, d0, B, Hh, d, &g, st, pick(3), pick(4), nullptr);
        break;
      case 1:
        r = fva_reorder_ex(s0, d0, B, Hh, d, &g, any_ptr(), st, pick(2), pick(3), nullptr);
        break;
      case 2:
        r = fva_reorder_pool(s0, d0, any_ptr(), B, Hh, d, &g, any_ptr(), st, pick(3), nullptr);
        break;
      case 3: {
        fva_route_params prm;
        memset(&prm, 0, sizeof(prm));
        prm.top_p = (float)pick(1200) / 1000.f - 0.1f;
        prm.topk_floor = pick(10) - 1;
        prm.aug_budget = pick(3) ? 0 : (int64_t)pick(100000) - 10;
        fva_mask m = mask_of(pick(2));
        r = fva_route(s0, d0, B, Hh, d, &g, &prm, pick(8) ? &m : nullptr, any_ptr(),
                      (size_t)pick(1 << 20), pick(4), nullptr);
        break;
      }
      case 4: {
        fva_mask m = mask_of(false);
        r = fva_sparse_attn(s0, d0, any_ptr(), any_ptr(), B, Hh, d, &g, &m, 0.f,
                            pick(4) | (pick(2) ? FVA_TRACE : 0), any_ptr(), (size_t)pick(1 << 16),
                            any_ptr(), pick(2) ? nullptr : any_ptr(), nullptr);
        break;
      }
      case 5: {
        fva_mask m = mask_of(false);
        r = fva_sparse_attn_noalloc(s0, d0, any_ptr(), any_ptr(), B, Hh, d, &g, &m, 0.f, pick(4),
                                    nullptr, nullptr, nullptr);
        break;
      }
      case 6:
        r = fva_dense_attn(s0, d0, any_ptr(), any_ptr(), B, Hh, d, &g, 0.f, nullptr, nullptr);
        break;
      case 7: {
        size_t tb = 0;
        r = fva_tile_order_bytes(&g, &tb);
        if (r == FVA_OK) r = fva_tile_order(&g, pick(3), any_ptr(), tb + pick(3) - 1, nullptr);
        break;
      }
      default: {
        std::vector<int64_t> bud((size_t)(B > 0 && Hh > 0 ? B * Hh : 1), 100);
        fva_mask m = mask_of(pick(2));
        r = fva_topup(B, Hh, d, &g, pick(4) ? bud.data() : nullptr, &m, any_ptr(),
                      (size_t)pick(1 << 20), nullptr);
        break;
      }
    }
    EXPECT(r <= 0 && r >= FVA_ERR_HIP);
    if (r != FVA_OK) {
      EXPECT(g_launches == before);
      EXPECT(fva_last_error()[0] != '\0');
    }
  }
}

int main() {
  fixed_cases();
  random_cases(20000);
  if (g_fail) {
    fprintf(stderr, "%d expectations failed\n", g_fail);
    return 1;
  }
  printf("all cases passed (%d launches reached the stubs)\n", g_launches);
  return 0;
}
