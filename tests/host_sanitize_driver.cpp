// Host-only driver for the virtual-rank planners (fva_rlb_plan,
// fva_sasa_budget), built with g++ under AddressSanitizer and UBSan by
// tests/test_host_sanitizers.py.  It runs seeded random cases and argument
// edge cases, checks the invariants every plan must satisfy, and exits
// non-zero on any violation; the sanitizers abort on memory errors or
// undefined behaviour.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <vector>

#include "fva_internal.hpp"

namespace fva {
// the library's error recorder lives in the HIP translation unit
fva_status fail(fva_status s, const char* fmt, ...) {
  char buf[256];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  return s;
}
}  // namespace fva

static uint64_t g_state = 0x243F6A8885A308D3ull;
static uint32_t next_u32() {  // 64-bit LCG (Knuth's MMIX constants), top bits
  g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(g_state >> 33);
}
static int uniform(int lo, int hi) { return lo + (int)(next_u32() % (uint32_t)(hi - lo + 1)); }

static int g_bad = 0;
#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      fprintf(stderr, "invariant failed at line %d: %s\n", __LINE__, #c); \
      ++g_bad;                                                        \
    }                                                                 \
  } while (0)

static void one_case(const std::vector<int32_t>& W, int ranks, int topo, float alpha) {
  const int n = (int)W.size();
  std::vector<int32_t> to(ranks, 7777), hd(ranks, 7777), roh(n, 7777);
  fva_rlb_stats st;
  const fva_status s = fva_rlb_plan(W.data(), n, ranks, topo, to.data(), hd.data(), roh.data(), &st);
  if (s != FVA_OK) return;
  // every rank sends at most one of its heads and receives exactly as many as it sends
  std::vector<int> recv(ranks, 0), sent(ranks, 0);
  for (int r = 0; r < ranks; ++r) {
    CHECK(to[r] >= -1 && to[r] < ranks && to[r] != r);
    if (to[r] >= 0) {
      CHECK(hd[r] >= 0 && hd[r] < n);
      CHECK((int64_t)hd[r] * ranks / n == r);  // the head starts on rank r (contiguous placement)
      CHECK(roh[hd[r]] == to[r]);
      ++recv[to[r]];
      ++sent[r];
    } else {
      CHECK(hd[r] == -1);
    }
  }
  for (int r = 0; r < ranks; ++r) CHECK(recv[r] == sent[r]);
  for (int h = 0; h < n; ++h) CHECK(roh[h] >= 0 && roh[h] < ranks);
  CHECK(st.lambda_after <= st.lambda_before + 1e-6);
  CHECK(st.migrations >= 0 && st.migrations <= ranks);
  std::vector<int64_t> budget(n, -1), after(ranks, -1);
  const int64_t cap = (int64_t)uniform(1, 4096);
  if (fva_sasa_budget(W.data(), n, ranks, roh.data(), alpha, cap, budget.data(), after.data()) ==
      FVA_OK) {
    int64_t maxload = 0;
    std::vector<int64_t> load(ranks, 0);
    for (int h = 0; h < n; ++h) {
      CHECK(budget[h] >= W[h]);
      CHECK(budget[h] <= std::max<int64_t>(cap, W[h]));
      load[roh[h]] += W[h];
    }
    for (int r = 0; r < ranks; ++r) maxload = std::max(maxload, load[r]);
    for (int r = 0; r < ranks; ++r) CHECK(after[r] <= std::max<int64_t>(maxload, load[r]));
  }
}

int main() {
  // seeded random cases over both topologies
  for (int it = 0; it < 400; ++it) {
    const int n = uniform(1, 48);
    const int topo = (it & 1) ? FVA_RLB_RING : FVA_RLB_PAIRS;
    const int rmax = topo == FVA_RLB_PAIRS ? std::min(n, FVA_RLB_MAX_PAIR_RANKS) : n;
    const int ranks = uniform(1, rmax);
    std::vector<int32_t> W(n);
    const int spread = uniform(0, 3);
    for (int h = 0; h < n; ++h)
      W[h] = spread == 0 ? 5 : (int32_t)(next_u32() % (spread == 3 ? 1000000u : 1000u));
    one_case(W, ranks, topo, (float)uniform(0, 100) / 100.0f);
  }
  // the largest pair search and a long ring
  {
    std::vector<int32_t> W(FVA_RLB_MAX_PAIR_RANKS * 3);
    for (auto& x : W) x = (int32_t)(next_u32() % 5000u);
    one_case(W, FVA_RLB_MAX_PAIR_RANKS, FVA_RLB_PAIRS, 0.5f);
    std::vector<int32_t> V(512);
    for (auto& x : V) x = (int32_t)(next_u32() % 5000u);
    one_case(V, 256, FVA_RLB_RING, 1.0f);
  }
  // argument errors return a status before touching the outputs
  {
    int32_t W[3] = {1, 2, 3}, to[4], hd[4], roh[3];
    int64_t b[3], a[4];
    fva_rlb_stats st;
    CHECK(fva_rlb_plan(W, 3, 4, FVA_RLB_PAIRS, to, hd, roh, &st) != FVA_OK);   // ranks > heads
    CHECK(fva_rlb_plan(W, 3, 0, FVA_RLB_RING, to, hd, roh, &st) != FVA_OK);    // no ranks
    CHECK(fva_rlb_plan(W, 3, 2, 99, to, hd, roh, &st) != FVA_OK);              // topology
    CHECK(fva_rlb_plan(nullptr, 3, 2, FVA_RLB_RING, to, hd, roh, &st) != FVA_OK);
    int32_t neg[2] = {1, -1};
    CHECK(fva_rlb_plan(neg, 2, 1, FVA_RLB_RING, to, hd, roh, &st) != FVA_OK);
    std::vector<int32_t> many(2 * (FVA_RLB_MAX_PAIR_RANKS + 1), 1);
    std::vector<int32_t> t2(FVA_RLB_MAX_PAIR_RANKS + 1), h2(FVA_RLB_MAX_PAIR_RANKS + 1),
        r2(many.size());
    CHECK(fva_rlb_plan(many.data(), (int32_t)many.size(), FVA_RLB_MAX_PAIR_RANKS + 1,
                       FVA_RLB_PAIRS, t2.data(), h2.data(), r2.data(), &st) != FVA_OK);
    int32_t roh_bad[3] = {0, 5, 1};
    CHECK(fva_sasa_budget(W, 3, 2, roh_bad, 0.5f, 100, b, a) != FVA_OK);     // rank out of range
    int32_t roh_ok[3] = {0, 0, 1};
    CHECK(fva_sasa_budget(W, 3, 2, roh_ok, 1.5f, 100, b, a) != FVA_OK);      // alpha > 1
  }
  if (g_bad) {
    fprintf(stderr, "%d invariant violations\n", g_bad);
    return 1;
  }
  printf("host planners: all cases passed\n");
  return 0;
}
