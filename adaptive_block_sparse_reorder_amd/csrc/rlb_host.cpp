// Runtime load balancing and slack-aware budgets on virtual ranks (FVAttn
// page, section 3.2: post-mask head migration under a one-send-one-receive
// constraint, minimizing the critical-path load first and the rank-load
// variance second; section 3.3: per-rank slack turned into extra mask budget
// through an augmentation coefficient).  Host code only: it consumes the
// realized per-head workloads W_h that fva_route writes.
//
// Placement before balancing is the contiguous Ulysses split: head h lives on
// rank floor(h * R / nheads).  A plan is a permutation pi of the ranks; rank r
// sends one of its heads to pi(r) and receives one from pi^-1(r); fixed points
// do not migrate.
//
// Pair topology: pi is an involution (disjoint swaps).  For a fixed matching
// the objective separates over pairs: the best critical path M* is the max of
// the unpaired loads and of each pair's smallest achievable pair-max; each
// pair then independently takes, among its swaps whose pair-max is <= M*, the
// one with the smallest sum of squared loads.  Every matching is enumerated,
// so the plan is exact for the pair space.
//
// Ring topology: pi(r) = r+1 mod R with every rank sending.  Exact by dynamic
// programming around the cycle for the critical path, then again for the sum
// of squares under that critical path.
//
// When no plan shortens the critical path the identity (no migration) is
// returned, since migrating would cost communication without benefit.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <chrono>
#include <functional>
#include <limits>
#include <vector>

#include "fva_internal.hpp"

namespace fva {
namespace {

struct Objective {
  int64_t mx;
  long double sq;  // sum of squared loads
  bool better_than(const Objective& o) const { return mx < o.mx || (mx == o.mx && sq < o.sq); }
};

struct Placement {
  int R, H;
  std::vector<int> first;  // first head of rank r
  std::vector<int> count;  // heads on rank r
  std::vector<int64_t> load;
};

Placement contiguous(const int32_t* W, int H, int R) {
  Placement p;
  p.R = R;
  p.H = H;
  p.first.assign(R, 0);
  p.count.assign(R, 0);
  p.load.assign(R, 0);
  for (int h = 0; h < H; ++h) {
    const int r = (int)((int64_t)h * R / H);
    if (p.count[r] == 0) p.first[r] = h;
    ++p.count[r];
    p.load[r] += W[h];
  }
  return p;
}

// best plan within the pair (involution) space
void plan_pairs(const int32_t* W, const Placement& P, std::vector<int>& send_to,
                std::vector<int>& send_head, Objective& best) {
  const int R = P.R;
  // every swap (a in H_r, b in H_s) of every pair r < s, and its best pair-max
  struct Opt { int64_t pmax; long double psq; int a, b; };
  std::vector<std::vector<Opt>> opts(R * R);
  std::vector<int64_t> minmax(R * R, std::numeric_limits<int64_t>::max());
  for (int r = 0; r < R; ++r)
    for (int s = r + 1; s < R; ++s) {
      auto& v = opts[r * R + s];
      for (int ia = 0; ia < P.count[r]; ++ia)
        for (int ib = 0; ib < P.count[s]; ++ib) {
          const int a = P.first[r] + ia, b = P.first[s] + ib;
          const int64_t lr = P.load[r] - W[a] + W[b], ls = P.load[s] - W[b] + W[a];
          v.push_back({std::max(lr, ls), (long double)lr * lr + (long double)ls * ls, a, b});
          minmax[r * R + s] = std::min(minmax[r * R + s], std::max(lr, ls));
        }
    }
  // enumerate involutions: recursively pair the lowest unassigned rank
  std::vector<int> mate(R, -2);
  auto evaluate = [&]() {
    int64_t M = 0;
    for (int r = 0; r < R; ++r) {
      if (mate[r] < 0) M = std::max(M, P.load[r]);
      else if (mate[r] > r) M = std::max(M, minmax[r * R + mate[r]]);
    }
    long double sq = 0;
    std::vector<int> to(R, -1), hd(R, -1);
    for (int r = 0; r < R; ++r) {
      if (mate[r] < 0) {
        sq += (long double)P.load[r] * P.load[r];
      } else if (mate[r] > r) {
        const Opt* pick = nullptr;
        for (const Opt& o : opts[r * R + mate[r]])
          if (o.pmax <= M && (!pick || o.psq < pick->psq)) pick = &o;
        sq += pick->psq;
        to[r] = mate[r];
        hd[r] = pick->a;
        to[mate[r]] = r;
        hd[mate[r]] = pick->b;
      }
    }
    const Objective ob{M, sq};
    if (ob.better_than(best)) {
      best = ob;
      send_to = to;
      send_head = hd;
    }
  };
  // depth-first enumeration of matchings: the lowest unassigned rank either
  // stays or pairs with a higher unassigned rank
  struct Rec {
    std::vector<int>& mate;
    int R;
    const std::function<void()>& eval;
    void go(int r) {
      while (r < R && mate[r] != -2) ++r;
      if (r == R) { eval(); return; }
      mate[r] = -1;
      go(r + 1);
      for (int s = r + 1; s < R; ++s)
        if (mate[s] == -2) {
          mate[r] = s;
          mate[s] = r;
          go(r + 1);
          mate[s] = -2;
        }
      mate[r] = -2;
    }
  };
  const std::function<void()> ev = evaluate;
  Rec{mate, R, ev}.go(0);
}

// best plan within the unidirectional ring (every rank sends to r+1)
void plan_ring(const int32_t* W, const Placement& P, std::vector<int>& send_to,
               std::vector<int>& send_head, Objective& best) {
  const int R = P.R;
  if (R < 2) return;
  for (int r = 0; r < R; ++r)
    if (P.count[r] == 0) return;  // a rank with no head cannot send
  int maxc = 0;
  for (int r = 0; r < R; ++r) maxc = std::max(maxc, P.count[r]);
  const int64_t INF = std::numeric_limits<int64_t>::max();
  // load of rank r when it sends head index i and rank r-1 sends head index j
  auto lnew = [&](int r, int i, int j) {
    const int rp = (r + R - 1) % R;
    return P.load[r] - W[P.first[r] + i] + W[P.first[rp] + j];
  };
  Objective bestring{INF, 0};
  std::vector<int> bestchoice;
  for (int i0 = 0; i0 < P.count[0]; ++i0) {
    // pass 1: min over choices of the max load, fixing rank 0's head i0
    std::vector<std::vector<int64_t>> f(R, std::vector<int64_t>(maxc, INF));
    f[0][i0] = std::numeric_limits<int64_t>::min();  // rank 0's load is closed at the end
    for (int r = 1; r < R; ++r)
      for (int i = 0; i < P.count[r]; ++i)
        for (int j = 0; j < P.count[r - 1]; ++j) {
          if (f[r - 1][j] == INF) continue;
          const int64_t v = std::max(f[r - 1][j], lnew(r, i, j));
          f[r][i] = std::min(f[r][i], v);
        }
    int64_t M = INF;
    for (int j = 0; j < P.count[R - 1]; ++j)
      if (f[R - 1][j] != INF) M = std::min(M, std::max(f[R - 1][j], lnew(0, i0, j)));
    if (M == INF || M > bestring.mx) continue;
    // pass 2: min sum of squares with every load <= M, with back-pointers
    const long double NOPE = std::numeric_limits<long double>::infinity();
    std::vector<std::vector<long double>> g(R, std::vector<long double>(maxc, NOPE));
    std::vector<std::vector<int>> bp(R, std::vector<int>(maxc, -1));
    g[0][i0] = 0;
    for (int r = 1; r < R; ++r)
      for (int i = 0; i < P.count[r]; ++i)
        for (int j = 0; j < P.count[r - 1]; ++j) {
          if (g[r - 1][j] == NOPE) continue;
          const int64_t l = lnew(r, i, j);
          if (l > M) continue;
          const long double v = g[r - 1][j] + (long double)l * l;
          if (v < g[r][i]) { g[r][i] = v; bp[r][i] = j; }
        }
    long double bsq = NOPE;
    int bj = -1;
    for (int j = 0; j < P.count[R - 1]; ++j) {
      if (g[R - 1][j] == NOPE) continue;
      const int64_t l0 = lnew(0, i0, j);
      if (l0 > M) continue;
      const long double v = g[R - 1][j] + (long double)l0 * l0;
      if (v < bsq) { bsq = v; bj = j; }
    }
    if (bj < 0) continue;
    const Objective ob{M, bsq};
    if (ob.better_than(bestring)) {
      bestring = ob;
      bestchoice.assign(R, 0);
      bestchoice[0] = i0;
      int j = bj;
      for (int r = R - 1; r >= 1; --r) {
        bestchoice[r] = j;
        j = bp[r][j];
      }
    }
  }
  if (!bestchoice.empty() && bestring.better_than(best)) {
    best = bestring;
    for (int r = 0; r < R; ++r) {
      send_to[r] = (r + 1) % R;
      send_head[r] = P.first[r] + bestchoice[r];
    }
  }
}

}  // namespace
}  // namespace fva

using namespace fva;

extern "C" {

fva_status fva_rlb_plan(const int32_t* head_count, int32_t nheads, int32_t ranks,
                        int32_t topology, int32_t* send_to, int32_t* send_head,
                        int32_t* rank_of_head, fva_rlb_stats* stats) {
  if (!head_count || !send_to || !send_head || !rank_of_head || !stats)
    return fail(FVA_ERR_INVALID_ARG, "null pointer");
  if (nheads <= 0 || ranks <= 0 || ranks > nheads)
    return fail(FVA_ERR_INVALID_ARG, "need 0 < ranks <= nheads");
  if (topology != FVA_RLB_PAIRS && topology != FVA_RLB_RING)
    return fail(FVA_ERR_INVALID_ARG, "topology %d", topology);
  if (topology == FVA_RLB_PAIRS && ranks > FVA_RLB_MAX_PAIR_RANKS)
    return fail(FVA_ERR_UNSUPPORTED, "pair topology enumerates matchings of at most %d ranks",
                FVA_RLB_MAX_PAIR_RANKS);
  for (int h = 0; h < nheads; ++h)
    if (head_count[h] < 0) return fail(FVA_ERR_INVALID_ARG, "negative workload");
  const auto t0 = std::chrono::steady_clock::now();
  const Placement P = contiguous(head_count, nheads, ranks);
  // identity plan
  Objective best{0, 0};
  for (int r = 0; r < ranks; ++r) {
    best.mx = std::max(best.mx, P.load[r]);
    best.sq += (long double)P.load[r] * P.load[r];
  }
  const int64_t max_before = best.mx;
  std::vector<int> to(ranks, -1), hd(ranks, -1);
  Objective cand = best;
  if (topology == FVA_RLB_PAIRS) plan_pairs(head_count, P, to, hd, cand);
  else plan_ring(head_count, P, to, hd, cand);
  // migrate only when the critical path gets shorter
  if (!(cand.mx < best.mx)) {
    std::fill(to.begin(), to.end(), -1);
    std::fill(hd.begin(), hd.end(), -1);
    cand = best;
  }
  const auto t1 = std::chrono::steady_clock::now();
  for (int h = 0; h < nheads; ++h) rank_of_head[h] = (int32_t)((int64_t)h * ranks / nheads);
  int migr = 0;
  for (int r = 0; r < ranks; ++r) {
    send_to[r] = to[r];
    send_head[r] = hd[r];
    if (to[r] >= 0) {
      rank_of_head[hd[r]] = to[r];
      ++migr;
    }
  }
  int64_t total = 0;
  for (int h = 0; h < nheads; ++h) total += head_count[h];
  const double mean = (double)total / ranks;
  memset(stats, 0, sizeof(*stats));
  stats->max_before = max_before;
  stats->max_after = cand.mx;
  stats->mean = mean;
  stats->lambda_before = mean > 0 ? (double)max_before / mean : 1.0;
  stats->lambda_after = mean > 0 ? (double)cand.mx / mean : 1.0;
  stats->solve_us = std::chrono::duration<double, std::micro>(t1 - t0).count();
  stats->migrations = migr;
  return FVA_OK;
}

fva_status fva_sasa_budget(const int32_t* head_count, int32_t nheads, int32_t ranks,
                           const int32_t* rank_of_head, float alpha, int64_t head_cap,
                           int64_t* head_budget, int64_t* rank_load_after) {
  if (!head_count || !rank_of_head || !head_budget) return fail(FVA_ERR_INVALID_ARG, "null pointer");
  if (nheads <= 0 || ranks <= 0) return fail(FVA_ERR_INVALID_ARG, "need positive sizes");
  if (!(alpha >= 0.f && alpha <= 1.f)) return fail(FVA_ERR_INVALID_ARG, "alpha must be in [0, 1]");
  if (head_cap < 0) return fail(FVA_ERR_INVALID_ARG, "head_cap < 0");
  std::vector<int64_t> load(ranks, 0);
  std::vector<std::vector<int>> heads(ranks);
  for (int h = 0; h < nheads; ++h) {
    const int r = rank_of_head[h];
    if (r < 0 || r >= ranks) return fail(FVA_ERR_INVALID_ARG, "rank_of_head[%d] = %d", h, r);
    if (head_count[h] < 0) return fail(FVA_ERR_INVALID_ARG, "negative workload");
    load[r] += head_count[h];
    heads[r].push_back(h);
  }
  const int64_t lmax = *std::max_element(load.begin(), load.end());
  for (int h = 0; h < nheads; ++h) head_budget[h] = head_count[h];
  for (int r = 0; r < ranks; ++r) {
    const int n = (int)heads[r].size();
    int64_t extra = (int64_t)floor((double)alpha * (double)(lmax - load[r]));
    if (n == 0 || extra <= 0) continue;
    // split evenly over the rank's heads (remainder to the lower head ids),
    // each head capped at head_cap pairs
    const int64_t q = extra / n, rem = extra % n;
    for (int k = 0; k < n; ++k) {
      const int h = heads[r][k];
      const int64_t want = head_count[h] + q + (k < rem ? 1 : 0);
      head_budget[h] = std::min<int64_t>(std::max<int64_t>(want, head_count[h]),
                                         std::max<int64_t>(head_cap, head_count[h]));
    }
  }
  if (rank_load_after) {
    for (int r = 0; r < ranks; ++r) rank_load_after[r] = 0;
    for (int h = 0; h < nheads; ++h) rank_load_after[rank_of_head[h]] += head_budget[h];
  }
  return FVA_OK;
}

}  // extern "C"
