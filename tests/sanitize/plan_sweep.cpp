// Host-only sweep of ra_ring_plan, built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_plan_sanitized.py (the planner is
// plain C++; no HIP is involved).  For every layout, order, rank and P it
// asks for the item count, fills a buffer of exactly that size, and also
// passes a buffer one item short (the planner must count past max_items
// without writing there).  Every item is checked against the row and key
// ranges.  Prints "ok" and exits 0, or names the failing case.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "ra.h"

static int fails = 0;

static void fail(const char *what, long long S, long long Sk, int P, int kind, int order, int rank) {
  if (++fails <= 10)
    std::printf("FAIL %s: Sq=%lld Sk=%lld P=%d kind=%d order=%d rank=%d\n", what, S, Sk, P, kind, order, rank);
}

static void check_case(long long Sq, long long Sk, int P, int kind, int order, int rank) {
  ra_layout L{};
  L.kind = (ra_layout_kind)kind;
  L.order = (ra_order)order;
  L.rank = rank;
  L.fuse_merge = 1;
  const int n = ra_ring_plan(Sq, Sk, P, &L, nullptr, 0);
  if (n < 0) return;  // not a valid combination
  // exact-size buffer on the heap: an overflow is caught by the sanitizer
  ra_plan_item *items = static_cast<ra_plan_item *>(std::malloc(sizeof(ra_plan_item) * (n > 0 ? n : 1)));
  if (ra_ring_plan(Sq, Sk, P, &L, items, n) != n) fail("count changed", Sq, Sk, P, kind, order, rank);
  for (int i = 0; i < n; ++i) {
    const ra_plan_item &it = items[i];
    if (it.step < 0 || it.step >= P) fail("step range", Sq, Sk, P, kind, order, rank);
    if (it.nseg < 1 || it.nseg > 2) fail("nseg", Sq, Sk, P, kind, order, rank);
    if (it.q_start < 0 || it.q_len < 0 || it.q_start + it.q_len > Sq) fail("query rows", Sq, Sk, P, kind, order, rank);
    if (rank >= 0 && kind <= RA_LAYOUT_ZIGZAG_CAUSAL && it.rank != rank) fail("rank", Sq, Sk, P, kind, order, rank);
    for (int s = 0; s < it.nseg && s < 2; ++s) {
      const ra_plan_seg &g = it.seg[s];
      if (g.kv_start < 0 || g.kv_len < 0 || g.kv_start + g.kv_len > Sk) fail("key rows", Sq, Sk, P, kind, order, rank);
      if (g.kv_rank < 0 || g.kv_rank >= P) fail("kv rank", Sq, Sk, P, kind, order, rank);
    }
  }
  std::free(items);
  if (n > 0) {  // one item short: counts all, writes n - 1
    ra_plan_item *few = static_cast<ra_plan_item *>(std::malloc(sizeof(ra_plan_item) * (n - 1 > 0 ? n - 1 : 1)));
    if (ra_ring_plan(Sq, Sk, P, &L, n - 1 > 0 ? few : nullptr, n - 1) != n) fail("short buffer count", Sq, Sk, P, kind, order, rank);
    std::free(few);
  }
}

int main() {
  const long long sizes[] = {0, 1, 2, 7, 16, 31, 32, 96, 100, 257, 960, 1000, 6000, 24000, 1048576};
  int cases = 0;
  for (long long Sq : sizes)
    for (int P = 0; P <= 17; ++P)
      for (int kind = -1; kind <= 5; ++kind)
        for (int order = 0; order <= 2; ++order)
          for (int rank = -2; rank <= P; ++rank) {
            check_case(Sq, Sq, P, kind, order, rank);             // ring layouts: Sq == Sk
            check_case(Sq, Sq * 3 + 5, P, kind, order, rank);     // K/V-sharded: Sq <= Sk
            check_case(Sq + 1, Sq, P, kind, order, rank);         // rejected where Sq > Sk matters
            cases += 3;
          }
  // the largest counts: 16 ranks, zigzag, every rank at every step
  check_case((long long)1 << 30, (long long)1 << 30, 16, RA_LAYOUT_ZIGZAG_CAUSAL, RA_ORDER_TOKENRING, -1);
  if (fails) {
    std::printf("%d failures in %d cases\n", fails, cases);
    return 1;
  }
  std::printf("ok %d cases\n", cases);
  return 0;
}
