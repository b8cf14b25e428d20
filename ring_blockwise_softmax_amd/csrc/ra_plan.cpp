// Host-side ring planner: which (query rows, key segments) pairs each emulated
// rank computes at each step.  Pure C++, no HIP runtime call.
//
// Sources (pages cited by title and section):
//  * Ring Attention record (anthology-of-the-sota, Liu et al. 2023): each
//    device keeps its query block and passes its K/V block to its neighbour
//    every step, so at step t rank r holds K/V of rank (r - t) mod P.
//  * TokenRing review (pith.science), "Core claim" and the Algorithm 1 major
//    comment (paper section 3.2): K/V stays put and query blocks travel; read
//    with step = the 1-based iteration i and all ranks mod P, rank j computes
//    Q_{(j - i + 1) mod P} at iteration i, so the owner r receives at step t
//    (= i - 1) the partial made with K/V rank (r + t) mod P.
//  * Zigzag causal partition (TokenRing review, "If this is right" and the
//    section 3.3.2 minor comment): 2P chunks of S/(2P) tokens, rank r owns
//    chunks r and 2P-1-r.  With the causal mask on global positions, chunk
//    pair (query chunk a, key chunk b) is full if b < a, lower-triangular if
//    b == a and fully masked (skipped) if b > a.
//  * K/V-sharded layouts (TokenRing review, "Reading between the lines": the
//    decode / chunked-prefill extension): the queries have one owner, each
//    rank keeps its K/V block and returns its partial to the owner.  In the
//    causal variant the queries are the last Sq of the Sk positions, so a
//    block is fully visible when its last key precedes the first query and
//    causal otherwise; block 0 is visible to every query.
#include <stdint.h>

#include "ra.h"

namespace {

struct Emitter {
  ra_plan_item *items;
  int max_items;
  int count = 0;
  void emit(const ra_plan_item &it) {
    if (items && count < max_items) items[count] = it;
    ++count;
  }
};

ra_plan_item make_item(int step, int rank, int64_t q0, int64_t qn) {
  ra_plan_item it{};
  it.step = step;
  it.rank = rank;
  it.q_start = q0;
  it.q_len = qn;
  it.q_pos0 = q0;
  it.nseg = 0;
  it.first = 0;
  return it;
}

void add_seg(ra_plan_item &it, int64_t k0, int64_t kn, int causal, int kv_rank) {
  ra_plan_seg &s = it.seg[it.nseg++];
  s.kv_start = k0;
  s.kv_len = kn;
  s.causal = causal;
  s.kv_rank = kv_rank;
}

}  // namespace

extern "C" int ra_ring_plan(int64_t Sq, int64_t Sk, int P, const ra_layout *layout, ra_plan_item *items,
                            int max_items) {
  if (!layout || P < 1 || P > 16 || Sq < 0 || Sk < 0 || max_items < 0) return -1;
  if (layout->order != RA_ORDER_RING && layout->order != RA_ORDER_TOKENRING) return -1;
  const int kind = layout->kind;
  const int rank = layout->rank;
  Emitter em{items, max_items};

  auto kv_rank_at = [&](int r, int t) {
    return layout->order == RA_ORDER_RING ? ((r - t) % P + P) % P : (r + t) % P;
  };

  if (kind == RA_LAYOUT_KV_SHARDED || kind == RA_LAYOUT_KV_SHARDED_CAUSAL) {
    if (Sk % P != 0 || (rank != -1 && rank != 0)) return -1;
    const bool causal = kind == RA_LAYOUT_KV_SHARDED_CAUSAL;
    if (causal && Sq > Sk) return -1;
    const int64_t m = Sk / P;
    const int64_t qpos0 = causal ? Sk - Sq : 0;  // position of query row 0
    for (int t = 0; t < P; ++t) {
      const int s = kv_rank_at(0, t);
      ra_plan_item it = make_item(t, 0, 0, Sq);
      it.q_pos0 = qpos0;
      // causal only where the block reaches past the first query's position
      // (its last key, s*m + m - 1, is after qpos0); earlier blocks are full
      add_seg(it, s * m, m, causal && s * m + m - 1 > qpos0, s);
      it.first = (t == 0);
      em.emit(it);
    }
    return em.count;
  }

  if (Sq != Sk) return -1;
  const int64_t S = Sq;
  if (rank < -1 || rank >= P) return -1;
  const int r0 = rank < 0 ? 0 : rank, r1 = rank < 0 ? P - 1 : rank;

  if (kind == RA_LAYOUT_CONTIG || kind == RA_LAYOUT_CONTIG_CAUSAL) {
    if (S % P != 0) return -1;
    const int64_t n = S / P;
    const bool causal = kind == RA_LAYOUT_CONTIG_CAUSAL;
    for (int t = 0; t < P; ++t)
      for (int r = r0; r <= r1; ++r) {
        const int s = kv_rank_at(r, t);
        if (causal && s > r) continue;  // every key after every query
        ra_plan_item it = make_item(t, r, r * n, n);
        add_seg(it, s * n, n, causal && s == r, s);
        it.first = (s == r);  // the diagonal block comes first in both orders
        em.emit(it);
      }
    return em.count;
  }

  if (kind == RA_LAYOUT_ZIGZAG_CAUSAL) {
    if (S % (2 * P) != 0) return -1;
    const int64_t c = S / (2 * P);
    for (int t = 0; t < P; ++t)
      for (int r = r0; r <= r1; ++r) {
        const int s = kv_rank_at(r, t);
        const int a = r, b = 2 * P - 1 - r;    // query chunks of rank r
        const int ka = s, kb = 2 * P - 1 - s;  // key chunks of rank s
        const int first = (s == r);
        if (s < r) {
          // chunk a sees key chunk s fully (s < a); chunk b sees it fully;
          // key chunk 2P-1-s > b is masked for both.
          ra_plan_item ia = make_item(t, r, a * c, c);
          add_seg(ia, ka * c, c, 0, s);
          ia.first = first;
          em.emit(ia);
          ra_plan_item ib = make_item(t, r, b * c, c);
          add_seg(ib, ka * c, c, 0, s);
          ib.first = first;
          em.emit(ib);
        } else if (s > r) {
          // chunk a is before both key chunks (masked); chunk b sees both.
          ra_plan_item ib = make_item(t, r, b * c, c);
          add_seg(ib, ka * c, c, 0, s);
          add_seg(ib, kb * c, c, 0, s);
          ib.first = first;
          em.emit(ib);
        } else {
          ra_plan_item ia = make_item(t, r, a * c, c);
          add_seg(ia, ka * c, c, 1, s);
          ia.first = 1;
          em.emit(ia);
          ra_plan_item ib = make_item(t, r, b * c, c);
          add_seg(ib, ka * c, c, 0, s);
          add_seg(ib, kb * c, c, 1, s);
          ib.first = 1;
          em.emit(ib);
        }
      }
    return em.count;
  }
  return -1;
}
