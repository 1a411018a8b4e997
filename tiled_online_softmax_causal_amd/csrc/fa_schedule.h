// Work-item schedules of the resident attention forward grid (host and device).
//
// Under the causal rule of the aiml.sh page "Speed up long contexts with
// FlashAttention" (lab.py, tiled_flash_attention: the key loop of a query
// block stops at the diagonal), query block qb of a head visits qb + 1 key
// ranges, so work items (head, query block) differ in weight.  A resident grid
// of G workgroups (one per CU) deals the items out as fixed lists; this file
// defines those lists and a cost model the host uses to pick a list order.
// Everything here is plain integer arithmetic, compiled for the host as well,
// so a CPU test enumerates the lists and checks that every item is computed
// exactly once.
//
// Orders (all heaviest query block first):
//   kOne       one item per workgroup (G >= items); heads grouped per XCD when
//              the head count is a multiple of 8
//   kXcdHead   heads grouped per XCD (workgroups are dispatched round-robin over
//              the 8 XCDs, so workgroup w runs on XCD w % 8); the P = G / 8
//              workgroups of an XCD take its items P at a time, head by head,
//              the order reversed every other round ("snake")
//   kXcdBlock  as kXcdHead, but the XCD's heads take each query-block level in
//              turn, so a round holds items of near-equal weight when a head's
//              items do not fill whole rounds
//   kFlatHead  no XCD grouping (head count not a multiple of 8): one snake over
//              all items, head by head
//   kFlatBlock one snake over all items, query-block level by level
//
#pragma once

#include <hip/hip_runtime.h>

namespace fa {
namespace sched {

enum Order { kOne = 0, kXcdHead = 1, kXcdBlock = 2, kFlatHead = 3, kFlatBlock = 4 };

// Launch-wide schedule parameters (uniform over the grid).
struct Plan {
  int order;
  int G;     // workgroups
  int n_qb;  // query blocks per head
  int BH;    // heads (batch x heads)
  int hs;    // XCD orders: heads per XCD in the static lists (all of them, or those in front of a pool)
};

__host__ __device__ inline int heads_per_xcd(const Plan& p) { return p.BH >> 3; }

// The k-th item of workgroup w's static list; false once the list is over.
// In XCD orders the list covers the first hs heads of each XCD (local head
// index bh / 8 < hs); the rest, if any, form the balanced schedule's pool.
__host__ __device__ inline bool static_item(const Plan& p, int w, int k, int& bh, int& qb) {
  const int n_qb = p.n_qb;
  if (p.order == kOne) {
    if (k > 0 || w >= p.BH * n_qb) return false;
    if ((p.BH & 7) == 0) {
      const int xcd = w & 7, idx = w >> 3;
      bh = (idx / n_qb) * 8 + xcd;
      qb = n_qb - 1 - idx % n_qb;
    } else {
      bh = w / n_qb;
      qb = n_qb - 1 - w % n_qb;
    }
    return true;
  }
  if (p.order == kXcdHead || p.order == kXcdBlock) {
    const int P = p.G >> 3, xcd = w & 7, j = w >> 3;
    const int idx = P * k + ((k & 1) ? P - 1 - j : j);
    if (idx >= p.hs * n_qb) return false;
    int hl, a;
    if (p.order == kXcdHead) {
      hl = idx / n_qb;
      a = idx - hl * n_qb;
    } else {
      a = idx / p.hs;
      hl = idx - a * p.hs;
    }
    bh = hl * 8 + xcd;
    qb = n_qb - 1 - a;
    return true;
  }
  // flat snake over every item
  const int G = p.G;
  const int idx = G * k + ((k & 1) ? G - 1 - w : w);
  if (idx >= p.BH * n_qb) return false;
  int a;
  if (p.order == kFlatHead) {
    bh = idx / n_qb;
    a = idx - bh * n_qb;
  } else {
    a = idx / p.BH;
    bh = idx - a * p.BH;
  }
  qb = n_qb - 1 - a;
  return true;
}

// The static list of an XCD order (kXcdHead or kXcdBlock) only: the same
// lists as static_item, in less code (the balanced kernel uses it).
__host__ __device__ inline bool static_item_xcd(const Plan& p, int w, int k, int& bh, int& qb) {
  const int n_qb = p.n_qb;
  const int P = p.G >> 3, xcd = w & 7, j = w >> 3;
  const int idx = P * k + ((k & 1) ? P - 1 - j : j);
  if (idx >= p.hs * n_qb) return false;
  const bool head = p.order == kXcdHead;
  const int div = head ? n_qb : p.hs;
  const int a = idx / div, r = idx - a * div;
  bh = (head ? a : r) * 8 + xcd;
  qb = n_qb - 1 - (head ? r : a);
  return true;
}

// Pool of the balanced schedule: on XCD x, pool position i (0 <= i < pool_len)
// is local head hs + i / n_qb, query block n_qb - 1 - i % n_qb.
__host__ __device__ inline int pool_len(const Plan& p) { return (heads_per_xcd(p) - p.hs) * p.n_qb; }
__host__ __device__ inline void pool_item(const Plan& p, int xcd, int i, int& bh, int& qb) {
  bh = (p.hs + i / p.n_qb) * 8 + xcd;
  qb = p.n_qb - 1 - i % p.n_qb;
}

// Key tiles of query block qb (BQ rows) for a sequence of S keys in tiles of BK.
__host__ __device__ inline int item_tiles(int qb, int S, int BQ, int BK, bool causal) {
  const int kv_end = causal ? (qb * BQ + BQ < S ? qb * BQ + BQ : S) : S;
  return (kv_end + BK - 1) / BK;
}

// Modelled time of the busiest workgroup of a static plan, in key tiles: each
// item costs its tiles plus item_cost (the per-item overhead in tile units).
// Host only (it walks every list).
inline double plan_makespan(const Plan& p, int S, int BQ, int BK, bool causal, double item_cost) {
  double worst = 0.0;
  for (int w = 0; w < p.G; ++w) {
    double t = 0.0;
    int bh, qb;
    for (int k = 0; static_item(p, w, k, bh, qb); ++k) t += item_tiles(qb, S, BQ, BK, causal) + item_cost;
    worst = t > worst ? t : worst;
  }
  return worst;
}

}  // namespace sched
}  // namespace fa
