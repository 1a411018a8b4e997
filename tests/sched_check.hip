// Host-only check of the resident forward grid's work lists (fa_schedule.h):
// for every order, grid size, head count and query-block count below, the
// static lists of all workgroups plus the balanced schedule's pools must
// cover every (head, query block) item exactly once, and every list must be
// in bounds; the balanced kernel's XCD-only list function must deal the same
// lists.  Prints one line per failure and a summary; exits 1 on failure.
#include <cstdio>
#include <vector>

#include "fa_schedule.h"

namespace sc = fa::sched;

static bool check(int order, int G, int BH, int n_qb, bool balanced, long& n_items_checked) {
  const int n_items = BH * n_qb;
  const bool grouped = BH % 8 == 0 && G % 8 == 0;
  if (order == sc::kOne && G < n_items) return true;  // not a kOne launch
  if ((order == sc::kXcdHead || order == sc::kXcdBlock) && !grouped) return true;
  if (balanced && (!(order == sc::kXcdHead || order == sc::kXcdBlock) || BH < 64)) return true;
  const int hx = BH / 8;
  sc::Plan p{order, G, n_qb, BH, grouped ? (balanced ? hx - (hx / 8 > 1 ? hx / 8 : 1) : hx) : 0};
  std::vector<int> seen(n_items, 0);
  bool ok = true;
  auto mark = [&](int bh, int qb, const char* what, int w, int k) {
    if (bh < 0 || bh >= BH || qb < 0 || qb >= n_qb) {
      std::printf("FAIL order %d G %d BH %d n_qb %d bal %d: %s w %d k %d out of range (%d, %d)\n", order, G, BH, n_qb,
                  (int)balanced, what, w, k, bh, qb);
      ok = false;
      return;
    }
    ++seen[bh * n_qb + qb];
  };
  for (int w = 0; w < G; ++w) {
    int bh, qb;
    for (int k = 0; sc::static_item(p, w, k, bh, qb); ++k) {
      mark(bh, qb, "static", w, k);
      if (k > n_items) {
        std::printf("FAIL order %d: list of w %d does not end\n", order, w);
        return false;
      }
    }
  }
  if (balanced)
    for (int x = 0; x < 8; ++x)
      for (int i = 0; i < sc::pool_len(p); ++i) {
        int bh, qb;
        sc::pool_item(p, x, i, bh, qb);
        mark(bh, qb, "pool", x, i);
      }
  for (int i = 0; i < n_items; ++i)
    if (seen[i] != 1) {
      std::printf("FAIL order %d G %d BH %d n_qb %d bal %d: item (%d, %d) computed %d times\n", order, G, BH, n_qb,
                  (int)balanced, i / n_qb, i % n_qb, seen[i]);
      ok = false;
      break;
    }
  // the balanced kernel's smaller XCD-only function deals the same lists
  if (order == sc::kXcdHead || order == sc::kXcdBlock)
    for (int w = 0; w < G; ++w)
      for (int k = 0;; ++k) {
        int b1 = -1, q1 = -1, b2 = -1, q2 = -1;
        const bool v1 = sc::static_item(p, w, k, b1, q1), v2 = sc::static_item_xcd(p, w, k, b2, q2);
        if (v1 != v2 || (v1 && (b1 != b2 || q1 != q2))) {
          std::printf("FAIL order %d G %d BH %d n_qb %d: static_item_xcd differs at w %d k %d\n", order, G, BH,
                      n_qb, w, k);
          ok = false;
          break;
        }
        if (!v1) break;
      }
  n_items_checked += n_items;
  return ok;
}

int main() {
  const int orders[] = {sc::kOne, sc::kXcdHead, sc::kXcdBlock, sc::kFlatHead, sc::kFlatBlock};
  const int grids[] = {8, 16, 24, 64, 248, 256, 304};
  const int heads[] = {1, 3, 5, 8, 12, 16, 24, 32, 64, 96, 256};
  const int qbs[] = {1, 2, 3, 7, 10, 16, 31, 32, 33, 64};
  long plans = 0, items = 0;
  int fails = 0;
  for (int order : orders)
    for (int G : grids)
      for (int BH : heads)
        for (int n_qb : qbs)
          for (int bal = 0; bal < 2; ++bal) {
            const long before = items;
            if (!check(order, G, BH, n_qb, bal != 0, items)) ++fails;
            if (items != before) ++plans;
          }
  // the one-item-per-workgroup launch uses G = items exactly
  for (int BH : heads)
    for (int n_qb : qbs) {
      const long before = items;
      if (!check(sc::kOne, BH * n_qb, BH, n_qb, false, items)) ++fails;
      if (items != before) ++plans;
    }
  // the page's worked example: one head, S = 64 in 16 x 16 tiles, causal, visits 10 tiles
  const sc::Plan one{sc::kFlatHead, 1, 4, 1, 0};
  std::printf("page_tiles %g\n", sc::plan_makespan(one, 64, 16, 16, true, 0.0));
  std::printf("plans %ld items %ld failures %d\n", plans, items, fails);
  return fails ? 1 : 0;
}
