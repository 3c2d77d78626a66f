// Planner of the per-(loop, layer) cell kinds (host code, no GPU).
//
// "LoopKV: Loop-Aware KV Cache Compression for Serving Looped Transformers"
// (arXiv:2611.04137), Abstract: each cell is stored at 4 bits, at 2 bits or reuses the
// final loop's KV of its layer; the damages measured cell by cell roughly add up to the
// model's (sentence on the measurements on Ouro); the plan reads as little as possible
// while its predicted damage and its storage stay within their budgets (sentence on the
// planner).
// With additive damage, reads and storage this is a multiple-choice knapsack with two
// budgets; it is solved exactly here.
//
// Method: dynamic programming over the cells in order. A state is a partial plan of the
// first i cells summarized by its (storage, damage, reads) sums; a state that another one
// dominates (no larger in all three) can be dropped, because every completion of it is
// also a completion of the dominating state, at no larger cost in any sum. Each level keeps
// only the non-dominated states within the budgets: candidates are sorted by storage, then
// damage, then reads, and a candidate is kept when the least reads among kept states of no
// larger storage and damage is larger than its own (a staircase of damage -> least reads).
// The answer is the least-reads state after the last cell, traced back through parent
// links. Sums run in cell order in float64, so a given table always gives the same plan.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <map>
#include <vector>

#include "loopkv.h"

namespace lkv {
loopkv_status planner_fail(loopkv_status s, const char* msg);   // runtime.cpp: sets the error text
loopkv_status planner_ok();
}  // namespace lkv

namespace {

struct State {
  double d, r;       // damage and reads of the partial plan
  int64_t s;         // storage of the partial plan
  int32_t parent;    // index of the state of the previous level (-1: empty plan)
  uint8_t kind;      // kind of the last cell
};

// Damage -> least reads among kept states, strictly decreasing in reads as damage grows.
class Staircase {
 public:
  // least reads of a kept state with damage <= d (+inf if none)
  double least(double d) const {
    auto it = m_.upper_bound(d);
    if (it == m_.begin()) return INFINITY;
    return std::prev(it)->second;
  }
  void insert(double d, double r) {   // caller checked r < least(d)
    auto it = m_.lower_bound(d);
    while (it != m_.end() && it->second >= r) it = m_.erase(it);
    m_[d] = r;
  }

 private:
  std::map<double, double> m_;
};

constexpr size_t kMaxStates = size_t(1) << 22;   // states kept over all levels

}  // namespace

extern "C" loopkv_status loopkv_plan_search(int32_t n_loops, int32_t n_layers, const loopkv_cell_cost* costs,
                                             double damage_budget, int64_t storage_budget, uint8_t* kinds_out,
                                             double* damage_out, double* reads_out, int64_t* storage_out) {
  if (!costs || !kinds_out) return lkv::planner_fail(LOOPKV_ERR_INVALID_ARG, "null argument");
  if (n_loops < 1 || n_layers < 1 || (int64_t)n_loops * n_layers > LOOPKV_MAX_PLAN_CELLS)
    return lkv::planner_fail(LOOPKV_ERR_INVALID_ARG, "n_loops x n_layers must be in [1, LOOPKV_MAX_PLAN_CELLS]");
  if (!(damage_budget >= 0.0) || storage_budget < 0)   // NaN fails the first test
    return lkv::planner_fail(LOOPKV_ERR_INVALID_ARG, "budgets must be >= 0 (damage may be +inf)");
  const int n = n_loops * n_layers;
  for (int c = 0; c < n; ++c)
    for (int k = 0; k < 3; ++k) {
      const loopkv_cell_cost& x = costs[c];
      if (!(x.damage[k] >= 0.0) || !std::isfinite(x.damage[k]) || !(x.reads[k] >= 0.0) ||
          !std::isfinite(x.reads[k]) || x.storage[k] < 0 || x.storage[k] > (int64_t(1) << 40))
        return lkv::planner_fail(LOOPKV_ERR_INVALID_ARG,
                                 "costs must be finite and >= 0 (storage < 2^40)");
    }

  std::vector<State> all;
  all.push_back(State{0.0, 0.0, 0, -1, 0});
  std::vector<int32_t> level{0};
  std::vector<State> cand;
  for (int c = 0; c < n; ++c) {
    const bool final_loop = c / n_layers == n_loops - 1;
    const int nk = final_loop ? 2 : 3;   // the final loop cannot reuse
    cand.clear();
    for (int32_t idx : level) {
      const State e = all[idx];
      for (int k = 0; k < nk; ++k) {
        const int64_t s2 = e.s + costs[c].storage[k];
        if (s2 > storage_budget) continue;
        const double d2 = e.d + costs[c].damage[k];
        if (d2 > damage_budget) continue;
        cand.push_back(State{d2, e.r + costs[c].reads[k], s2, idx, (uint8_t)k});
      }
    }
    if (cand.empty()) return lkv::planner_fail(LOOPKV_ERR_PLAN, "no plan meets the damage and storage budgets");
    std::sort(cand.begin(), cand.end(), [](const State& a, const State& b) {
      if (a.s != b.s) return a.s < b.s;
      if (a.d != b.d) return a.d < b.d;
      if (a.r != b.r) return a.r < b.r;
      if (a.parent != b.parent) return a.parent < b.parent;
      return a.kind < b.kind;
    });
    Staircase stair;
    std::vector<int32_t> next;
    for (const State& x : cand) {
      if (stair.least(x.d) <= x.r) continue;   // dominated by a kept state
      stair.insert(x.d, x.r);
      if (all.size() >= kMaxStates)
        return lkv::planner_fail(LOOPKV_ERR_UNSUPPORTED, "plan search exceeds its state limit");
      next.push_back((int32_t)all.size());
      all.push_back(x);
    }
    level.swap(next);
  }
  int32_t best = level[0];
  for (int32_t idx : level) {
    const State& a = all[idx];
    const State& b = all[best];
    if (a.r < b.r || (a.r == b.r && (a.d < b.d || (a.d == b.d && a.s < b.s)))) best = idx;
  }
  if (damage_out) *damage_out = all[best].d;
  if (reads_out) *reads_out = all[best].r;
  if (storage_out) *storage_out = all[best].s;
  for (int c = n - 1, idx = best; c >= 0; --c) {
    kinds_out[c] = all[idx].kind;
    idx = all[idx].parent;
  }
  return lkv::planner_ok();
}
