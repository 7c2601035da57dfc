// planner.cpp -- 128-aligned compensation planner (host code).
//
// The DeepEP compensation PR (Python section) describes a water-filling
// chunk-migration planner with expert-affinity batching, a makespan guard, a
// cost-aware no-op and 128-aligned chunks; the TEMPO summary (section 2)
// gives the tile-aware cost of an expert on a device: an activation floor
// plus a cost per 128-row M-tile.  This planner takes the per-expert token
// counts the layout produces (after the count exchange, on every rank), with
// expert e homed on rank e / (E / ws), and moves whole 128-row chunks of one
// expert at a time from the most loaded rank to the least loaded one:
//   - of all (expert, chunk count) moves it takes the one that minimises the
//     pair's new maximum load, preferring an expert the receiver already
//     computes (no new activation floor), then the lower expert id, then
//     the smaller move;
//   - a move is admitted only if the receiver ends below the current
//     makespan, so the makespan never rises;
//   - it stops when the two loads differ by at most one tile or no move is
//     admitted, and discards the whole plan if the makespan fell by less than
//     min_gain (the cost of migrating is not worth it).
// Costs are integers so the plan is exact and reproducible.  Each move lowers
// the load vector (sorted descending) lexicographically, so the loop ends.
#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "moe_dispatch.h"

namespace {

constexpr int64_t kChunk = 128;

int64_t tiles(int64_t rows) { return (rows + kChunk - 1) / kChunk; }

struct MoveKey {
  int64_t pair_max;
  int32_t new_on_dst;  // 0 if the receiver already computes the expert
  int32_t expert;
  int64_t chunks;
  bool operator<(const MoveKey& o) const {
    if (pair_max != o.pair_max) return pair_max < o.pair_max;
    if (new_on_dst != o.new_on_dst) return new_on_dst < o.new_on_dst;
    if (expert != o.expert) return expert < o.expert;
    return chunks < o.chunks;
  }
};

}  // namespace

extern "C" int moe_plan_compensation(const int32_t* expert_counts, int32_t num_experts,
                                     int32_t ep_world_size, int64_t tile_cost,
                                     int64_t activation_cost, int64_t min_gain,
                                     int32_t max_moves, int32_t* moves, int32_t* n_moves,
                                     int64_t* rank_loads, int64_t* makespan_before,
                                     int64_t* makespan_after, int64_t* ideal) {
  if (expert_counts == nullptr || n_moves == nullptr || rank_loads == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (num_experts < 1 || num_experts > (1 << 20) || ep_world_size < 1 ||
      num_experts % ep_world_size != 0)
    return MOE_ERR_INVALID_ARG;
  if (tile_cost <= 0 || activation_cost < 0 || max_moves < 0) return MOE_ERR_INVALID_ARG;
  if (max_moves > 0 && moves == nullptr) return MOE_ERR_INVALID_ARG;
  for (int32_t e = 0; e < num_experts; ++e)
    if (expert_counts[e] < 0) return MOE_ERR_INVALID_ARG;

  const int32_t ws = ep_world_size;
  const int32_t per_rank = num_experts / ws;
  // rows[r * E + e]: rows of expert e computed on rank r
  std::vector<int64_t> rows((size_t)ws * num_experts, 0);
  for (int32_t e = 0; e < num_experts; ++e)
    rows[(size_t)(e / per_rank) * num_experts + e] = expert_counts[e];

  std::vector<int64_t> load(ws, 0);
  int64_t total = 0;
  for (int32_t r = 0; r < ws; ++r) {
    for (int32_t e = 0; e < num_experts; ++e) {
      const int64_t a = rows[(size_t)r * num_experts + e];
      if (a > 0) load[r] += activation_cost + tile_cost * tiles(a);
    }
    total += load[r];
  }
  const std::vector<int64_t> load0 = load;
  int64_t before = 0;
  for (int32_t r = 0; r < ws; ++r) before = load[r] > before ? load[r] : before;

  int32_t count = 0;
  while (count < max_moves) {
    int32_t src = 0, dst = 0;
    for (int32_t r = 1; r < ws; ++r) {
      if (load[r] > load[src]) src = r;
      if (load[r] < load[dst]) dst = r;
    }
    const int64_t ls = load[src], ld = load[dst];
    if (ls - ld <= tile_cost) break;

    bool found = false;
    MoveKey best{};
    int64_t best_src = 0, best_dst = 0;
    for (int32_t e = 0; e < num_experts; ++e) {
      const int64_t a = rows[(size_t)src * num_experts + e];
      const int64_t m_max = a / kChunk;
      if (m_max < 1) continue;
      const bool on_dst = rows[(size_t)dst * num_experts + e] > 0;
      const int64_t new_act = on_dst ? 0 : activation_cost;
      const int64_t target = ls - ld - new_act;
      int64_t cand[3] = {m_max, -1, -1};
      if (target > 0) {
        cand[1] = target / (2 * tile_cost);
        cand[2] = cand[1] + 1;
      }
      for (int64_t m : cand) {
        if (m < 1 || m > m_max) continue;
        const bool empties = m * kChunk == a;
        const int64_t s_new = ls - m * tile_cost - (empties ? activation_cost : 0);
        const int64_t d_new = ld + m * tile_cost + new_act;
        if (d_new >= ls) continue;  // makespan guard
        const MoveKey key{s_new > d_new ? s_new : d_new, on_dst ? 0 : 1, e, m};
        if (!found || key < best) {
          found = true;
          best = key;
          best_src = s_new;
          best_dst = d_new;
        }
      }
    }
    if (!found) break;
    const int64_t moved = best.chunks * kChunk;
    rows[(size_t)src * num_experts + best.expert] -= moved;
    rows[(size_t)dst * num_experts + best.expert] += moved;
    load[src] = best_src;
    load[dst] = best_dst;
    moves[4 * count + 0] = best.expert;
    moves[4 * count + 1] = src;
    moves[4 * count + 2] = dst;
    moves[4 * count + 3] = (int32_t)moved;
    ++count;
  }

  int64_t after = 0;
  for (int32_t r = 0; r < ws; ++r) after = load[r] > after ? load[r] : after;
  if (before - after < min_gain) {  // cost-aware no-op
    count = 0;
    load = load0;
    after = before;
  }
  *n_moves = count;
  for (int32_t r = 0; r < ws; ++r) rank_loads[r] = load[r];
  if (makespan_before) *makespan_before = before;
  if (makespan_after) *makespan_after = after;
  if (ideal) *ideal = (total + ws - 1) / ws;
  return MOE_OK;
}
