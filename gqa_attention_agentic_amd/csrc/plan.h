// Host planner: turns group/branch metadata into units, M-tiles, KV shards
// and work items for the attention kernels (pure C++, no HIP).
//
// The planner owns every control decision (ADR-0060 GQA fused attention, §7:
// the kernel is given bases, counters and ranges, and derives addresses):
// which units exist, how many shards each KV range gets, which (M-tile,
// shard) pairs are entirely in the causal future and are dropped before
// launch (§5.4 tile classes), and where each partial lands.
#pragma once
#include <stdint.h>

#include <string>
#include <vector>

#include "plan_types.h"

namespace gqa {

struct PlanInput {
  int32_t H_q = 0, H_kv = 0, D = 0, page_size = 0, dtype = 0, causal = 0;
  std::vector<int32_t> g_start, g_len;            // per group
  std::vector<int32_t> b_group, b_qlen, b_priv;   // per branch
  std::vector<int32_t> splits_override;           // empty or n_groups + n_branches
  int32_t n_cu = 256;                             // compute units of the device
  int32_t wide_per_cu = 1;                        // resident workgroups per CU, 128/256-row kernel
  int32_t narrow_per_cu = 1;                      // resident workgroups per CU, 32-row kernel
};

struct Plan {
  std::vector<UnitDesc> units;
  std::vector<BranchDesc> branches;
  std::vector<TileInfo> tiles;
  std::vector<WorkItem> wide;       // items for the 128/256-row kernel, in bin order
  std::vector<WorkItem> narrow;     // items for the 32-row kernel, in bin order
  // Workgroup b of a kernel runs items [bins[b], bins[b+1]) in order; there
  // are at most as many bins as workgroups stay resident on the device.
  std::vector<int32_t> wide_bins;
  std::vector<int32_t> narrow_bins;
  std::vector<int32_t> api_splits;  // per group prefix, then per branch suffix
  std::vector<int32_t> unit_slot;   // unit -> index in api_splits
  int64_t part_rows = 0;            // partial rows in the workspace
  int64_t n_kv_tiles = 0;           // (item, KV tile) pairs
  int64_t merge_rows = 0;           // output rows with two or more partials
  int32_t max_row_parts = 0;        // largest partial count of any output row
  std::vector<TokRec> tok_rec;      // per query token
  std::vector<CombTok> combs;       // per token whose rows have two or more partials
  int32_t n_counter_slots = 0;      // tokens combined in the narrow launch (CombTok::slot)
  bool merge_launch = false;        // some row is left to the separate merge kernel
  // Both kernels have items and run side by side on disjoint sets of compute
  // units (wide_cus + narrow_cus = the device's); else each gets all of them.
  bool concurrent = false;
  int32_t wide_cus = 0, narrow_cus = 0;
  int32_t max_splits = 0;
  int32_t n_q_tokens = 0;
  int32_t n_shared_tokens = 0;
  int32_t max_branch_pages = 0;     // pages the longest private suffix needs
};

// Checks sizes and relations; returns "" when the metadata is usable.
std::string validate_plan_input(const PlanInput& in);

// Builds the plan (validate first). Returns "" on success.
std::string build_plan(const PlanInput& in, Plan* out);

}  // namespace gqa
