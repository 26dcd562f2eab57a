// Host-only check of the attention planner (plan.cpp), built with
// AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_plan_sanitizers.py. It plans a list of fixed metadata sets and
// a seeded run of random small ones, and checks on every plan:
//   * every visible (unit, token, g, KV head, key) pair is covered by
//     exactly one work item (AHBM Agentic Runtime Architecture, §1.3: the
//     combined rows stay independent; ADR-0060 GQA fused attention, §4 and
//     §5.4: shards partition the keys, all-future tiles are dropped);
//   * items stay inside their unit's rows and keys, and their partial rows
//     inside the workspace; bins cover every item once, in order;
//   * every token record holds the token's context position, and a token
//     with two or more partials has a combination record whose counts match
//     the items that cover it;
//   * malformed metadata is refused with a message, never planned.
// Exit status 0 and a final "plan_check ok" line mean every check passed.
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <set>
#include <string>
#include <tuple>
#include <vector>

#include "plan.h"

using namespace gqa;

namespace {

int g_failures = 0;

void expect(bool ok, const std::string& what) {
  if (!ok) {
    std::printf("FAIL: %s\n", what.c_str());
    ++g_failures;
  }
}

struct Case {
  std::string name;
  PlanInput in;
};

PlanInput make(int H_q, int H_kv, int D, int ps, int dtype, int causal, std::vector<int> shared,
               std::vector<std::tuple<int, int, int>> branches, std::vector<int> splits = {}) {
  PlanInput in;
  in.H_q = H_q;
  in.H_kv = H_kv;
  in.D = D;
  in.page_size = ps;
  in.dtype = dtype;
  in.causal = causal;
  int acc = 0;
  for (int s : shared) {
    in.g_start.push_back(acc);
    in.g_len.push_back(s);
    acc += s;
  }
  for (auto& b : branches) {
    in.b_group.push_back(std::get<0>(b));
    in.b_qlen.push_back(std::get<1>(b));
    in.b_priv.push_back(std::get<2>(b));
  }
  in.splits_override = splits;
  return in;
}

PlanInput on_cus(int n_cu, PlanInput in) {
  in.n_cu = n_cu;
  return in;
}

// Checks one plan against the metadata it was built from.
void check_plan(const std::string& name, const PlanInput& in, const Plan& P) {
  const int G = in.H_q / in.H_kv;
  const int nb = (int)in.b_group.size();
  // token -> (branch, position)
  std::vector<int> tok_branch, tok_pos;
  for (int b = 0; b < nb; ++b) {
    const int C = in.g_len[in.b_group[b]] + in.b_priv[b];
    for (int t = 0; t < in.b_qlen[b]; ++t) {
      tok_branch.push_back(b);
      tok_pos.push_back(C - in.b_qlen[b] + t);
    }
  }
  const int ntok = (int)tok_pos.size();
  expect(P.n_q_tokens == ntok, name + ": token count");
  expect((int)P.tok_rec.size() == ntok, name + ": token records");
  for (int t = 0; t < ntok && t < (int)P.tok_rec.size(); ++t)
    expect(P.tok_rec[t].pos == tok_pos[t], name + ": token position");

  // coverage: (unit, token, g, kv, key) -> count; and items per (token, kv)
  std::map<std::tuple<int, int, int, int, int>, int> cover;
  std::map<std::pair<int, int>, int> items_per_tok_kv;
  int64_t n_items = 0;
  for (int pass = 0; pass < 2; ++pass) {
    const std::vector<WorkItem>& list = pass ? P.narrow : P.wide;
    const std::vector<int32_t>& bins = pass ? P.narrow_bins : P.wide_bins;
    expect(!bins.empty() && bins.front() == 0 && bins.back() == (int32_t)list.size(), name + ": bins cover the items");
    for (size_t b = 0; b + 1 < bins.size(); ++b) expect(bins[b] <= bins[b + 1], name + ": bins in order");
    // chains: inside one bin, consecutive shards of one (unit, KV head, M-tile)
    for (size_t b = 0; b + 1 < bins.size(); ++b)
      for (int32_t x = bins[b]; x < bins[b + 1]; ++x) {
        const WorkItem& w = list[x];
        expect(pass == 0 || w.chain == 0, name + ": no chains on the 32-row kernel");
        const bool prev = x > bins[b] && (list[x - 1].chain & kChainContinued);
        expect(prev == ((w.chain & kChainContinues) != 0), name + ": a chain's items are consecutive");
        if (prev) {
          const WorkItem& p = list[x - 1];
          if (p.unit == w.unit) {
            expect(p.kv == w.kv && p.tile == w.tile && p.split + 1 == w.split && p.key_end == w.key_begin &&
                       p.part_row == w.part_row,
                   name + ": a chain continues its own M-tile's next shard");
          } else {
            // from a single-branch group's prefix into that branch's suffix
            const UnitDesc& pu = P.units[p.unit];
            const UnitDesc& wu = P.units[w.unit];
            expect(pu.kind == kShared && wu.kind == kPrivate && pu.branch_lo == wu.branch_lo &&
                       pu.branch_hi == pu.branch_lo + 1 && p.kv == w.kv && p.tile == w.tile &&
                       p.split + 1 == pu.n_splits && w.split == 0 && p.row_begin == w.row_begin &&
                       p.n_rows == w.n_rows && p.tok_begin == w.tok_begin,
                   name + ": a chain crosses only from a lone branch's prefix into its suffix");
          }
        }
        if (x + 1 == bins[b + 1]) expect(!(w.chain & kChainContinued), name + ": a chain ends inside its bin");
      }
    for (const WorkItem& w : list) {
      ++n_items;
      expect(w.unit >= 0 && w.unit < (int)P.units.size(), name + ": item unit");
      if (w.unit < 0 || w.unit >= (int)P.units.size()) continue;
      const UnitDesc& u = P.units[w.unit];
      expect(w.kv >= 0 && w.kv < in.H_kv, name + ": item KV head");
      expect(w.n_rows > 0 && w.n_rows <= u.bm, name + ": item rows within an M-tile");
      expect(w.row_begin >= 0 && w.row_begin + w.n_rows <= u.n_tok * G, name + ": item rows within the unit");
      expect(w.row_begin % G == 0, name + ": M-tiles hold whole tokens");
      expect(0 <= w.key_begin && w.key_begin < w.key_end && w.key_end <= u.key_len, name + ": item keys");
      const TileInfo& ti = P.tiles[u.tile_off + w.tile];
      if (ti.part_off >= 0) {
        expect(w.part_row >= 0 && w.part_row + w.n_rows <= P.part_rows, name + ": partial rows inside the workspace");
      } else {
        // a tile without workspace rows: each of its tokens has one partial
        for (int r = w.row_begin; r < w.row_begin + w.n_rows; r += G)
          expect(P.tok_rec[u.tok_begin + r / G].comb < 0, name + ": a tile without workspace rows writes directly");
      }
      expect((pass == 1) == (u.bm == kNarrowRows), name + ": item on the kernel of its M-tile size");
      std::set<int> toks;
      for (int r = w.row_begin; r < w.row_begin + w.n_rows; ++r) {
        const int tok = u.tok_begin + r / G, g = r % G;
        toks.insert(tok);
        for (int k = w.key_begin; k < w.key_end; ++k) {
          if (in.causal && u.key_pos0 + k > tok_pos[tok]) continue;
          ++cover[std::make_tuple(w.unit, tok, g, w.kv, k)];
        }
      }
      // a chain of shards leaves one partial: count its first item only
      if (!(w.chain & kChainContinues))
        for (int tok : toks) ++items_per_tok_kv[{tok, w.kv}];
    }
  }
  // expected visible pairs, unit by unit
  int64_t expected = 0;
  for (size_t ui = 0; ui < P.units.size(); ++ui) {
    const UnitDesc& u = P.units[ui];
    for (int tok = u.tok_begin; tok < u.tok_begin + u.n_tok; ++tok)
      for (int k = 0; k < u.key_len; ++k) {
        if (in.causal && u.key_pos0 + k > tok_pos[tok]) continue;
        for (int g = 0; g < G; ++g)
          for (int kv = 0; kv < in.H_kv; ++kv) {
            ++expected;
            auto it = cover.find(std::make_tuple((int)ui, tok, g, kv, k));
            expect(it != cover.end() && it->second == 1, name + ": visible pair covered exactly once");
          }
      }
  }
  expect((int64_t)cover.size() == expected, name + ": no pair outside the visible set");
  // every branch's visible keys are split between its prefix and suffix units
  int64_t branch_pairs = 0;
  for (int tok = 0; tok < ntok; ++tok) {
    const int b = tok_branch[tok];
    const int C = in.g_len[in.b_group[b]] + in.b_priv[b];
    branch_pairs += (int64_t)(in.causal ? tok_pos[tok] + 1 : C) * G * in.H_kv;
  }
  expect(branch_pairs == expected, name + ": units cover each branch's whole context");
  // combination records; the tokens combined in the narrow launch each own
  // one arrival-counter slot, and no two share one
  std::vector<int> slot_owner(P.n_counter_slots, -1);
  for (int ci = 0; ci < (int)P.combs.size(); ++ci) {
    const CombTok& c = P.combs[ci];
    if (c.need > 0) {
      const bool in_range = c.slot >= 0 && c.slot < P.n_counter_slots;
      expect(in_range, name + ": counter slot in range");
      if (in_range) {
        expect(slot_owner[c.slot] < 0, name + ": counter slot used once");
        slot_owner[c.slot] = ci;
      }
    } else {
      expect(c.slot == -1, name + ": no counter slot for a token the merge kernel combines");
    }
  }
  for (int x = 0; x < P.n_counter_slots; ++x) expect(slot_owner[x] >= 0, name + ": every counter slot used");
  for (int tok = 0; tok < ntok; ++tok) {
    const int ci = P.tok_rec[tok].comb;
    for (int kv = 0; kv < in.H_kv; ++kv) {
      const int n = items_per_tok_kv.count({tok, kv}) ? items_per_tok_kv[{tok, kv}] : 0;
      if (ci < 0) {
        expect(n <= 1, name + ": a token without a combination record has at most one partial");
      } else {
        expect(ci < (int)P.combs.size(), name + ": combination index");
        if (ci >= (int)P.combs.size()) continue;
        const CombTok& c = P.combs[ci];
        expect(c.live[0] + c.live[1] == n && n >= 2, name + ": partial count of a combined token");
        expect(c.need == 0 || c.need == n, name + ": arrivals awaited");
        for (int x = 0; x < 2; ++x)
          if (c.live[x] > 0)
            expect(c.p[x] >= 0 && c.p[x] + ((int64_t)(in.H_kv - 1) * c.live[x] + c.live[x] - 1) * c.stride[x] + G <= P.part_rows,
                   name + ": combination rows inside the workspace");
      }
    }
  }
}

void run_case(const Case& c) {
  Plan P;
  const std::string err = build_plan(c.in, &P);
  expect(err.empty(), c.name + ": planned (" + err + ")");
  if (err.empty()) check_plan(c.name, c.in, P);
  if (err.empty() && c.name.find("chains") != std::string::npos) {
    bool any = false;
    for (const WorkItem& w : P.wide) any |= w.chain != 0;
    expect(any, c.name + ": the shards of its M-tiles form chains");
  }
}

}  // namespace

int main() {
  std::vector<Case> cases = {
      {"tiny_fp32", make(2, 1, 64, 4, 1, 1, {64}, {{0, 4, 8}, {0, 4, 8}}, {3, 1, 1})},
      {"fanout", make(8, 2, 128, 16, 0, 1, {300}, {{0, 5, 37}, {0, 7, 50}, {0, 20, 100}})},
      {"prefill_splits", make(4, 1, 128, 16, 0, 1, {700}, {{0, 700, 0}}, {3, 0})},
      {"mixed", make(8, 2, 128, 16, 0, 1, {0, 130}, {{0, 1, 1}, {0, 1, 70}, {0, 1, 300}, {1, 3, 40}, {1, 2, 9}})},
      {"reach", make(4, 2, 128, 16, 0, 1, {100}, {{0, 30, 10}})},
      {"noncausal", make(4, 2, 128, 16, 0, 0, {257}, {{0, 2, 3}}, {5, 2})},
      {"page12", make(8, 2, 64, 12, 0, 1, {333}, {{0, 9, 30}, {0, 1, 0}, {0, 4, 5}})},
      {"page1", make(16, 2, 128, 1, 0, 1, {64}, {{0, 3, 9}, {0, 2, 5}})},
      {"zero_q", make(16, 2, 128, 16, 0, 1, {90}, {{0, 3, 10}, {0, 0, 20}, {0, 2, 5}})},
      {"empty_group", make(16, 2, 128, 16, 0, 1, {0, 50}, {{1, 4, 0}})},
      {"max_group_bf16", make(256, 1, 64, 16, 0, 1, {150}, {{0, 2, 30}, {0, 3, 17}})},
      {"max_group_fp32", make(128, 1, 64, 8, 1, 1, {90}, {{0, 2, 10}})},
      {"many_decodes", make(16, 2, 128, 16, 0, 1, {400}, {{0, 1, 0}, {0, 1, 1}, {0, 1, 2}, {0, 1, 3}, {0, 1, 4},
                                                           {0, 1, 5}, {0, 1, 6}, {0, 1, 7}, {0, 1, 8}})},
      {"huge_splits", make(16, 2, 128, 16, 0, 1, {40}, {{0, 3, 3}}, {4096, 4096})},
      {"decode_8k", make(64, 8, 128, 16, 0, 0, {8192}, {{0, 1, 0}}, {32, 0})},
      // many (KV head, M-tile) jobs per workgroup on an 8-CU device: chains
      {"prefill_chains", on_cus(8, make(16, 4, 128, 16, 0, 1, {300}, {{0, 300, 0}}, {3, 0}))},
      {"prefill_chains_fp32", on_cus(8, make(16, 4, 64, 16, 1, 1, {200}, {{0, 200, 0}}, {4, 0}))},
      {"join_chains", on_cus(8, make(16, 4, 128, 16, 0, 1, {150}, {{0, 250, 250}}, {3, 2}))},
      {"join_chains_one_shard", on_cus(8, make(16, 4, 128, 16, 0, 1, {150}, {{0, 250, 250}}, {1, 1}))},
      {"fanout_chains", on_cus(8, make(16, 4, 128, 16, 0, 1, {150}, {{0, 70, 40}, {0, 90, 30}}, {3, 2, 2}))},
  };
  for (const Case& c : cases) run_case(c);

  // Seeded random small metadata, heuristic and forced split counts.
  std::mt19937 rng(12345);
  auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  const int gs[] = {1, 2, 3, 8};
  for (int it = 0; it < 300; ++it) {
    const int H_kv = uni(1, 3), G = gs[uni(0, 3)];
    const int ng = uni(1, 3);
    std::vector<int> shared;
    for (int g = 0; g < ng; ++g) shared.push_back(uni(0, 3) == 0 ? 0 : uni(1, 400));
    std::vector<std::tuple<int, int, int>> br;
    for (int g = 0; g < ng; ++g)
      for (int k = uni(0, 4); k > 0; --k) {
        const int priv = uni(0, 3) == 0 ? 0 : uni(1, 200);
        const int ctx = shared[g] + priv;
        br.emplace_back(g, ctx == 0 ? 0 : uni(0, std::min(ctx, 40)), priv);
      }
    std::vector<int> splits;
    if (uni(0, 2) == 0)
      for (size_t u = 0; u < shared.size() + br.size(); ++u) splits.push_back(uni(0, 9));
    PlanInput in = make(G * H_kv, H_kv, uni(0, 1) ? 128 : 64, gs[uni(0, 3)] * 4, uni(0, 3) == 0 ? 1 : 0,
                        uni(0, 4) != 0, shared, br, splits);
    in.n_cu = 8 * uni(1, 32);
    run_case({"random#" + std::to_string(it), in});
  }

  // Malformed metadata: refused with a message.
  std::vector<Case> bad = {
      {"negative_len", make(8, 2, 128, 16, 0, 1, {-1}, {{0, 1, 0}})},
      {"q_past_context", make(8, 2, 128, 16, 0, 1, {10}, {{0, 20, 5}})},
      {"group_out_of_range", make(8, 2, 128, 16, 0, 1, {10}, {{3, 1, 0}})},
      {"groups_interleaved", make(8, 2, 128, 16, 0, 1, {10, 10}, {{0, 1, 0}, {1, 1, 0}, {0, 1, 0}})},
      {"splits_length", make(8, 2, 128, 16, 0, 1, {10}, {{0, 1, 0}}, {1})},
      {"splits_range", make(8, 2, 128, 16, 0, 1, {10}, {{0, 1, 0}}, {5000, 0})},
      {"heads", make(9, 2, 128, 16, 0, 1, {10}, {{0, 1, 0}})},
  };
  for (const Case& c : bad) {
    Plan P;
    const std::string err = build_plan(c.in, &P);
    expect(!err.empty(), c.name + ": malformed metadata refused");
  }
  if (g_failures) {
    std::printf("plan_check: %d failures\n", g_failures);
    return 1;
  }
  std::printf("plan_check ok\n");
  return 0;
}
