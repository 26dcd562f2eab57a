// Host planner for shared-prefix GQA attention (see plan.h).
#include "plan.h"

#include <algorithm>
#include <array>
#include <cmath>
#include <cstdio>
#include <functional>
#include <limits>
#include <map>
#include <queue>

namespace gqa {

namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

std::string fmt(const char* f, long long a = 0, long long b = 0, long long c = 0) {
  char buf[256];
  std::snprintf(buf, sizeof buf, f, a, b, c);
  return buf;
}

// Shard boundaries of a key range of length L into S shards. Long shards are
// aligned to the kernel's KV tile so that only the last tile of a unit is
// ragged; short ones are cut evenly (shard boundaries are not observable in
// the result: ADR-0060 GQA fused attention, §4 -- the merge is associative
// and commutative).
std::vector<int32_t> shard_bounds(int32_t L, int32_t S, int32_t tile) {
  std::vector<int32_t> b;
  if (L <= 0) return b;
  S = std::max(1, std::min(S, L));
  b.push_back(0);
  const bool align = (int64_t)L >= (int64_t)S * 2 * tile;
  for (int32_t s = 1; s < S; ++s) {
    int64_t x = (int64_t)s * L / S;
    if (align) x = std::min<int64_t>(L, ceil_div(x, tile) * tile);
    if (x > b.back() && x < L) b.push_back((int32_t)x);
  }
  b.push_back(L);
  return b;
}

struct UnitWork {
  int32_t unit;
  std::vector<int32_t> tile_tok;       // unit-local first token of each M-tile, then n_tok
  std::vector<int32_t> tile_key_end;   // causal clamp per M-tile (unit-local keys)
  int32_t tile_of(int32_t tok) const {  // M-tile of unit-local token tok
    return (int32_t)(std::upper_bound(tile_tok.begin(), tile_tok.end(), tok) - tile_tok.begin()) - 1;
  }
};

// Token boundaries of the M-tiles of a unit with n_tok tokens of G rows each,
// at most `cap` tokens per tile (bm / G: a tile holds whole tokens). The
// fewest tiles are used and the work is spread evenly over them, so that the
// tiles of one unit keep the same pace through its K/V tiles (a full tile
// next to a small remnant would run behind it and fetch the shared K/V a
// second time). A wave computes 32 rows whether or not they are all valid,
// so when whole tokens fill whole waves (G divides 32) the tiles get whole
// waves each -- as many waves as the tokens need, the counts differing by at
// most one; otherwise the tokens themselves are spread evenly.
std::vector<int32_t> tile_bounds(int32_t n_tok, int32_t G, int32_t cap) {
  const int32_t ntile = (int32_t)ceil_div(n_tok, cap);
  std::vector<int32_t> b(1, 0);
  if (32 % G == 0 && cap % (32 / G) == 0) {
    const int32_t tpw = 32 / G;                       // tokens per wave
    const int32_t waves = (int32_t)ceil_div(n_tok, tpw);
    const int32_t per = waves / ntile, extra = waves % ntile;
    for (int32_t t = 0; t < ntile; ++t)
      b.push_back(std::min(n_tok, b.back() + (per + (t < extra ? 1 : 0)) * tpw));
  } else {
    const int32_t tpt = (int32_t)ceil_div(n_tok, ntile);
    for (int32_t t = 0; t < ntile; ++t) b.push_back(std::min(n_tok, b.back() + tpt));
  }
  b.back() = n_tok;
  return b;
}

// Makespan of a list of item costs on `slots` identical workers, largest
// first (list scheduling in the order the kernel's grid is issued).
double lpt_makespan(std::vector<double> cost, int slots) {
  std::sort(cost.begin(), cost.end(), std::greater<double>());
  std::priority_queue<double, std::vector<double>, std::greater<double>> heap;
  for (int i = 0; i < slots; ++i) heap.push(0.0);
  double mk = 0.0;
  for (double c : cost) {
    double t = heap.top() + c;
    heap.pop();
    heap.push(t);
    mk = std::max(mk, t);
  }
  return mk;
}

// Fixed cost of an item in key units (descriptor and Q loads, the first
// tile's latency, the partial write-back): about one and a half 64-key tiles.
constexpr double kItemFixedKeys = 96.0;
// Extra cost of each further shard of a chain (a barrier and the restart of
// the K/V ring): a quarter of a 64-key tile.
constexpr double kChainStepKeys = 16.0;
constexpr int kXcds = 8;

double item_cost(const WorkItem& w) { return (double)(w.key_end - w.key_begin) + kItemFixedKeys; }

// List scheduling of items (visited in `order`, largest first) onto `nb`
// bins: each goes to the least-loaded bin. Returns the largest bin load.
double lpt_assign(const std::vector<double>& cost, const std::vector<size_t>& order, int nb,
                  std::vector<int>* bin_of) {
  typedef std::pair<double, int> Slot;
  std::priority_queue<Slot, std::vector<Slot>, std::greater<Slot>> heap;
  for (int b = 0; b < nb; ++b) heap.push(Slot(0.0, b));
  double mk = 0.0;
  for (size_t i : order) {
    Slot s = heap.top();
    heap.pop();
    (*bin_of)[i] = s.second;
    s.first += cost[i];
    mk = std::max(mk, s.first);
    heap.push(s);
  }
  return mk;
}

// Packs a kernel's items into at most `slots` bins, one per resident
// workgroup, so that every workgroup starts at once and runs its bin's items
// back to back; the hardware then never has to queue a workgroup behind a
// long one. The unit of packing is a job: one item, or a chain (the
// consecutive shards of one (unit, KV head, M-tile) -- for a group with a
// single branch, the prefix's shards followed by the suffix's -- which must
// run in order in one workgroup). Jobs are placed largest first, so the tail
// of each bin holds the short ones.
//
// Workgroups are dealt to the 8 XCDs of the chip round-robin by launch
// index and each XCD has its own L2, so bin b runs on XCD b % 8. Jobs that
// read the same KV range (same unit, KV head and shard -- for chains, the
// same unit and KV head) are kept on one XCD, so their K/V tiles are
// fetched into one L2 once: such groups go to the least-loaded XCD, largest
// first, and each XCD's jobs to its least-loaded bins. That placement is
// kept unless plain list scheduling over all bins would finish more than 2%
// sooner.
void bin_items(std::vector<WorkItem>* items, const std::vector<int64_t>& chain_key, int slots, int n_cu,
               std::vector<int32_t>* bins) {
  const size_t n = items->size();
  bins->assign(1, 0);
  if (n == 0) return;
  // Jobs: the items of one chain (same chain_key, >= 0), in the order they
  // were made, which is chain order; every other item alone.
  std::vector<std::vector<size_t>> job;
  {
    std::map<int64_t, size_t> chain_job;
    for (size_t i = 0; i < n; ++i) {
      if ((*items)[i].chain == 0) {
        job.push_back({i});
        continue;
      }
      auto ins = chain_job.emplace(chain_key[i], job.size());
      if (ins.second) job.emplace_back();
      job[ins.first->second].push_back(i);
    }
  }
  const size_t nj = job.size();
  const int nb = (int)std::min<int64_t>((int64_t)nj, std::max(1, slots));
  std::vector<double> cost(nj, 0.0);
  for (size_t j = 0; j < nj; ++j) {
    for (size_t i : job[j]) cost[j] += (double)((*items)[i].key_end - (*items)[i].key_begin);
    cost[j] += kItemFixedKeys + kChainStepKeys * (double)(job[j].size() - 1);
  }
  // Largest first; ties in a fixed order of the first item's fields.
  std::vector<size_t> order(nj);
  for (size_t j = 0; j < nj; ++j) order[j] = j;
  auto key_of = [&](size_t j) {
    const WorkItem& w = (*items)[job[j].front()];
    return std::array<int32_t, 4>{w.unit, w.split, w.kv, w.tile};
  };
  std::stable_sort(order.begin(), order.end(), [&](size_t a, size_t b) {
    if (cost[a] != cost[b]) return cost[a] > cost[b];
    return key_of(a) < key_of(b);
  });
  std::vector<int> bin_of(nj, 0);
  const double mk_plain = lpt_assign(cost, order, nb, &bin_of);
  if (n_cu % kXcds == 0 && nb % kXcds == 0 && nb >= 2 * kXcds) {
    const int per = nb / kXcds;
    std::map<std::array<int32_t, 3>, size_t> gid;
    std::vector<double> gcost;
    std::vector<size_t> group_of(nj);
    for (size_t j = 0; j < nj; ++j) {
      const WorkItem& w = (*items)[job[j].front()];
      const std::array<int32_t, 3> k{w.unit, w.kv, w.chain ? -1 : w.split};
      auto ins = gid.emplace(k, gcost.size());
      if (ins.second) gcost.push_back(0.0);
      group_of[j] = ins.first->second;
      gcost[ins.first->second] += cost[j];
    }
    std::vector<size_t> gorder(gcost.size());
    for (size_t g = 0; g < gorder.size(); ++g) gorder[g] = g;
    std::stable_sort(gorder.begin(), gorder.end(), [&](size_t a, size_t b) { return gcost[a] > gcost[b]; });
    std::vector<int> xcd_of(gcost.size(), 0);
    lpt_assign(gcost, gorder, kXcds, &xcd_of);
    std::vector<std::vector<size_t>> on_xcd(kXcds);
    for (size_t j : order) on_xcd[xcd_of[group_of[j]]].push_back(j);   // largest first
    std::vector<int> local(nj, 0);
    double mk_xcd = 0.0;
    for (int x = 0; x < kXcds; ++x) mk_xcd = std::max(mk_xcd, lpt_assign(cost, on_xcd[x], per, &local));
    if (mk_xcd <= mk_plain * 1.02) {
      for (int x = 0; x < kXcds; ++x)
        for (size_t j : on_xcd[x]) bin_of[j] = local[j] * kXcds + x;
    }
  }
  // Items of bin b: its jobs in the (largest-first) order they were
  // assigned, each job's items in shard order.
  std::vector<int32_t> count(nb + 1, 0);
  for (size_t j = 0; j < nj; ++j) count[bin_of[j] + 1] += (int32_t)job[j].size();
  for (int b = 0; b < nb; ++b) count[b + 1] += count[b];
  bins->assign(count.begin(), count.end());
  std::vector<WorkItem> out(n);
  for (size_t j : order)
    for (size_t i : job[j]) out[count[bin_of[j]]++] = (*items)[i];
  *items = std::move(out);
}

// A forward with both MFMA-bound (wide) and KV-bandwidth-bound (narrow)
// items runs the two attention kernels side by side on disjoint sets of
// compute units: the narrow items need only part of the chip to stream at
// HBM speed, and the wide ones compute on the rest. With one resident
// workgroup per CU for each kernel, both grids are resident at once. The
// split (a multiple of the XCD count, so that both grids stay evenly spread
// over the XCDs) is the one for which the later of the two is predicted to
// finish first:
//   wide:   (M-tile, key) pairs / wide CUs x time per key of an M-tile;
//   narrow: the larger of (K/V bytes / HBM bandwidth) and (K/V bytes /
//           narrow CUs / one CU's streaming rate).
// It is decided before the shard counts, which then fill each share.
// The rates are fitted to runs of the two kernels side by side with forced
// splits (one MI355X): a 256-row bf16 M-tile costs ~31 ns per key, a CU of
// the narrow kernel streams ~35 GB/s of K/V, HBM sustains ~5.5 TB/s.
constexpr double kWideNsPerKeyBf16 = 31.0;
constexpr double kHbmBytesPerNs = 5500.0;
constexpr double kCuBytesPerNs = 35.0;

void split_cus(double wide_keys, double narrow_keys, const PlanInput& in, int32_t* wide_cus, int32_t* narrow_cus) {
  const int esize = (in.dtype == 0) ? 2 : 4;
  // fp32: half the rows per M-tile at 1/16 of the matrix rate.
  const double wide_ns_per_key = (in.dtype == 0) ? kWideNsPerKeyBf16 : kWideNsPerKeyBf16 * 8.0;
  const double bytes_n = narrow_keys * 2.0 * in.D * esize;
  double best = 1e300;
  *narrow_cus = kXcds;
  for (int32_t c = kXcds; c <= in.n_cu - kXcds; c += kXcds) {
    const double tw = wide_keys * wide_ns_per_key / (in.n_cu - c);
    const double tn = std::max(bytes_n / kHbmBytesPerNs, bytes_n / (c * kCuBytesPerNs));
    const double t = std::max(tw, tn);
    if (t < best) {
      best = t;
      *narrow_cus = c;
    }
  }
  *wide_cus = in.n_cu - *narrow_cus;
}

}  // namespace

std::string validate_plan_input(const PlanInput& in) {
  if (in.H_q <= 0 || in.H_kv <= 0) return "num_q_heads and num_kv_heads must be > 0";
  if (in.H_q % in.H_kv != 0) return "num_q_heads must be a multiple of num_kv_heads";
  if (in.D != 64 && in.D != 128) return "head_dim must be 64 or 128";
  if (in.H_q / in.H_kv > ((in.dtype == 0) ? kWideRowsBf16 : kWideRows))
    return "too many query heads per KV head for one M-tile";
  if (in.page_size <= 0 || in.page_size > 4096) return "page_size must be in 1..4096";
  const size_t ng = in.g_start.size(), nb = in.b_group.size();
  if (in.g_len.size() != ng) return "group arrays differ in length";
  if (in.b_qlen.size() != nb || in.b_priv.size() != nb) return "branch arrays differ in length";
  if (!in.splits_override.empty() && in.splits_override.size() != ng + nb)
    return "splits_override must have n_groups + n_branches entries";
  int64_t q_total = 0;
  for (size_t g = 0; g < ng; ++g) {
    if (in.g_start[g] < 0 || in.g_len[g] < 0) return fmt("group %lld: negative start or length", (long long)g);
  }
  int32_t last_group = -1;
  std::vector<char> closed(ng, 0);
  for (size_t b = 0; b < nb; ++b) {
    const int32_t g = in.b_group[b];
    if (g < 0 || (size_t)g >= ng) return fmt("branch %lld: group %lld out of range", (long long)b, g);
    if (in.b_qlen[b] < 0 || in.b_priv[b] < 0) return fmt("branch %lld: negative length", (long long)b);
    if ((int64_t)in.b_qlen[b] > (int64_t)in.g_len[g] + in.b_priv[b])
      return fmt("branch %lld: q_len %lld exceeds its context", (long long)b, in.b_qlen[b]);
    if (g != last_group) {
      if (closed[g]) return fmt("branches of group %lld are not consecutive", g);
      if (last_group >= 0) closed[last_group] = 1;
      last_group = g;
    }
    q_total += in.b_qlen[b];
  }
  if (q_total > (int64_t)std::numeric_limits<int32_t>::max() / in.H_q)
    return "too many query rows";
  for (int32_t s : in.splits_override)
    if (s < 0 || s > 4096) return "splits_override entries must be in 0..4096";
  return "";
}

std::string build_plan(const PlanInput& in, Plan* P) {
  std::string err = validate_plan_input(in);
  if (!err.empty()) return err;
  *P = Plan();
  const int32_t G = in.H_q / in.H_kv;
  const int32_t ng = (int32_t)in.g_start.size(), nb = (int32_t)in.b_group.size();
  const int32_t wide_rows = (in.dtype == 0) ? kWideRowsBf16 : kWideRows;

  // Branches: token ranges and context lengths; per-token positions (host only).
  P->branches.resize(nb);
  std::vector<int32_t> pos_of_tok;
  int32_t q_acc = 0;
  for (int32_t b = 0; b < nb; ++b) {
    BranchDesc& d = P->branches[b];
    d.q_begin = q_acc;
    d.q_len = in.b_qlen[b];
    d.ctx_len = in.g_len[in.b_group[b]] + in.b_priv[b];
    d.unit_sh = d.unit_pr = -1;
    d.group = in.b_group[b];
    for (int32_t t = 0; t < d.q_len; ++t) pos_of_tok.push_back(d.ctx_len - d.q_len + t);
    q_acc += d.q_len;
    P->max_branch_pages = std::max<int32_t>(P->max_branch_pages,
                                            (int32_t)ceil_div(in.b_priv[b], in.page_size));
  }
  P->n_q_tokens = q_acc;
  for (int32_t g = 0; g < ng; ++g)
    P->n_shared_tokens = std::max(P->n_shared_tokens, in.g_start[g] + in.g_len[g]);

  // Units: each group's prefix (rows = all its branches' tokens), then each
  // branch's private suffix.
  std::vector<int32_t> api_slot;   // unit -> index in the API's split list
  for (int32_t g = 0; g < ng; ++g) {
    int32_t lo = -1, hi = -1, ntok = 0;
    for (int32_t b = 0; b < nb; ++b)
      if (in.b_group[b] == g) {
        if (lo < 0) lo = b;
        hi = b + 1;
        ntok += in.b_qlen[b];
      }
    if (lo < 0 || ntok == 0 || in.g_len[g] == 0) continue;
    UnitDesc u{};
    u.kind = kShared;
    u.tok_begin = P->branches[lo].q_begin;
    u.n_tok = ntok;
    u.src = in.g_start[g];
    u.key_len = in.g_len[g];
    u.key_pos0 = 0;
    u.branch_lo = lo;
    u.branch_hi = hi;
    for (int32_t b = lo; b < hi; ++b) P->branches[b].unit_sh = (int32_t)P->units.size();
    api_slot.push_back(g);
    P->units.push_back(u);
  }
  for (int32_t b = 0; b < nb; ++b) {
    if (in.b_priv[b] == 0 || in.b_qlen[b] == 0) continue;
    UnitDesc u{};
    u.kind = kPrivate;
    u.tok_begin = P->branches[b].q_begin;
    u.n_tok = in.b_qlen[b];
    u.src = b;
    u.key_len = in.b_priv[b];
    u.key_pos0 = in.g_len[in.b_group[b]];
    u.branch_lo = b;
    u.branch_hi = b + 1;
    P->branches[b].unit_pr = (int32_t)P->units.size();
    api_slot.push_back(ng + b);
    P->units.push_back(u);
  }

  // M-tiles (whole tokens, so every row of a token shares one M-tile of
  // each unit; see tile_bounds) and their causal key clamp.
  const int32_t nu = (int32_t)P->units.size();
  std::vector<UnitWork> uw(nu);
  for (int32_t ui = 0; ui < nu; ++ui) {
    UnitDesc& u = P->units[ui];
    const int64_t M = (int64_t)u.n_tok * G;
    u.bm = (M <= kNarrowRows) ? kNarrowRows : wide_rows;
    const int32_t cap = u.bm / G;
    uw[ui].unit = ui;
    uw[ui].tile_tok = tile_bounds(u.n_tok, G, cap);
    const int32_t ntile = (int32_t)uw[ui].tile_tok.size() - 1;
    u.tpt = uw[ui].tile_tok[1] - uw[ui].tile_tok[0];
    uw[ui].tile_key_end.resize(ntile);
    for (int32_t t = 0; t < ntile; ++t) {
      const int64_t t0 = uw[ui].tile_tok[t], t1 = uw[ui].tile_tok[t + 1];
      int32_t pmax = -1;
      for (int64_t tok = u.tok_begin + t0; tok < u.tok_begin + t1; ++tok)
        pmax = std::max(pmax, pos_of_tok[tok]);
      int64_t kend = u.key_len;
      if (in.causal) kend = std::min<int64_t>(u.key_len, std::max<int64_t>(0, (int64_t)pmax - u.key_pos0 + 1));
      uw[ui].tile_key_end[t] = (int32_t)kend;
    }
  }

  // Compute units of each attention kernel (see split_cus).
  {
    double wk = 0.0, nk = 0.0;
    for (int32_t ui = 0; ui < nu; ++ui)
      for (int32_t kend : uw[ui].tile_key_end)
        (P->units[ui].bm == kNarrowRows ? nk : wk) += (double)kend * in.H_kv;
    P->wide_cus = P->narrow_cus = in.n_cu;
    P->concurrent = false;
    if (wk > 0.0 && nk > 0.0 && in.wide_per_cu == 1 && in.narrow_per_cu == 1 && in.n_cu % kXcds == 0 &&
        in.n_cu >= 2 * kXcds) {
      split_cus(wk, nk, in, &P->wide_cus, &P->narrow_cus);
      P->concurrent = true;
    }
  }

  // Split counts: the caller's override, else the heuristic below.
  std::vector<int32_t> S(nu, 0);
  auto override_of = [&](int32_t ui) -> int32_t {
    return in.splits_override.empty() ? 0 : in.splits_override[api_slot[ui]];
  };
  // KV-bandwidth-bound units (<= 32 rows, decode-like): cut their total K/V
  // stream into equal-length shards (at least 256 keys), as many as give
  // every item about 256 KiB to stream, but no fewer than half and no more
  // than one per resident workgroup (ADR-0060, §5.2-§5.3: decode is bound by
  // KV loads). A workgroup runs its items one after another, each paying a
  // full memory latency and its partial write, so a second item per
  // workgroup costs more than the finer balance gains; a short stream is
  // bound by latency rather than bandwidth, and there fewer, longer shards
  // leave fewer partials to combine. Measured on MI355X (one decode, H_kv 8,
  // d 128): 8k tokens 18.2 us at 16 shards against 19.9 at 32; 2k tokens
  // 11.6 us at 8 against 13.0 at 4; four 8k decodes 35 us at 8 shards each
  // against 48 us at 16.
  const int64_t slots = (int64_t)std::max(1, in.narrow_per_cu) * P->narrow_cus;
  const int64_t wide_slots = (int64_t)std::max(1, in.wide_per_cu) * P->wide_cus;
  {
    int64_t wn = 0;
    for (int32_t ui = 0; ui < nu; ++ui)
      if (P->units[ui].bm == kNarrowRows && override_of(ui) == 0) wn += (int64_t)in.H_kv * P->units[ui].key_len;
    const int64_t bytes = wn * 2 * in.D * (in.dtype == 0 ? 2 : 4);   // K and V
    const int64_t items = std::min(slots, std::max((slots + 1) / 2, ceil_div(bytes, 256 << 10)));
    const int64_t chunk = std::max<int64_t>(256, ceil_div(wn, items));
    for (int32_t ui = 0; ui < nu; ++ui)
      if (P->units[ui].bm == kNarrowRows && override_of(ui) == 0)
        S[ui] = (int32_t)std::max<int64_t>(1, ceil_div(P->units[ui].key_len, chunk));
  }
  // MFMA-bound units (fan-out, prefill): choose one shard length for all of
  // them by estimating the makespan of the resulting items on the resident
  // slots (largest first) plus the cost of writing and merging partials --
  // the runtime cost model of AHBM Agentic Runtime Architecture, §4.5 in
  // one-GPU form: more shards fill more compute units but add merge traffic.
  {
    std::vector<int32_t> wide_auto;
    int32_t maxlen = 0;
    for (int32_t ui = 0; ui < nu; ++ui)
      if (P->units[ui].bm != kNarrowRows && override_of(ui) == 0) {
        wide_auto.push_back(ui);
        maxlen = std::max(maxlen, P->units[ui].key_len);
      }
    if (!wide_auto.empty()) {
      // Cost units: one key of one item (the time a wave spends on one key
      // with 32 rows); fixed per-item cost ~ 96 keys; a partial row costs
      // its bytes at HBM speed relative to MFMA time per key.
      const double item_fixed = kItemFixedKeys;
      const double merge_per_row = 0.002 * in.D / 128.0;
      double best = 1e300;
      int32_t best_chunk = maxlen;
      const int32_t max_cand = std::min<int32_t>(64, std::max<int32_t>(1, maxlen / kWideKeys));
      for (int32_t cand = 1; cand <= max_cand; ++cand) {
        const int32_t chunk = (int32_t)ceil_div(ceil_div(maxlen, cand), kWideKeys) * kWideKeys;
        std::vector<double> cost;
        double partial_rows = 0.0;
        for (int32_t ui : wide_auto) {
          const UnitDesc& u = P->units[ui];
          const int32_t s = (int32_t)ceil_div(u.key_len, chunk);
          std::vector<int32_t> bnd = shard_bounds(u.key_len, s, kWideKeys);
          for (size_t t = 0; t < uw[ui].tile_key_end.size(); ++t) {
            const int32_t kend = uw[ui].tile_key_end[t];
            const int64_t rows = (int64_t)(uw[ui].tile_tok[t + 1] - uw[ui].tile_tok[t]) * G;
            int live = 0;
            for (size_t k = 0; k + 1 < bnd.size(); ++k) {
              if (bnd[k] >= kend) break;
              ++live;
              const int32_t keys = std::min(bnd[k + 1], kend) - bnd[k];
              for (int32_t kv = 0; kv < in.H_kv; ++kv) cost.push_back(item_fixed + keys);
            }
            if (live > 1) partial_rows += (double)live * rows * in.H_kv;
          }
        }
        const double total = lpt_makespan(cost, (int)wide_slots) + merge_per_row * partial_rows;
        if (total < best * 0.999) {
          best = total;
          best_chunk = chunk;
        }
      }
      for (int32_t ui : wide_auto) S[ui] = (int32_t)ceil_div(P->units[ui].key_len, best_chunk);
    }
  }
  for (int32_t ui = 0; ui < nu; ++ui)
    if (override_of(ui) > 0) S[ui] = override_of(ui);

  // Shard boundaries and live shard counts per M-tile.
  P->api_splits.assign(ng + nb, 0);
  P->unit_slot = api_slot;
  std::vector<std::vector<int32_t>> bounds(nu);
  std::vector<int32_t> shards_live;   // per tile: live shards (TileInfo::live counts partials)
  for (int32_t ui = 0; ui < nu; ++ui) {
    UnitDesc& u = P->units[ui];
    const int32_t tile_keys = (u.bm != kNarrowRows) ? kWideKeys : kNarrowKeys;
    bounds[ui] = shard_bounds(u.key_len, S[ui], tile_keys);
    u.n_splits = (int32_t)bounds[ui].size() - 1;
    P->api_splits[api_slot[ui]] = u.n_splits;
    P->max_splits = std::max(P->max_splits, u.n_splits);
    u.tile_off = (int32_t)P->tiles.size();
    for (size_t t = 0; t < uw[ui].tile_key_end.size(); ++t) {
      TileInfo ti{};
      while (ti.live < u.n_splits && bounds[ui][ti.live] < uw[ui].tile_key_end[t]) ++ti.live;
      ti.part_off = -1;
      shards_live.push_back(ti.live);
      P->tiles.push_back(ti);
    }
  }
  // Chains: when the MFMA-bound items of the forward form at least two
  // (unit, KV head, M-tile) jobs per resident workgroup, the live shards of
  // each such job run back to back in one workgroup (bin_items keeps them
  // together, in shard order). The kernel carries the rows' (m, l, O) state
  // from one shard into the next in registers -- the log-sum-exp merge of
  // ADR-0060 GQA fused attention, §4, applied before anything is spilled --
  // and writes one partial per job (or the result itself), so such a tile
  // counts a single partial. With fewer jobs the shards stay independent
  // items, which is what fills the device.
  std::vector<char> chained(nu, 0);
  {
    int64_t jobs = 0;
    for (int32_t ui = 0; ui < nu; ++ui) {
      const UnitDesc& u = P->units[ui];
      if (u.bm == kNarrowRows) continue;
      for (size_t t = 0; t < uw[ui].tile_key_end.size(); ++t) {
        const int32_t live = shards_live[u.tile_off + t];
        jobs += live > 0 ? in.H_kv : 0;
      }
    }
    if (jobs >= 2 * wide_slots)
      for (int32_t ui = 0; ui < nu; ++ui)
        if (P->units[ui].bm != kNarrowRows) {
          chained[ui] = 1;
          for (size_t t = 0; t < uw[ui].tile_key_end.size(); ++t) {
            TileInfo& ti = P->tiles[P->units[ui].tile_off + t];
            ti.live = std::min(ti.live, 1);
          }
        }
  }
  // Across units: when a group has a single branch, its prefix unit and its
  // suffix unit have the same tokens cut into the same M-tiles, so each
  // (KV head, M-tile) chain can run on from the prefix's last shard into the
  // suffix's shards and end with the row's only partial -- the result,
  // written directly (a continuation prefill after a join). The prefix
  // tiles then leave no partial of their own.
  std::vector<char> cross(nb, 0);
  for (int32_t b = 0; b < nb; ++b) {
    const BranchDesc& br = P->branches[b];
    if (br.unit_sh < 0 || br.unit_pr < 0 || !chained[br.unit_sh] || !chained[br.unit_pr]) continue;
    const UnitDesc& us = P->units[br.unit_sh];
    const UnitDesc& up = P->units[br.unit_pr];
    if (us.branch_hi - us.branch_lo != 1 || us.tok_begin != up.tok_begin || uw[br.unit_sh].tile_tok != uw[br.unit_pr].tile_tok)
      continue;
    bool ok = true;
    for (size_t t = 0; t + 1 < uw[br.unit_pr].tile_tok.size(); ++t)
      ok &= shards_live[up.tile_off + t] > 0 && shards_live[us.tile_off + t] > 0;
    if (!ok) continue;
    cross[b] = 1;
    for (size_t t = 0; t + 1 < uw[br.unit_sh].tile_tok.size(); ++t) P->tiles[us.tile_off + t].live = 0;
  }
  std::vector<int32_t> cross_into(nu, -1);   // prefix unit -> the suffix unit its chains run into
  std::vector<char> cross_from(nu, 0);       // suffix unit whose chains start in the prefix
  for (int32_t b = 0; b < nb; ++b)
    if (cross[b]) {
      cross_into[P->branches[b].unit_sh] = P->branches[b].unit_pr;
      cross_from[P->branches[b].unit_pr] = 1;
    }

  // A tile's rows need workspace rows only if some token of the tile has two
  // or more live partials over its prefix and suffix units; otherwise every
  // row of the tile writes O / l directly.
  std::vector<char> tile_needs(P->tiles.size(), 0);
  for (int32_t b = 0; b < nb; ++b) {
    const BranchDesc& br = P->branches[b];
    const int32_t us[2] = {br.unit_sh, br.unit_pr};
    for (int32_t t = 0; t < br.q_len; ++t) {
      const int32_t tok = br.q_begin + t;
      int32_t n = 0, tix[2] = {-1, -1};
      for (int x = 0; x < 2; ++x) {
        if (us[x] < 0) continue;
        const UnitDesc& u = P->units[us[x]];
        tix[x] = u.tile_off + uw[us[x]].tile_of(tok - u.tok_begin);
        n += P->tiles[tix[x]].live;
      }
      if (n >= 2)
        for (int x = 0; x < 2; ++x)
          if (tix[x] >= 0) tile_needs[tix[x]] = 1;
    }
  }
  // Workspace offsets and items (with the chain key of each, for binning:
  // a chain is named by its first unit, KV head and M-tile).
  int64_t part = 0;
  std::vector<int64_t> key_wide, key_narrow;
  for (int32_t ui = 0; ui < nu; ++ui) {
    UnitDesc& u = P->units[ui];
    const int32_t tile_keys = (u.bm != kNarrowRows) ? kWideKeys : kNarrowKeys;
    const std::vector<int32_t>& bnd = bounds[ui];
    for (size_t t = 0; t < uw[ui].tile_key_end.size(); ++t) {
      const int32_t kend = uw[ui].tile_key_end[t];
      TileInfo& ti = P->tiles[u.tile_off + t];
      const int32_t live = shards_live[u.tile_off + t];   // items of the tile per KV head
      const int32_t parts = ti.live;                      // partials of the tile per KV head
      const int32_t row_begin = uw[ui].tile_tok[t] * G;
      const int32_t n_rows = (uw[ui].tile_tok[t + 1] - uw[ui].tile_tok[t]) * G;
      // A tile's partials are packed at its own row count: rows of the
      // kernel's M-tile past the tile's rows get no workspace.
      if (tile_needs[u.tile_off + t]) {
        ti.part_off = part;
        part += (int64_t)in.H_kv * parts * n_rows;
      }
      for (int32_t s = 0; s < live; ++s) {
        for (int32_t kv = 0; kv < in.H_kv; ++kv) {
          WorkItem w{};
          w.unit = ui;
          w.kv = kv;
          w.row_begin = row_begin;
          w.n_rows = n_rows;
          w.key_begin = bnd[s];
          w.key_end = std::min(bnd[s + 1], kend);
          w.split = s;
          w.tile = (int32_t)t;
          w.kind = u.kind;
          w.src = u.src;
          w.tok_begin = u.tok_begin;
          w.key_pos0 = u.key_pos0;
          // Rows of a tile without workspace rows all write directly; the
          // kernel never uses part_row for them.
          w.part_row = ti.part_off >= 0 ? ti.part_off + ((int64_t)kv * parts + (chained[ui] ? 0 : s)) * n_rows : 0;
          const bool first = s == 0 && !cross_from[ui], last = s + 1 == live && cross_into[ui] < 0;
          w.chain = chained[ui] ? ((first ? 0 : kChainContinues) | (last ? 0 : kChainContinued)) : 0;
          w.pad1 = 0;
          P->n_kv_tiles += ceil_div(w.key_end - w.key_begin, tile_keys);
          int32_t head_unit = ui;   // the unit a cross-unit chain starts in
          if (cross_from[ui])
            for (int32_t v = 0; v < nu; ++v)
              if (cross_into[v] == ui) head_unit = v;
          const int64_t key = ((int64_t)head_unit * in.H_kv + kv) * (1 << 20) + (int64_t)t;
          (u.bm != kNarrowRows ? key_wide : key_narrow).push_back(key);
          (u.bm != kNarrowRows ? P->wide : P->narrow).push_back(w);
        }
      }
    }
  }
  P->part_rows = part;

  bin_items(&P->wide, key_wide, in.wide_per_cu * P->wide_cus, P->wide_cus, &P->wide_bins);
  bin_items(&P->narrow, key_narrow, in.narrow_per_cu * P->narrow_cus, P->narrow_cus, &P->narrow_bins);

  // Per-token records. All G rows of a token lie in one M-tile of each of
  // its units, so they have the same partials: live shards of that tile in
  // the prefix unit plus in the suffix unit. Tokens whose rows have two or
  // more get a combination record. A token whose partials all come from
  // narrow items is combined by the last of them to finish (need = the
  // number of such items per KV head); any other goes to the merge kernel.
  P->tok_rec.assign(P->n_q_tokens, TokRec{0, -1});
  P->combs.clear();
  P->n_counter_slots = 0;
  for (int32_t b = 0; b < nb; ++b) {
    const BranchDesc& br = P->branches[b];
    for (int32_t t = 0; t < br.q_len; ++t) {
      const int32_t tok = br.q_begin + t;
      TokRec& tr = P->tok_rec[tok];
      tr.pos = pos_of_tok[tok];
      CombTok c{};
      int32_t n = 0;
      bool narrow_only = true;
      const int32_t us[2] = {br.unit_sh, br.unit_pr};
      for (int x = 0; x < 2; ++x) {
        if (us[x] < 0) continue;
        const UnitDesc& u = P->units[us[x]];
        const int32_t tl = uw[us[x]].tile_of(tok - u.tok_begin);
        const TileInfo& ti = P->tiles[u.tile_off + tl];
        c.p[x] = ti.part_off + (int64_t)(tok - u.tok_begin - uw[us[x]].tile_tok[tl]) * G;
        c.live[x] = ti.live;
        c.stride[x] = (uw[us[x]].tile_tok[tl + 1] - uw[us[x]].tile_tok[tl]) * G;
        n += ti.live;
        if (ti.live > 0 && u.bm != kNarrowRows) narrow_only = false;
      }
      P->max_row_parts = std::max(P->max_row_parts, n);
      if (n < 2) continue;
      P->merge_rows += (int64_t)G * in.H_kv;
      c.need = narrow_only ? n : 0;
      c.slot = narrow_only ? P->n_counter_slots++ : -1;
      if (!narrow_only) P->merge_launch = true;
      tr.comb = (int32_t)P->combs.size();
      P->combs.push_back(c);
    }
  }
  return "";
}

}  // namespace gqa
