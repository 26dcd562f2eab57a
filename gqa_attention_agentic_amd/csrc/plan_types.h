// Plan records shared by the host planner and the HIP kernels.
//
// A *unit* is one KV range that a set of query rows attends to: either a
// group's shared prefix (rows = every query token of every branch in the
// group, times the G query heads of a KV head) or one branch's private
// suffix (rows = that branch's query tokens times G). This is the combined-Q
// batching of AHBM Agentic Runtime Architecture, §1.3/§3.2 together with the
// GQA fold of ADR-0060 GQA fused attention, §5.2: the M dimension of both
// products is (token, g), so one K/V tile serves all of them.
//
// A unit's rows are cut into M-tiles of whole tokens (at most `bm` rows)
// and its keys into `n_splits` shards (ADR-0060, §4 split-and-combine). A
// *work item* is one (unit, KV head, M-tile, shard); each produces an
// (m, l, O) partial per row, or the final O / LSE directly when that row has
// exactly one live partial (ADR-0060, §0.5.4, N = 1).
//
// Everything a kernel needs about its rows is precomputed here (ADR-0060,
// §7: the issuing side owns control, the kernel is handed bases and
// counts): the work item carries its unit's fields and its workspace row,
// and one record per query token gives the token's position and, when its
// rows have several partials, where they are. A kernel therefore issues no
// chain of dependent metadata loads.
#pragma once
#include <stdint.h>

namespace gqa {

constexpr int kWideRows = 128;    // rows per M-tile of the fp32 MFMA kernel (4 waves x 32)
constexpr int kWideRowsBf16 = 256;  // rows per M-tile of the bf16 MFMA kernel (8 waves x 32)
constexpr int kNarrowRows = 32;   // rows per M-tile of the KV-bandwidth-bound kernel
constexpr int kWideKeys = 64;     // keys per KV tile, wide kernel
constexpr int kNarrowKeys = 32;   // keys per KV tile and wave, narrow kernel

enum UnitKind : int32_t { kShared = 0, kPrivate = 1 };

// Host-side unit record (the kernels see its fields through the items).
struct UnitDesc {
  int32_t kind;        // UnitKind
  int32_t tok_begin;   // first query token of the unit (index into q)
  int32_t n_tok;       // query tokens in the unit; rows = n_tok * G
  int32_t src;         // shared: first token of the prefix in k_shared; private: branch id
  int32_t key_len;     // keys in the unit
  int32_t key_pos0;    // context position of the unit's key 0
  int32_t bm;          // row stride of an M-tile (kWideRows[Bf16] or kNarrowRows)
  int32_t tpt;         // query tokens of the unit's first M-tile (at most bm / G: an M-tile holds
                       // whole tokens; the planner spreads the unit's tokens evenly over its tiles)
  int32_t tile_off;    // index of the unit's first M-tile in the tile table
  int32_t branch_lo;   // branches whose tokens form the unit: [branch_lo, branch_hi)
  int32_t branch_hi;
  int32_t n_splits;    // shards of the key range
};

struct BranchDesc {
  int32_t q_begin;     // first query token
  int32_t q_len;
  int32_t ctx_len;     // shared_len + private_len
  int32_t unit_sh;     // unit index of the group's prefix, -1 if none
  int32_t unit_pr;     // unit index of the private suffix, -1 if none
  int32_t group;
};

// Per M-tile of a unit (host side): how many of the unit's shards are live
// for the tile (shards are in key order and liveness under causality is a
// prefix), and where the tile's partials start in the workspace.
struct TileInfo {
  int32_t live;        // partials per row from this tile: its live shards, 1 when they form a chain,
                       // 0 when its chain continues into the suffix unit
  int64_t part_off;    // first partial row (-1: none); row layout ((kv * live + s) * rows + r_in_tile),
                       // rows = the tile's rows
};

struct WorkItem {
  int32_t unit;
  int32_t kv;          // KV head
  int32_t row_begin;   // first row of the M-tile within the unit
  int32_t n_rows;      // valid rows (<= bm)
  int32_t key_begin;   // unit-local key range [key_begin, key_end)
  int32_t key_end;
  int32_t split;       // shard index (partial slot)
  int32_t tile;        // M-tile index within the unit
  // Copies of the unit's fields, so that nothing but this record is needed
  // before the Q loads and the K/V stream go out.
  int32_t kind;
  int32_t src;
  int32_t tok_begin;
  int32_t key_pos0;
  int64_t part_row;    // workspace row of the item's row 0 (its row r: part_row + r)
  int32_t chain;       // kChainContinues | kChainContinued, or 0 for an item on its own
  int32_t pad1;
};

// WorkItem::chain bits. The shards of one (unit, KV head, M-tile) may form a
// chain: the items run back to back in one workgroup, in shard order, and
// the rows' (m, l, O) state passes from one to the next in registers. In a
// group with a single branch, a prefix tile's chain continues into the
// shards of the same rows' suffix tile.
constexpr int32_t kChainContinues = 1;   // starts from the previous item's state (no Q load)
constexpr int32_t kChainContinued = 2;   // hands its state to the next item (no write)

// Per query token.
struct TokRec {
  int32_t pos;         // context position of the token
  int32_t comb;        // index into the combination records, or -1 when each
                       // of its rows has a single partial (written directly)
};

// Where the partials of a token's rows are, for a token whose rows have two
// or more: for its group-prefix unit (0) and its private-suffix unit (1),
// row (tok, g) of KV head kv has shard s at workspace row
// p[x] + (kv * live[x] + s) * stride[x] + g, stride being the rows of the
// token's M-tile in that unit (a tile's partials are packed: a decode
// token's 8 rows take 8 workspace rows per shard, not the kernel's 32). The rows are combined in the narrow
// launch when need > 0 (the number of narrow items per KV head that write
// them; the last to finish combines), otherwise by the merge kernel.
struct CombTok {
  int64_t p[2];
  int32_t live[2];
  int32_t stride[2];
  int32_t need;
  int32_t slot;        // need > 0: the token's arrival counters, one per KV head, are
                       // counters[(slot * H_kv + kv) * kCounterStride]; -1 otherwise
};

// Distance in 32-bit words between two arrival counters: one 128-byte line
// each, so that the atomics of different (token, KV head) pairs, which all
// land within a few microseconds of each other, do not queue on one line.
constexpr int kCounterStride = 32;

}  // namespace gqa
