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
// A unit's rows are cut into M-tiles of `bm` rows and its keys into
// `n_splits` shards (ADR-0060, §4 split-and-combine). A *work item* is one
// (unit, KV head, M-tile, shard); each produces an (m, l, O) partial per row,
// or the final O / LSE directly when that row has exactly one live partial
// (ADR-0060, §0.5.4, N = 1).
#pragma once
#include <stdint.h>

namespace gqa {

constexpr int kWideRows = 128;    // rows per M-tile of the fp32 MFMA kernel (4 waves x 32)
constexpr int kWideRowsBf16 = 256;  // rows per M-tile of the bf16 MFMA kernel (8 waves x 32)
constexpr int kNarrowRows = 32;   // rows per M-tile of the KV-bandwidth-bound kernel
constexpr int kWideKeys = 64;     // keys per KV tile, wide kernel
constexpr int kNarrowKeys = 32;   // keys per KV tile and wave, narrow kernel

enum UnitKind : int32_t { kShared = 0, kPrivate = 1 };

struct UnitDesc {
  int32_t kind;        // UnitKind
  int32_t tok_begin;   // first query token of the unit (index into q)
  int32_t n_tok;       // query tokens in the unit; rows = n_tok * G
  int32_t src;         // shared: first token of the prefix in k_shared; private: branch id
  int32_t key_len;     // keys in the unit
  int32_t key_pos0;    // context position of the unit's key 0
  int32_t bm;          // rows per M-tile (kWideRows or kNarrowRows)
  int32_t tile_off;    // index of the unit's first M-tile in the tile table
  int32_t branch_lo;   // branches whose tokens form the unit: [branch_lo, branch_hi)
  int32_t branch_hi;
  int32_t n_splits;    // shards of the key range
  int32_t pad;
};

struct BranchDesc {
  int32_t q_begin;     // first query token
  int32_t q_len;
  int32_t ctx_len;     // shared_len + private_len
  int32_t unit_sh;     // unit index of the group's prefix, -1 if none
  int32_t unit_pr;     // unit index of the private suffix, -1 if none
  int32_t group;
  int32_t pad0, pad1;
};

// Per M-tile of a unit: how many of the unit's shards are live for the
// tile (shards are in key order and liveness under causality is a prefix),
// and where the tile's partials start in the workspace.
struct TileInfo {
  int32_t live;        // live shards
  int32_t pad;
  int64_t part_off;    // first partial row; row layout: ((kv * live + s) * bm + r_in_tile)
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
  // Copies of the unit's kind, src and tok_begin, so that the Q loads and
  // the K/V stream can be issued before the unit record arrives.
  int32_t kind;
  int32_t src;
  int32_t tok_begin;
  int32_t pad;
};

}  // namespace gqa
