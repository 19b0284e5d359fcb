// Host-side slice validation and block-sparse planning (plain C++17, no HIP).
//
// The plan is the block-level sparsity structure of the slice mask: for each
// tile of rows, the tiles of columns that some slice makes visible, each
// tagged FULL (no mask needed) or PARTIAL (mask per cell).  It plays the role
// of the BlockMask in the FlexAttention paper summary, section 4 (block
// sparsity: non-masked block counts plus indices; full blocks skip the mask),
// built here from the slice list of flex_flash_attn_func (MagiAttention issue
// on dummy/padded slices: empty slices are dropped by the scheduler).
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace ffa {

enum : int32_t { kFull = 0, kCausal = 1 };
enum : int32_t { kEntryFull = 0, kEntryPartial = 1 };

// One non-empty slice; r is its index in the caller's list.
struct Slice {
  int32_t qs, qe, ks, ke, type, r;
};

// One visited tile pair: the other axis' tile, the slice, FULL/PARTIAL.
struct PlanEntry {
  int32_t other;
  int32_t slice;  // index into the compact (non-empty) slice list
  int32_t kind;
};

struct Plan {
  int64_t n_tiles = 0;
  std::vector<int64_t> row_ptr;    // [n_tiles + 1]
  std::vector<PlanEntry> entries;  // grouped by tile
  std::vector<int32_t> order;      // tiles by descending entry count
};

// Checks slice r against the token counts: "" if it is valid (no
// allocation then), else a message.
std::string check_slice(int64_t Tq, int64_t Tk, const int32_t* q_ranges, const int32_t* k_ranges,
                        const int32_t* types, int r);

// Checks the slice list against the token counts and keeps the non-empty
// slices (in the caller's order).  Returns "" on success, else a message.
std::string validate_slices(int64_t Tq, int64_t Tk, const int32_t* q_ranges,
                            const int32_t* k_ranges, const int32_t* types, int R,
                            std::vector<Slice>* out);

// Rejects slice lists in which two slices cover the same cell.  O(R^2) in
// the number of slices; used when FFA_DEBUG is set.  Returns "" if disjoint.
std::string check_disjoint(const std::vector<Slice>& s);

// Builds the plan for bm x bn tiles.  transpose == false: tiles are q tiles
// (rows), `other` is a k tile.  transpose == true: tiles are k tiles and
// `other` is a q tile.  Within each tile the entries are sorted by `other`
// and then by the slice's bounds, so the order is the same whatever the
// position of the slices (or of empty slices) in the caller's list.
void build_plan(const std::vector<Slice>& slices, int64_t Tq, int64_t Tk, int bm, int bn,
                bool transpose, Plan* plan);

// Slices that cover exactly the blocks of a BlockMask-style list: query
// block b (rows [b*block_q, (b+1)*block_q) clipped to Tq) sees the key
// blocks idx[b*width .. b*width + num[b]) (any order, no repeats).  Runs of
// adjacent key blocks become one key range, and a key range that continues
// over consecutive query blocks becomes one slice, so sliding-window and
// local-global lists give a few slices per block row, not one per block.
// All slices are FULL, sorted by (qs, ks) and disjoint.  Returns "" on
// success, else a message.
struct RangePair {
  int32_t qs, qe, ks, ke;
};
std::string block_slices(int64_t Tq, int64_t Tk, int block_q, int block_k, const int32_t* num,
                         const int32_t* idx, int width, std::vector<RangePair>* out);

}  // namespace ffa
