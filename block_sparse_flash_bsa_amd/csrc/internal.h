// Internal definitions shared by the host planner and the forward launcher.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "bsattn.h"

namespace bsa {

// Device row descriptor: entries [start, start + count) of the entry array.
struct RowDesc {
  int32_t start;
  int32_t count;
};

// Two work items that read the same K/V head, run by one workgroup of the
// paired kernel over the union of their key-block lists.  item[1] is -1 when
// the item has no partner.
struct PairDesc {
  int32_t item[2];
  int32_t start;   // first union entry
  int32_t count;   // union entries
};

// Union entry encoding: (key block << 4) | state(item 0) | state(item 1) << 2,
// state 0 = FULL, 1 = PARTIAL (token mask), 2 = not in that item's list.
constexpr int kPairFull = 0, kPairPartial = 1, kPairAbsent = 2;
inline int32_t encode_pair_entry(int32_t j, int s0, int s1) { return (j << 4) | s0 | (s1 << 2); }

// Entry encoding in device memory: (key block << 1) | partial.
inline int32_t encode_entry(int32_t j, bool partial) { return (j << 1) | (partial ? 1 : 0); }

// Record a failure detail for bsa_last_error() and return `status`.
bsa_status_t fail(bsa_status_t status, const char* fmt, ...);
void clear_error();

// Supported kernel instantiations (dtype, head_dim, block_size).
bool kernel_supported(int32_t dtype, int32_t head_dim, int32_t block_size);

}  // namespace bsa

struct bsa_plan {
  bsa_problem_t prob{};        // scale resolved to its effective value
  // Token-level mask parameters for PARTIAL tiles.  When token_rule is 0 the
  // window/global part of the predicate is uniform over every tile (block
  // units or a bitmap), so only the causal cut is applied inside a tile.
  int32_t causal = 0;
  int32_t token_rule = 0;
  int64_t wl = -1, wr = -1, gk = 0, gq = 0;
  int32_t layout_heads = 1;
  int32_t nb = 0;
  std::vector<std::vector<int32_t>> row_ptr;   // [layout_heads][nb + 1]
  std::vector<std::vector<int32_t>> col_idx;   // [layout_heads][nnz_h]
  std::vector<std::vector<uint8_t>> flags;     // [layout_heads][nnz_h]
  std::vector<int32_t> work;                   // [launch slots], -1 = idle
  // Paired launch (bf16 kernel): pairs, their union entries and launch order.
  bool paired = false;
  std::vector<bsa::PairDesc> pairs;
  std::vector<int32_t> pair_entries;
  std::vector<int32_t> pair_work;              // [pair launch slots], -1 = idle
  bsa_plan_info_t info{};
  // Device copy (bsa_plan only).
  int device = -1;
  void* dev_mem = nullptr;
  const bsa::RowDesc* d_rows = nullptr;        // [layout_heads * nb]
  const int32_t* d_entries = nullptr;          // [nnz]
  const int32_t* d_work = nullptr;             // [launch slots]
  const bsa::PairDesc* d_pairs = nullptr;
  const int32_t* d_pair_entries = nullptr;
  const int32_t* d_pair_work = nullptr;
};

namespace bsa {
// The C function bsa_plan() hides the struct tag in C++; use this alias.
using Plan = struct ::bsa_plan;
}  // namespace bsa
