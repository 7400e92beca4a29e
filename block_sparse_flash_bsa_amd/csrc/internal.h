// Internal definitions shared by the host planner and the forward launcher.
#pragma once

#include <atomic>
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
  int32_t from_bitmap = 0;     // the layout was given as a block bitmap
  int64_t wl = -1, wr = -1, gk = 0, gq = 0;
  int32_t layout_heads = 1;
  int32_t nb = 0;
  std::vector<std::vector<int32_t>> row_ptr;   // [layout_heads][nb + 1]
  std::vector<std::vector<int32_t>> col_idx;   // [layout_heads][nnz_h]
  std::vector<std::vector<uint8_t>> flags;     // [layout_heads][nnz_h]
  std::vector<int32_t> work;                   // [launch slots], -1 = idle
  bsa_plan_info_t info{};
  // Launch queues (queue.h) of the bf16 tile kernels: [0] the forward and
  // dQ over `work`, [1] dK/dV over the descriptors.  Slots [0,
  // queue_static[k]) run one workgroup each; the rest of XCD x's run
  // (queue_tail[k][x] slots) is a queue that 8 * queue_dyn_per_xcd[k]
  // further workgroups drain.  d_queue: [16] queue lengths ([0..7] launch 0,
  // [8..15] launch 1), then kQueueCounterSets sets of 16 int32 (8 queue
  // counters and a done counter), one set per launch in turn.
  int64_t queue_static[2] = {0, 0};
  int64_t queue_dyn_per_xcd[2] = {0, 0};
  int32_t queue_tail[2][8] = {};
  int32_t* d_queue = nullptr;
  std::atomic<uint32_t> queue_launches{0};
  // Backward: the CSR transposed (per k-block, the ascending q-blocks whose
  // lists hold it, same flags) and the launch order of the dK/dV kernel,
  // items (b * Hkv + hk) * nb + j.  Static plans only.
  std::vector<std::vector<int32_t>> colT_ptr;  // [layout_heads][nb + 1]
  std::vector<std::vector<int32_t>> rowT_idx;  // [layout_heads][nnz_h]
  std::vector<std::vector<uint8_t>> flagsT;    // [layout_heads][nnz_h]
  std::vector<int32_t> work_kv;                // [launch slots] item, -1 = idle
  // A long column (the k-block of a global key is read by every q-block) is
  // cut into chunks of at most kv_chunk entries of the group's walk; slot s
  // runs entries [kv_desc[s].begin, .end) and writes its float32 partial dK,
  // dV to scratch slot kv_desc[s].partial (-1: a whole column, written as the
  // final bf16 rows).  kv_reduce lists the split columns and their partials.
  struct KvDesc {
    int32_t item, begin, end, partial;
  };
  std::vector<KvDesc> kv_desc;                 // [launch slots]
  std::vector<KvDesc> kv_reduce;               // {item, first partial, count, 0}
  int32_t kv_chunk = 0;
  int64_t kv_partials = 0;
  int64_t kv_reduce_launch = 0;                // workgroups (x) of the reduction launch
  // Dynamic plans (bf16 backward): bsa_plan_set_bitmap cuts the long walks
  // on the device, by the rule above.  The first kv_extra_slots launch slots
  // take every chunk of a split column after its first (which keeps the
  // column's own slot); at most kv_partials chunks exist at once (the chunk
  // length doubles until they fit), and *d_kv_count is the number of split
  // columns in d_kv_reduce.
  int64_t kv_extra_slots = 0;
  // Device copy (bsa_plan and bsa_plan_dynamic).
  int device = -1;
  void* dev_mem = nullptr;
  const bsa::RowDesc* d_rows = nullptr;        // [layout_heads * nb]
  const int32_t* d_entries = nullptr;          // [nnz], or [entry_capacity] for a dynamic plan
  const int32_t* d_work = nullptr;             // [launch slots]
  const bsa::RowDesc* d_cols = nullptr;        // [layout_heads * nb] transposed rows
  const int32_t* d_entries_t = nullptr;        // [nnz] (q block << 1) | partial
  const int32_t* d_work_kv = nullptr;          // [dK/dV launch slots] as int4 KvDesc
  const int32_t* d_kv_reduce = nullptr;        // [split columns] as int4 KvDesc
  float* d_kv_scratch = nullptr;               // [kv_partials][2][128][128] float32
  const int32_t* d_kv_count = nullptr;         // dynamic: split columns written by set_bitmap
  int32_t* d_kv_walk = nullptr;                // dynamic: [Hkv * nb] walk length of (hk, j)
  int64_t* d_kv_pre = nullptr;                 // dynamic: [Hkv * nb] packed chunk prefixes
  int32_t* d_kv_head = nullptr;                // dynamic: [8] chunk length and totals
  const int32_t* d_kv_slot = nullptr;          // dynamic: [B * Hkv * nb] item -> slot after the extra ones
  void* dev_scratch = nullptr;                 // allocation behind d_kv_scratch
  // Dynamic plans: the CSR is written on the device by bsa_plan_set_bitmap;
  // d_counts is its per-row scratch [layout_heads * nb], d_scan the scan's
  // per-block sums [ceil(layout_heads * nb / 1024) + 1].
  int32_t dynamic = 0;
  int64_t entry_capacity = 0;
  int32_t* d_counts = nullptr;
  int64_t* d_scan = nullptr;
  // Dynamic plans without the causal cut: bsa_plan_set_bitmap reorders each
  // (KV head, batch entry) run of the launch order longest row first, as
  // build_work does for a static bitmap plan.  d_work_base is the order at
  // creation (q-blocks ascending), d_order [Hkv * nb] the q-blocks of each
  // KV head's run by descending row length; d_work is rewritten from both.
  const int32_t* d_work_base = nullptr;
  int32_t* d_order = nullptr;
};

namespace bsa {
constexpr int kQueueCounterSets = 64;        // queued launches of one plan that may run at once
constexpr size_t kQueueBytes = (16 + 16 * kQueueCounterSets) * sizeof(int32_t);
// The C function bsa_plan() hides the struct tag in C++; use this alias.
using Plan = struct ::bsa_plan;
}  // namespace bsa
