// Host planner: layout spec or block bitmap -> per-q-block CSR of key blocks
// with exact FULL/PARTIAL flags, plus the workgroup launch order.
//
// A query block walks only the key blocks its layout admits (step three of
// "How Does Flash-MSA Sparse Attention Work?", How Do Sparse Attention Kernels
// Work in GPU Clusters?).  The lists are built once on the host so the kernel
// never evaluates the layout per element except inside PARTIAL tiles (the
// precomputed-offsets advice in the FAQ of the same page).  Uneven row lengths
// make the forward a load-balancing problem (section "Distributed Training and
// Sparse Attention" of Flash MSA Sparse Attention Kernels Explained; "When
// Sparse Kernels Break" of the GPU-clusters page suggests grouping queries by
// how much work they have): the work order below balances cost per XCD.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <numeric>

#include "internal.h"

namespace bsa {

static thread_local std::string g_last_error;

bsa_status_t fail(bsa_status_t status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

void clear_error() { g_last_error.clear(); }

bool kernel_supported(int32_t dtype, int32_t head_dim, int32_t block_size) {
  if (dtype == BSA_BF16) return head_dim == 128 && block_size == 128;
  if (dtype == BSA_F32)
    return (head_dim == 64 || head_dim == 128) && (block_size == 64 || block_size == 128);
  return false;
}

namespace {

constexpr int kNumXcd = 8;  // MI355X: 8 XCDs; workgroup w is dispatched to XCD w % 8
// A dynamic plan keeps float32 partial dK/dV tiles (128 KiB each) for at most
// this many chunks of split walks: 128 MiB.
constexpr int64_t kDynamicPartials = 1024;

struct TokenRule {
  bool causal;
  int64_t N, wl, wr, gk, gq;

  // |A(q) n [k0, k1]| for one query, by inclusion-exclusion over the window
  // interval W and the global-key prefix G, both cut by causality.
  int64_t count(int64_t q, int64_t k0, int64_t k1) const {
    const int64_t hi = causal ? std::min(q, k1) : k1;
    if (hi < k0) return 0;
    if (q < gq) return hi - k0 + 1;
    const int64_t w_lo = std::max(k0, wl < 0 ? int64_t(0) : q - wl);
    const int64_t w_hi = std::min(hi, wr < 0 ? N - 1 : q + wr);
    const int64_t g_hi = std::min(hi, gk - 1);
    auto len = [](int64_t a, int64_t b) { return b >= a ? b - a + 1 : int64_t(0); };
    return len(w_lo, w_hi) + len(k0, g_hi) - len(w_lo, std::min(w_hi, g_hi));
  }
};

// Pair count of tile (i, j) for a token-unit spec.  O(1) when the tile is
// wholly inside the allowed region, else one interval count per query.
int64_t tile_count_tokens(const TokenRule& r, int64_t bs, int64_t i, int64_t j) {
  // The last block of a ragged sequence ends at N - 1.
  const int64_t q0 = i * bs, q1 = std::min(q0 + bs, r.N) - 1, k0 = j * bs, k1 = std::min(k0 + bs, r.N) - 1;
  const bool causal_full = !r.causal || k1 <= q0;
  if (causal_full) {
    const bool win_full = (r.wl < 0 || q1 - k0 <= r.wl) && (r.wr < 0 || k1 - q0 <= r.wr);
    if (win_full || k1 < r.gk || q1 < r.gq) return (q1 - q0 + 1) * (k1 - k0 + 1);
  }
  int64_t c = 0;
  for (int64_t q = q0; q <= q1; ++q) c += r.count(q, k0, k1);
  return c;
}

bool block_rule(const bsa_layout_t& L, int64_t i, int64_t j) {
  const bool in_w = (L.window_left < 0 || i - j <= L.window_left) &&
                    (L.window_right < 0 || j - i <= L.window_right);
  return in_w || j < L.global_keys || i < L.global_queries;
}

bsa_status_t validate(const bsa_problem_t* p, const bsa_layout_t* L) {
  if (!p || !L) return fail(BSA_ERR_INVALID_ARGUMENT, "problem and layout must not be NULL");
  if (p->batch < 0) return fail(BSA_ERR_INVALID_ARGUMENT, "batch must be >= 0 (got %d)", p->batch);
  if (p->num_heads < 1 || p->num_kv_heads < 1)
    return fail(BSA_ERR_INVALID_ARGUMENT, "num_heads and num_kv_heads must be >= 1 (got %d, %d)",
                p->num_heads, p->num_kv_heads);
  if (p->num_heads % p->num_kv_heads != 0)
    return fail(BSA_ERR_INVALID_ARGUMENT, "num_heads (%d) must be a multiple of num_kv_heads (%d)",
                p->num_heads, p->num_kv_heads);
  if (p->dtype != BSA_F32 && p->dtype != BSA_BF16)
    return fail(BSA_ERR_INVALID_ARGUMENT, "dtype must be BSA_F32 or BSA_BF16 (got %d)", p->dtype);
  if (p->head_dim < 1 || p->block_size < 1)
    return fail(BSA_ERR_INVALID_ARGUMENT, "head_dim and block_size must be >= 1 (got %d, %d)",
                p->head_dim, p->block_size);
  if (p->seq_len < 0)
    return fail(BSA_ERR_INVALID_ARGUMENT, "seq_len (%lld) must be >= 0", (long long)p->seq_len);
  if (!(std::isfinite(p->scale) && p->scale >= 0.f))
    return fail(BSA_ERR_INVALID_ARGUMENT, "scale must be 0 (default) or finite and > 0");
  if (p->schedule < BSA_SCHEDULE_DEFAULT || p->schedule > BSA_SCHEDULE_ROWMAJOR)
    return fail(BSA_ERR_INVALID_ARGUMENT, "unknown schedule %d", p->schedule);
  if (L->causal != 0 && L->causal != 1)
    return fail(BSA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1 (got %d)", L->causal);
  if (L->unit != BSA_UNIT_TOKENS && L->unit != BSA_UNIT_BLOCKS)
    return fail(BSA_ERR_INVALID_ARGUMENT, "unit must be BSA_UNIT_TOKENS or BSA_UNIT_BLOCKS");
  if (L->window_left < -1 || L->window_right < -1)
    return fail(BSA_ERR_INVALID_ARGUMENT, "window_left/right must be >= -1");
  if (L->global_keys < 0 || L->global_queries < 0)
    return fail(BSA_ERR_INVALID_ARGUMENT, "global_keys/global_queries must be >= 0");
  if (L->bitmap && L->bitmap_heads != 1 && L->bitmap_heads != p->num_heads)
    return fail(BSA_ERR_INVALID_ARGUMENT, "bitmap_heads must be 1 or num_heads (%d), got %d",
                p->num_heads, L->bitmap_heads);
  const int64_t nb = (p->seq_len + p->block_size - 1) / p->block_size;
  const int64_t items = int64_t(p->batch) * p->num_heads * nb;
  if (p->seq_len > (int64_t(1) << 30))
    return fail(BSA_ERR_INVALID_ARGUMENT, "seq_len %lld exceeds 2^30", (long long)p->seq_len);
  if (items > INT32_MAX / 2)
    return fail(BSA_ERR_INVALID_ARGUMENT, "problem too large: %lld work items", (long long)items);
  if (!kernel_supported(p->dtype, p->head_dim, p->block_size))
    return fail(BSA_ERR_UNSUPPORTED,
                "no kernel for dtype=%s head_dim=%d block_size=%d (bf16: 128/128; f32: 64|128 / 64|128)",
                p->dtype == BSA_BF16 ? "bf16" : "f32", p->head_dim, p->block_size);
  return BSA_OK;
}

void build_csr(Plan& P, const bsa_layout_t& L) {
  const int64_t bs = P.prob.block_size, nb = P.nb, N = P.prob.seq_len;
  const TokenRule rule{L.causal != 0, P.prob.seq_len, L.window_left, L.window_right,
                       L.global_keys, L.global_queries};
  const bool tokens = !L.bitmap && L.unit == BSA_UNIT_TOKENS;
  const int64_t full = bs * bs;
  auto len = [&](int64_t blk) { return std::min(bs, N - blk * bs); };   // rows of block blk
  P.row_ptr.assign(P.layout_heads, std::vector<int32_t>(nb + 1, 0));
  P.col_idx.assign(P.layout_heads, {});
  P.flags.assign(P.layout_heads, {});
  P.info.allowed_pairs = 0;
  int64_t pairs_per_layout_head_sum = 0;
  std::vector<int64_t> cand;
  for (int lh = 0; lh < P.layout_heads; ++lh) {
    auto& cols = P.col_idx[lh];
    auto& flg = P.flags[lh];
    const uint8_t* bm = L.bitmap ? L.bitmap + size_t(lh) * nb * nb : nullptr;
    int64_t pairs = 0;
    for (int64_t i = 0; i < nb; ++i) {
      if (tokens) {
        // Candidate key blocks: window span, global-key prefix, or all for a
        // global query row; causality caps them at the diagonal.
        cand.clear();
        const int64_t jmax = L.causal ? i : nb - 1;
        if (i * bs < L.global_queries) {
          for (int64_t j = 0; j <= jmax; ++j) cand.push_back(j);
        } else {
          const int64_t klo = L.window_left < 0 ? 0 : std::max<int64_t>(0, i * bs - L.window_left);
          const int64_t khi = L.window_right < 0 ? P.prob.seq_len - 1
                                                 : std::min(P.prob.seq_len - 1, (i + 1) * bs - 1 + L.window_right);
          const int64_t gblocks = (L.global_keys + bs - 1) / bs;
          for (int64_t j = 0; j < std::min(gblocks, nb); ++j) cand.push_back(j);
          for (int64_t j = klo / bs; j <= khi / bs; ++j) cand.push_back(j);
          std::sort(cand.begin(), cand.end());
          cand.erase(std::unique(cand.begin(), cand.end()), cand.end());
          while (!cand.empty() && cand.back() > jmax) cand.pop_back();
        }
        for (int64_t j : cand) {
          const int64_t c = tile_count_tokens(rule, bs, i, j);
          if (c == 0) continue;
          cols.push_back(int32_t(j));
          flg.push_back(c == full ? 0 : 1);
          pairs += c;
        }
      } else {
        for (int64_t j = 0; j < nb; ++j) {
          const bool on = bm ? bm[i * nb + j] != 0 : block_rule(L, i, j);
          if (!on) continue;
          const int64_t c = (!L.causal || j < i) ? len(i) * len(j) : (j == i ? len(i) * (len(i) + 1) / 2 : 0);
          if (c == 0) continue;
          cols.push_back(int32_t(j));
          flg.push_back(c == full ? 0 : 1);
          pairs += c;
        }
      }
      P.row_ptr[lh][i + 1] = int32_t(cols.size());
    }
    pairs_per_layout_head_sum += pairs;
  }
  int64_t nnz = 0, npart = 0, row_max = 0;
  for (int lh = 0; lh < P.layout_heads; ++lh) {
    nnz += int64_t(P.col_idx[lh].size());
    for (uint8_t f : P.flags[lh]) npart += f;
    for (int64_t i = 0; i < nb; ++i)
      row_max = std::max<int64_t>(row_max, P.row_ptr[lh][i + 1] - P.row_ptr[lh][i]);
  }
  // Every query head uses layout head 0 when the layout is shared.
  const int64_t head_mult = P.layout_heads == 1 ? P.prob.num_heads : 1;
  P.info.layout_heads = P.layout_heads;
  P.info.num_blocks = int32_t(nb);
  P.info.nnz = nnz;
  P.info.nnz_partial = npart;
  P.info.active_blocks = int64_t(P.prob.batch) * head_mult * nnz;
  P.info.allowed_pairs = int64_t(P.prob.batch) * head_mult * pairs_per_layout_head_sum;
  P.info.max_row_entries = int32_t(row_max);
}

// Cut a locality-ordered item list into one contiguous run per XCD with equal
// total cost; slot s = kNumXcd * r + x runs the r-th item of XCD x's run
// (idle slots hold -1).
template <class Cost>
std::vector<int32_t> xcd_slots(const std::vector<int32_t>& loc, Cost cost) {
  int64_t total = 0;
  for (int32_t it : loc) total += cost(it);
  std::vector<std::vector<int32_t>> seg(kNumXcd);
  int64_t acc = 0;
  for (int32_t it : loc) {
    const int64_t x = std::min<int64_t>(kNumXcd - 1, (acc * kNumXcd) / std::max<int64_t>(total, 1));
    seg[x].push_back(it);
    acc += cost(it);
  }
  size_t longest = 0;
  for (auto& sg : seg) longest = std::max(longest, sg.size());
  std::vector<int32_t> slots(longest * kNumXcd, -1);
  for (int x = 0; x < kNumXcd; ++x)
    for (size_t r = 0; r < seg[x].size(); ++r) slots[r * kNumXcd + x] = seg[x][r];
  return slots;
}

// Launch queue k of the bf16 tile kernels (queue.h): XCDs of one chip run
// the same work at speeds a few percent apart, and the launch ends with the
// slowest, so the last eighth of every XCD's rows of `slots` is left to
// workgroups that take slots as they free up, from any XCD's queue.  A
// quarter as many again as the queue rows run per XCD, so a fast XCD can
// take over that much of the others' ends.  Claiming a slot costs a round
// trip to memory or two, so only launches whose items average at least
// kQueueMinTiles tiles have a queue (row lengths of a dynamic plan are not
// known here: its launches keep one workgroup per slot).
constexpr int64_t kQueueMinRows = 16;
constexpr int64_t kQueueMinTiles = 16;
void build_queue(Plan& P, int k, const std::vector<int32_t>& slots, int64_t items, int64_t tiles) {
  P.queue_static[k] = int64_t(slots.size());
  P.queue_dyn_per_xcd[k] = 0;
  for (int32_t& t : P.queue_tail[k]) t = 0;
  const int64_t rows = int64_t(slots.size()) / kNumXcd;
  if (P.dynamic || items == 0 || tiles < kQueueMinTiles * items) return;
  if (int64_t(slots.size()) % kNumXcd != 0 || rows < kQueueMinRows) return;
  const int64_t tail_rows = (rows + 7) / 8;
  const int64_t cut = rows - tail_rows;
  // xcd_slots fills each XCD's rows from the first: its slots end at its
  // first idle one.
  for (int x = 0; x < kNumXcd; ++x) {
    int64_t len = 0;
    while (len < rows && slots[size_t(len * kNumXcd + x)] >= 0) ++len;
    P.queue_tail[k][x] = int32_t(std::max<int64_t>(0, len - cut));
  }
  P.queue_static[k] = cut * kNumXcd;
  P.queue_dyn_per_xcd[k] = tail_rows + (tail_rows + 3) / 4;
}

// The CSR transposed: for each layout head and k-block j, the ascending
// q-blocks i whose lists hold j, with the entry's flag.  The dK/dV part of
// the backward walks these lists.
void build_transpose(Plan& P) {
  const int64_t nb = P.nb;
  P.colT_ptr.assign(P.layout_heads, std::vector<int32_t>(nb + 1, 0));
  P.rowT_idx.assign(P.layout_heads, {});
  P.flagsT.assign(P.layout_heads, {});
  for (int lh = 0; lh < P.layout_heads; ++lh) {
    const auto& rp = P.row_ptr[lh];
    const auto& ci = P.col_idx[lh];
    auto& cp = P.colT_ptr[lh];
    for (int32_t j : ci) ++cp[j + 1];
    for (int64_t j = 0; j < nb; ++j) cp[j + 1] += cp[j];
    std::vector<int32_t> fill(cp.begin(), cp.end() - 1);
    P.rowT_idx[lh].resize(ci.size());
    P.flagsT[lh].resize(ci.size());
    for (int64_t i = 0; i < nb; ++i)          // ascending i keeps every column list sorted
      for (int32_t e = rp[i]; e < rp[i + 1]; ++e) {
        const int32_t at = fill[ci[e]]++;
        P.rowT_idx[lh][at] = int32_t(i);
        P.flagsT[lh][at] = P.flags[lh][e];
      }
  }
}

// Launch order of the dK/dV kernel: items (b * Hkv + hk) * nb + j in
// locality order (neighbouring k-blocks of one KV head share the q-blocks
// they read; KV head outer, batch entry next, as in the forward's order),
// cut per XCD by cost.  An item's walk is the concatenation of
// its group's transposed lists; walks longer than kv_chunk entries (twice the
// mean, at least 64) are cut into chunks that run as separate workgroups and
// write float32 partials, summed in chunk order by a reduction kernel, so a
// global key's column does not serialise the launch's tail.
void build_work_kv(Plan& P) {
  const int64_t B = P.prob.batch, H = P.prob.num_heads, Hkv = P.prob.num_kv_heads, nb = P.nb;
  const int64_t group = H / Hkv;
  const int64_t items = B * Hkv * nb;
  auto walk = [&](int64_t item) -> int64_t {
    const int64_t j = item % nb, hk = (item / nb) % Hkv;
    int64_t c = 0;
    for (int64_t h = hk * group; h < (hk + 1) * group; ++h) {
      const auto& cp = P.colT_ptr[P.layout_heads == 1 ? 0 : h];
      c += cp[j + 1] - cp[j];
    }
    return c;
  };
  int64_t total = 0;
  for (int64_t it = 0; it < items; ++it) total += walk(it);
  const int64_t mean = items ? (total + items - 1) / items : 0;
  P.kv_chunk = int32_t(std::max<int64_t>(64, 2 * mean));
  // Pieces in locality order: (item, begin, end, partial slot).
  std::vector<Plan::KvDesc> pieces;
  P.kv_reduce.clear();
  int64_t partials = 0;
  // For a bitmap, each (batch entry, KV head)'s k-blocks are taken longest
  // walk first, as the forward takes q-blocks (see build_work).
  std::vector<int64_t> order;
  order.reserve(items);
  for (int64_t hk = 0; hk < Hkv; ++hk)
    for (int64_t b = 0; b < B; ++b) {
      const size_t first = order.size();
      for (int64_t j = 0; j < nb; ++j) order.push_back((b * Hkv + hk) * nb + j);
      if (P.from_bitmap)
        std::stable_sort(order.begin() + first, order.end(),
                         [&](int64_t x, int64_t y) { return walk(x) > walk(y); });
    }
  for (int64_t l = 0; l < items; ++l) {
    const int64_t it = order[l];
    const int64_t n = walk(it);
    if (n <= P.kv_chunk) {
      pieces.push_back({int32_t(it), 0, int32_t(n), -1});
      continue;
    }
    const int64_t chunks = (n + P.kv_chunk - 1) / P.kv_chunk;
    P.kv_reduce.push_back({int32_t(it), int32_t(partials), int32_t(chunks), 0});
    for (int64_t c = 0; c < chunks; ++c)
      pieces.push_back({int32_t(it), int32_t(c * n / chunks), int32_t((c + 1) * n / chunks), int32_t(partials + c)});
    partials += chunks;
  }
  P.kv_partials = partials;
  std::vector<int32_t> loc(pieces.size());
  std::iota(loc.begin(), loc.end(), 0);
  // As for the forward (see build_work), a bitmap plan's runs take equal
  // item counts, unless walks were split (its pieces then differ in length
  // by design, and the cost split measured better).
  const bool unit = P.from_bitmap && P.kv_reduce.empty();
  const std::vector<int32_t> slots =
      loc.empty() ? loc
      : unit      ? xcd_slots(loc, [](int64_t) { return int64_t(1); })
                  : xcd_slots(loc, [&](int64_t k) { return int64_t(pieces[k].end - pieces[k].begin) + 1; });
  P.work_kv.assign(slots.size(), -1);
  P.kv_desc.assign(slots.size(), {-1, 0, 0, -1});
  for (size_t s = 0; s < slots.size(); ++s)
    if (slots[s] >= 0) {
      P.kv_desc[s] = pieces[slots[s]];
      P.work_kv[s] = pieces[slots[s]].item;
    }
  P.kv_reduce_launch = int64_t(P.kv_reduce.size());
  int64_t walked = 0;
  for (const auto& d : pieces) walked += d.end - d.begin;
  build_queue(P, 1, P.work_kv, int64_t(pieces.size()), walked);
}

// Launch order.  Item id = (b * H + h) * nb + i; cost = row length + 1.
void build_work(Plan& P) {
  const int64_t B = P.prob.batch, H = P.prob.num_heads, nb = P.nb;
  const int64_t group = P.prob.num_heads / P.prob.num_kv_heads;
  const int64_t items = B * H * nb;
  auto cost = [&](int64_t item) -> int64_t {
    if (P.dynamic) return 1;   // row lengths are only known on the device
    const int64_t i = item % nb, h = (item / nb) % H;
    const auto& rp = P.row_ptr[P.layout_heads == 1 ? 0 : h];
    return int64_t(rp[i + 1] - rp[i]) + 1;
  };
  P.work.clear();
  P.queue_static[0] = 0;
  P.queue_dyn_per_xcd[0] = 0;
  int schedule = P.prob.schedule == BSA_SCHEDULE_DEFAULT ? BSA_SCHEDULE_XCD : P.prob.schedule;
  if (schedule == BSA_SCHEDULE_ROWMAJOR || items == 0) {
    P.work.resize(items);
    std::iota(P.work.begin(), P.work.end(), 0);
  } else if (schedule == BSA_SCHEDULE_LPT) {
    std::vector<int32_t> order(items);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(),
                     [&](int32_t a, int32_t b) { return cost(a) > cost(b); });
    P.work = std::move(order);
  } else {
    // Locality order: heads sharing a KV head and neighbouring q-blocks are
    // adjacent, so the workgroups running together on one XCD read the same
    // K/V blocks through that XCD's L2.  KV heads are the outer loop and
    // batch entries the next, so every XCD's run holds all batch entries of
    // its KV heads: entries of different lengths (a variable-length batch)
    // load the XCDs evenly.
    // For a bitmap without the causal cut, neighbouring q-blocks share no
    // more K/V blocks than any two others, so a head's q-blocks are taken
    // longest row first instead: the workgroups that run together on an XCD
    // then have rows of about the same length, start and end about together,
    // and sweep the head's key blocks (in ascending order) at the same pace,
    // so the blocks they read at a time stay few enough for the XCD's L2.
    // Under the causal cut a row's length already grows with its q-block,
    // and the ascending order measured faster.
    std::vector<int32_t> loc;
    loc.reserve(items);
    std::vector<int32_t> order(nb);
    for (int64_t hk = 0; hk < H / group; ++hk)
      for (int64_t b = 0; b < B; ++b) {
        std::iota(order.begin(), order.end(), 0);
        if (P.from_bitmap && !P.dynamic && !P.causal) {
          const int64_t h0 = hk * group;
          std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
            return cost((b * H + h0) * nb + x) > cost((b * H + h0) * nb + y);
          });
        }
        for (int32_t i : order)
          for (int64_t g = 0; g < group; ++g) loc.push_back(int32_t((b * H + hk * group + g) * nb + i));
      }
    // Bitmap rows differ in length from head to head, and runs cut by tile
    // count split a (KV head, batch entry) run between two XCDs' L2s; equal
    // item counts keep whole runs on one XCD (when the runs divide evenly)
    // and leave the imbalance to the queue tail: random 32K forward 1.562 ->
    // 1.528 ms.
    P.work = P.from_bitmap ? xcd_slots(loc, [](int64_t) { return int64_t(1); }) : xcd_slots(loc, cost);
    int64_t tiles = 0;
    for (int32_t it : loc) tiles += cost(it) - 1;
    build_queue(P, 0, P.work, items, tiles);
  }
  if (P.queue_dyn_per_xcd[0] == 0) P.queue_static[0] = int64_t(P.work.size());
  P.info.work_items = items;
  P.info.launch_slots = int64_t(P.work.size());
}

bsa_status_t upload(Plan& P) {
  if (hipGetDevice(&P.device) != hipSuccess)
    return fail(BSA_ERR_DEVICE, "hipGetDevice failed: no usable HIP device");
  const size_t rows = size_t(P.layout_heads) * P.nb;
  const size_t nnz = size_t(P.info.nnz);
  const size_t slots = P.work.size();
  const size_t slots_kv = P.work_kv.size();
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  // [rows | entries | work | transposed rows | transposed entries | dK/dV work]
  const size_t off_entries = rows * sizeof(bsa::RowDesc);
  const size_t off_work = up(off_entries + nnz * sizeof(int32_t));
  const size_t off_cols = up(off_work + slots * sizeof(int32_t));
  const size_t off_entries_t = up(off_cols + rows * sizeof(bsa::RowDesc));
  const size_t off_work_kv = up(off_entries_t + nnz * sizeof(int32_t));
  const size_t off_kv_reduce = up(off_work_kv + slots_kv * sizeof(Plan::KvDesc));
  const size_t off_queue = up(off_kv_reduce + P.kv_reduce.size() * sizeof(Plan::KvDesc) + 16);
  const size_t bytes = off_queue + bsa::kQueueBytes;
  std::vector<unsigned char> host(bytes, 0);
  std::memcpy(host.data() + off_queue, P.queue_tail, sizeof(P.queue_tail));   // counters start at 0
  auto* rd = reinterpret_cast<bsa::RowDesc*>(host.data());
  auto* en = reinterpret_cast<int32_t*>(host.data() + off_entries);
  int32_t start = 0;
  for (int lh = 0; lh < P.layout_heads; ++lh) {
    for (int64_t i = 0; i < P.nb; ++i) {
      const int32_t a = P.row_ptr[lh][i], b = P.row_ptr[lh][i + 1];
      rd[size_t(lh) * P.nb + i] = {start + a, b - a};
    }
    for (size_t e = 0; e < P.col_idx[lh].size(); ++e)
      en[start + e] = bsa::encode_entry(P.col_idx[lh][e], P.flags[lh][e] != 0);
    start += int32_t(P.col_idx[lh].size());
  }
  if (slots) std::memcpy(host.data() + off_work, P.work.data(), slots * sizeof(int32_t));
  auto* cd = reinterpret_cast<bsa::RowDesc*>(host.data() + off_cols);
  auto* et = reinterpret_cast<int32_t*>(host.data() + off_entries_t);
  start = 0;
  for (int lh = 0; lh < P.layout_heads; ++lh) {
    for (int64_t j = 0; j < P.nb; ++j) {
      const int32_t a = P.colT_ptr[lh][j], b = P.colT_ptr[lh][j + 1];
      cd[size_t(lh) * P.nb + j] = {start + a, b - a};
    }
    for (size_t e = 0; e < P.rowT_idx[lh].size(); ++e)
      et[start + e] = bsa::encode_entry(P.rowT_idx[lh][e], P.flagsT[lh][e] != 0);
    start += int32_t(P.rowT_idx[lh].size());
  }
  if (slots_kv) std::memcpy(host.data() + off_work_kv, P.kv_desc.data(), slots_kv * sizeof(Plan::KvDesc));
  if (!P.kv_reduce.empty())
    std::memcpy(host.data() + off_kv_reduce, P.kv_reduce.data(), P.kv_reduce.size() * sizeof(Plan::KvDesc));
  hipError_t err = hipMalloc(&P.dev_mem, bytes);
  if (err != hipSuccess) {
    P.dev_mem = nullptr;
    return fail(err == hipErrorOutOfMemory ? BSA_ERR_OUT_OF_MEMORY : BSA_ERR_DEVICE,
                "hipMalloc(%zu) for the plan failed: %s", bytes, hipGetErrorString(err));
  }
  err = hipMemcpy(P.dev_mem, host.data(), bytes, hipMemcpyHostToDevice);
  if (err != hipSuccess) {
    (void)hipFree(P.dev_mem);
    P.dev_mem = nullptr;
    return fail(BSA_ERR_DEVICE, "plan upload failed: %s", hipGetErrorString(err));
  }
  auto* base = static_cast<unsigned char*>(P.dev_mem);
  P.d_rows = reinterpret_cast<const bsa::RowDesc*>(base);
  P.d_entries = reinterpret_cast<const int32_t*>(base + off_entries);
  P.d_work = reinterpret_cast<const int32_t*>(base + off_work);
  P.d_cols = reinterpret_cast<const bsa::RowDesc*>(base + off_cols);
  P.d_entries_t = reinterpret_cast<const int32_t*>(base + off_entries_t);
  P.d_work_kv = reinterpret_cast<const int32_t*>(base + off_work_kv);
  P.d_kv_reduce = reinterpret_cast<const int32_t*>(base + off_kv_reduce);
  P.d_queue = reinterpret_cast<int32_t*>(base + off_queue);
  if (P.kv_partials > 0 && P.prob.dtype == BSA_BF16 && P.prob.head_dim == 128 && P.prob.block_size == 128) {
    // float32 partial dK and dV of every chunk of a split column.
    const size_t sbytes = size_t(P.kv_partials) * 2 * 128 * 128 * sizeof(float);
    err = hipMalloc(&P.dev_scratch, sbytes);
    if (err != hipSuccess) {
      P.dev_scratch = nullptr;
      (void)hipFree(P.dev_mem);
      P.dev_mem = nullptr;
      return fail(err == hipErrorOutOfMemory ? BSA_ERR_OUT_OF_MEMORY : BSA_ERR_DEVICE,
                  "hipMalloc(%zu) for the backward's partial sums failed: %s", sbytes, hipGetErrorString(err));
    }
    P.d_kv_scratch = static_cast<float*>(P.dev_scratch);
  }
  P.info.on_device = 1;
  return BSA_OK;
}

bsa_status_t make_plan(const bsa_problem_t* problem, const bsa_layout_t* layout, bool dev,
                       bsa_plan_t* out) {
  bsa::clear_error();
  if (!out) return fail(BSA_ERR_INVALID_ARGUMENT, "out_plan must not be NULL");
  bsa_status_t st = validate(problem, layout);
  if (st != BSA_OK) return st;
  Plan* P = new (std::nothrow) Plan();
  if (!P) return fail(BSA_ERR_OUT_OF_MEMORY, "host allocation of the plan failed");
  try {
    P->prob = *problem;
    if (P->prob.scale == 0.f) P->prob.scale = 1.0f / std::sqrt(float(problem->head_dim));
    P->nb = int32_t((problem->seq_len + problem->block_size - 1) / problem->block_size);
    P->layout_heads = layout->bitmap ? layout->bitmap_heads : 1;
    P->causal = layout->causal;
    P->token_rule = (!layout->bitmap && layout->unit == BSA_UNIT_TOKENS) ? 1 : 0;
    P->from_bitmap = layout->bitmap ? 1 : 0;
    if (P->token_rule) {
      P->wl = layout->window_left;
      P->wr = layout->window_right;
      P->gk = layout->global_keys;
      P->gq = layout->global_queries;
    }
    build_csr(*P, *layout);
    build_work(*P);
    build_transpose(*P);
    build_work_kv(*P);
  } catch (const std::bad_alloc&) {
    delete P;
    return fail(BSA_ERR_OUT_OF_MEMORY, "host allocation while building the plan failed");
  }
  if (dev) {
    st = upload(*P);
    if (st != BSA_OK) {
      delete P;
      return st;
    }
  }
  *out = P;
  return BSA_OK;
}

// A plan whose CSR the device derives from a device-resident bitmap: the
// launch order (unit costs) and device arrays sized for the largest CSR.
bsa_status_t make_dynamic(const bsa_problem_t* problem, const bsa_layout_t* layout, bsa_plan_t* out) {
  bsa::clear_error();
  if (!out) return fail(BSA_ERR_INVALID_ARGUMENT, "out_plan must not be NULL");
  bsa_status_t st = validate(problem, layout);
  if (st != BSA_OK) return st;
  if (layout->bitmap)
    return fail(BSA_ERR_INVALID_ARGUMENT,
                "dynamic plan: layout->bitmap must be NULL (the bitmap is passed to bsa_plan_set_bitmap)");
  if (layout->bitmap_heads != 1 && layout->bitmap_heads != problem->num_heads)
    return fail(BSA_ERR_INVALID_ARGUMENT, "dynamic plan: bitmap_heads must be 1 or num_heads (%d), got %d",
                problem->num_heads, layout->bitmap_heads);
  if (layout->window_left != -1 || layout->window_right != -1 || layout->global_keys != 0 ||
      layout->global_queries != 0)
    return fail(BSA_ERR_INVALID_ARGUMENT,
                "dynamic plan: window_left/right must be -1 and global_keys/queries 0 (the bitmap is the layout)");
  // A seq_len the block does not divide ends in a shorter last block, as for
  // static plans: its tiles are PARTIAL (the device planner flags them).
  const int64_t nb = (problem->seq_len + problem->block_size - 1) / problem->block_size;
  const int64_t per_head = layout->causal ? nb * (nb + 1) / 2 : nb * nb;
  const int64_t cap = int64_t(layout->bitmap_heads) * per_head;
  if (cap > INT32_MAX)
    return fail(BSA_ERR_INVALID_ARGUMENT, "dynamic plan: %lld possible entries exceed 2^31 - 1",
                (long long)cap);
  Plan* P = new (std::nothrow) Plan();
  if (!P) return fail(BSA_ERR_OUT_OF_MEMORY, "host allocation of the plan failed");
  std::vector<int32_t> slot_of;   // dK/dV item -> its slot after the extra ones
  try {
    P->prob = *problem;
    if (P->prob.scale == 0.f) P->prob.scale = 1.0f / std::sqrt(float(problem->head_dim));
    P->nb = int32_t(nb);
    P->layout_heads = layout->bitmap_heads;
    P->causal = layout->causal;
    P->token_rule = 0;
    P->dynamic = 1;
    P->entry_capacity = cap;
    build_work(*P);
    // dK/dV launch order: one slot per (b, KV head, k-block), locality runs
    // per XCD with equal item counts.  For the bf16 backward, kv_extra_slots
    // slots (whole rounds of the XCD count, so every item keeps its XCD) go
    // before them for the chunks bsa_plan_set_bitmap cuts from long walks;
    // until then every walk is whole (and empty).
    const int64_t kv_items = int64_t(problem->batch) * problem->num_kv_heads * nb;
    std::vector<int32_t> loc(static_cast<size_t>(kv_items));
    std::iota(loc.begin(), loc.end(), 0);
    const std::vector<int32_t> order = loc.empty() ? loc : xcd_slots(loc, [](int64_t) { return int64_t(1); });
    const bool split = problem->dtype == BSA_BF16 && problem->head_dim == 128 && problem->block_size == 128;
    if (split && kv_items > 0) {
      P->kv_partials = std::min<int64_t>(kv_items, kDynamicPartials);
      P->kv_extra_slots = (P->kv_partials + kNumXcd - 1) / kNumXcd * kNumXcd;
      P->kv_reduce_launch = std::min<int64_t>(std::max<int64_t>(P->kv_partials / 2, 1), 64);
    }
    P->work_kv.assign(static_cast<size_t>(P->kv_extra_slots), -1);
    P->work_kv.insert(P->work_kv.end(), order.begin(), order.end());
    P->kv_desc.assign(P->work_kv.size(), {-1, 0, 0, -1});
    for (size_t s = 0; s < P->work_kv.size(); ++s)
      if (P->work_kv[s] >= 0) P->kv_desc[s] = {P->work_kv[s], 0, INT32_MAX, -1};
    P->queue_static[1] = int64_t(P->work_kv.size());   // no launch queue (lengths unknown here)
    P->queue_dyn_per_xcd[1] = 0;
    slot_of.assign(static_cast<size_t>(kv_items), -1);
    for (size_t s = 0; s < order.size(); ++s)
      if (order[s] >= 0) slot_of[static_cast<size_t>(order[s])] = int32_t(s);
  } catch (const std::bad_alloc&) {
    delete P;
    return fail(BSA_ERR_OUT_OF_MEMORY, "host allocation while building the plan failed");
  }
  P->info.layout_heads = P->layout_heads;
  P->info.num_blocks = int32_t(nb);
  P->info.nnz = P->info.nnz_partial = P->info.active_blocks = P->info.allowed_pairs = -1;
  P->info.max_row_entries = -1;
  if (hipGetDevice(&P->device) != hipSuccess) {
    delete P;
    return fail(BSA_ERR_DEVICE, "hipGetDevice failed: no usable HIP device");
  }
  // [rows | counts | entries | work | transposed rows | transposed entries |
  // dK/dV work | scan block sums | walk splitting: item slots, walks, chunk
  // prefixes, split columns, header], each part 256-byte aligned.
  const size_t rows = size_t(P->layout_heads) * P->nb;
  const bool split = P->kv_extra_slots > 0;
  const size_t kv_cols = split ? size_t(problem->num_kv_heads) * P->nb : 0;
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t off_counts = up(rows * sizeof(bsa::RowDesc));
  const size_t off_entries = off_counts + up(rows * sizeof(int32_t));
  const size_t off_work = off_entries + up(size_t(cap) * sizeof(int32_t));
  const size_t off_cols = off_work + up(P->work.size() * sizeof(int32_t));
  const size_t off_entries_t = off_cols + up(rows * sizeof(bsa::RowDesc));
  const size_t off_work_kv = off_entries_t + up(size_t(cap) * sizeof(int32_t));
  const size_t off_scan = off_work_kv + up(P->kv_desc.size() * sizeof(Plan::KvDesc));
  const size_t off_slot = off_scan + up(((rows + 1023) / 1024 + 1) * sizeof(int64_t));
  const size_t off_walk = off_slot + up((split ? slot_of.size() : 0) * sizeof(int32_t));
  const size_t off_pre = off_walk + up(kv_cols * sizeof(int32_t));
  const size_t off_reduce = off_pre + up(kv_cols * sizeof(int64_t));
  const size_t off_head = off_reduce + up(size_t(P->kv_partials) * sizeof(Plan::KvDesc));
  const size_t off_queue = off_head + up(8 * sizeof(int32_t));
  // Without the causal cut the launch order is re-sorted per bitmap (longest
  // row first): the order at creation and the per-KV-head q-block order.
  const bool reorder = !P->causal && !P->work.empty() &&
                       (P->prob.schedule == BSA_SCHEDULE_DEFAULT || P->prob.schedule == BSA_SCHEDULE_XCD);
  const size_t off_work_base = off_queue + up(bsa::kQueueBytes);
  const size_t off_order = off_work_base + up((reorder ? P->work.size() : 0) * sizeof(int32_t));
  const size_t bytes = off_order + (reorder ? size_t(problem->num_kv_heads) * P->nb * sizeof(int32_t) : 0);
  hipError_t err = hipMalloc(&P->dev_mem, bytes);
  if (err != hipSuccess) {
    P->dev_mem = nullptr;
    delete P;
    return fail(err == hipErrorOutOfMemory ? BSA_ERR_OUT_OF_MEMORY : BSA_ERR_DEVICE,
                "hipMalloc(%zu) for the dynamic plan failed: %s", bytes, hipGetErrorString(err));
  }
  auto* base = static_cast<unsigned char*>(P->dev_mem);
  // Empty rows and columns until the first bitmap arrives; the dK/dV order
  // never changes, the forward's only as above.
  err = hipMemset(base, 0, off_counts);
  if (err == hipSuccess) err = hipMemset(base + off_cols, 0, rows * sizeof(bsa::RowDesc));
  if (err == hipSuccess && !P->work.empty())
    err = hipMemcpy(base + off_work, P->work.data(), P->work.size() * sizeof(int32_t), hipMemcpyHostToDevice);
  if (err == hipSuccess && reorder)
    err = hipMemcpy(base + off_work_base, P->work.data(), P->work.size() * sizeof(int32_t), hipMemcpyHostToDevice);
  if (err == hipSuccess && !P->kv_desc.empty())
    err = hipMemcpy(base + off_work_kv, P->kv_desc.data(), P->kv_desc.size() * sizeof(Plan::KvDesc),
                    hipMemcpyHostToDevice);
  // No split column until the first bitmap arrives.
  if (err == hipSuccess) err = hipMemset(base + off_head, 0, 8 * sizeof(int32_t));
  // Launch queues: a dynamic plan has none (lengths 0; counters unused).
  if (err == hipSuccess) err = hipMemset(base + off_queue, 0, bsa::kQueueBytes);
  if (err == hipSuccess && split)
    err = hipMemcpy(base + off_slot, slot_of.data(), slot_of.size() * sizeof(int32_t), hipMemcpyHostToDevice);
  if (err == hipSuccess && split) {
    // float32 partial dK and dV of every chunk of a split column.
    const size_t sbytes = size_t(P->kv_partials) * 2 * 128 * 128 * sizeof(float);
    err = hipMalloc(&P->dev_scratch, sbytes);
    if (err != hipSuccess) {
      P->dev_scratch = nullptr;
      (void)hipFree(P->dev_mem);
      delete P;
      return fail(err == hipErrorOutOfMemory ? BSA_ERR_OUT_OF_MEMORY : BSA_ERR_DEVICE,
                  "hipMalloc(%zu) for the backward's partial sums failed: %s", sbytes, hipGetErrorString(err));
    }
    P->d_kv_scratch = static_cast<float*>(P->dev_scratch);
  }
  if (err != hipSuccess) {
    (void)hipFree(P->dev_mem);
    delete P;
    return fail(BSA_ERR_DEVICE, "dynamic plan upload failed: %s", hipGetErrorString(err));
  }
  P->d_rows = reinterpret_cast<const bsa::RowDesc*>(base);
  P->d_counts = reinterpret_cast<int32_t*>(base + off_counts);
  P->d_entries = reinterpret_cast<const int32_t*>(base + off_entries);
  P->d_work = reinterpret_cast<const int32_t*>(base + off_work);
  P->d_cols = reinterpret_cast<const bsa::RowDesc*>(base + off_cols);
  P->d_entries_t = reinterpret_cast<const int32_t*>(base + off_entries_t);
  P->d_work_kv = reinterpret_cast<const int32_t*>(base + off_work_kv);
  P->d_scan = reinterpret_cast<int64_t*>(base + off_scan);
  P->d_kv_reduce = reinterpret_cast<const int32_t*>(base + off_reduce);
  P->d_kv_head = reinterpret_cast<int32_t*>(base + off_head);
  P->d_queue = reinterpret_cast<int32_t*>(base + off_queue);
  P->d_kv_count = P->d_kv_head + 4;
  if (reorder) {
    P->d_work_base = reinterpret_cast<const int32_t*>(base + off_work_base);
    P->d_order = reinterpret_cast<int32_t*>(base + off_order);
  }
  if (split) {
    P->d_kv_slot = reinterpret_cast<const int32_t*>(base + off_slot);
    P->d_kv_walk = reinterpret_cast<int32_t*>(base + off_walk);
    P->d_kv_pre = reinterpret_cast<int64_t*>(base + off_pre);
  }
  P->info.on_device = 1;
  *out = P;
  return BSA_OK;
}

}  // namespace
}  // namespace bsa

extern "C" {

bsa_status_t bsa_plan_dynamic(const bsa_problem_t* problem, const bsa_layout_t* layout,
                              bsa_plan_t* out_plan) {
  return bsa::make_dynamic(problem, layout, out_plan);
}

bsa_status_t bsa_plan(const bsa_problem_t* problem, const bsa_layout_t* layout, bsa_plan_t* out_plan) {
  return bsa::make_plan(problem, layout, true, out_plan);
}

bsa_status_t bsa_plan_host(const bsa_problem_t* problem, const bsa_layout_t* layout,
                           bsa_plan_t* out_plan) {
  return bsa::make_plan(problem, layout, false, out_plan);
}

void bsa_plan_destroy(bsa_plan_t plan) {
  if (!plan) return;
  if (plan->dev_mem) {
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (cur != plan->device) (void)hipSetDevice(plan->device);
    (void)hipFree(plan->dev_mem);
    if (plan->dev_scratch) (void)hipFree(plan->dev_scratch);
    if (cur != plan->device && cur >= 0) (void)hipSetDevice(cur);
  }
  delete plan;
}

bsa_status_t bsa_plan_csr(bsa_plan_t plan, int32_t layout_head, const int32_t** row_ptr,
                          const int32_t** col_idx, const uint8_t** flags, int64_t* nnz) {
  bsa::clear_error();
  if (!plan || !row_ptr || !col_idx || !flags || !nnz)
    return bsa::fail(BSA_ERR_INVALID_ARGUMENT, "NULL argument to bsa_plan_csr");
  if (plan->dynamic)
    return bsa::fail(BSA_ERR_INVALID_ARGUMENT, "dynamic plan: its CSR lives on the device (bsa_plan_read_csr)");
  if (layout_head < 0 || layout_head >= plan->layout_heads)
    return bsa::fail(BSA_ERR_INVALID_ARGUMENT, "layout_head %d out of range [0, %d)", layout_head,
                     plan->layout_heads);
  *row_ptr = plan->row_ptr[layout_head].data();
  *col_idx = plan->col_idx[layout_head].data();
  *flags = plan->flags[layout_head].data();
  *nnz = int64_t(plan->col_idx[layout_head].size());
  return BSA_OK;
}

bsa_status_t bsa_plan_get_info(bsa_plan_t plan, bsa_plan_info_t* info) {
  bsa::clear_error();
  if (!plan || !info) return bsa::fail(BSA_ERR_INVALID_ARGUMENT, "NULL argument to bsa_plan_get_info");
  *info = plan->info;
  return BSA_OK;
}

bsa_status_t bsa_plan_work(bsa_plan_t plan, const int32_t** work, int64_t* slots) {
  bsa::clear_error();
  if (!plan || !work || !slots) return bsa::fail(BSA_ERR_INVALID_ARGUMENT, "NULL argument to bsa_plan_work");
  *work = plan->work.data();
  *slots = int64_t(plan->work.size());
  return BSA_OK;
}

int64_t bsa_plan_active_blocks(bsa_plan_t plan) { return plan ? plan->info.active_blocks : -1; }

bsa_status_t bsa_plan_csr_transposed(bsa_plan_t plan, int32_t layout_head, const int32_t** col_ptr,
                                     const int32_t** row_idx, const uint8_t** flags, int64_t* nnz) {
  bsa::clear_error();
  if (!plan || !col_ptr || !row_idx || !flags || !nnz)
    return bsa::fail(BSA_ERR_INVALID_ARGUMENT, "NULL argument to bsa_plan_csr_transposed");
  if (plan->dynamic)
    return bsa::fail(BSA_ERR_INVALID_ARGUMENT, "dynamic plan: its transposed CSR lives on the device");
  if (layout_head < 0 || layout_head >= plan->layout_heads)
    return bsa::fail(BSA_ERR_INVALID_ARGUMENT, "layout_head %d out of range [0, %d)", layout_head,
                     plan->layout_heads);
  *col_ptr = plan->colT_ptr[layout_head].data();
  *row_idx = plan->rowT_idx[layout_head].data();
  *flags = plan->flagsT[layout_head].data();
  *nnz = int64_t(plan->rowT_idx[layout_head].size());
  return BSA_OK;
}

bsa_status_t bsa_plan_work_kv(bsa_plan_t plan, const int32_t** work, int64_t* slots) {
  bsa::clear_error();
  if (!plan || !work || !slots)
    return bsa::fail(BSA_ERR_INVALID_ARGUMENT, "NULL argument to bsa_plan_work_kv");
  *work = plan->work_kv.data();
  *slots = int64_t(plan->work_kv.size());
  return BSA_OK;
}

const char* bsa_status_string(bsa_status_t s) {
  switch (s) {
    case BSA_OK: return "BSA_OK";
    case BSA_ERR_INVALID_ARGUMENT: return "BSA_ERR_INVALID_ARGUMENT";
    case BSA_ERR_UNSUPPORTED: return "BSA_ERR_UNSUPPORTED";
    case BSA_ERR_OUT_OF_MEMORY: return "BSA_ERR_OUT_OF_MEMORY";
    case BSA_ERR_DEVICE: return "BSA_ERR_DEVICE";
    default: return "BSA_ERR_UNKNOWN";
  }
}

const char* bsa_last_error(void) { return bsa::g_last_error.c_str(); }

int32_t bsa_abi_version(void) { return BSA_ABI_VERSION; }

}  // extern "C"
