// Device-side planner for dynamic plans: a block bitmap in device memory ->
// the per-q-block CSR of key blocks the forward walks, with FULL/PARTIAL
// flags, without a round trip through the host.
//
// The CSR is the same as the host planner's for a bitmap layout: tile (i, j)
// of layout head hl is an entry iff bitmap[hl][i][j] != 0 and, for a causal
// layout, j <= i; the diagonal tile of a causal layout is PARTIAL (the
// token-exact causal cut), and so is every tile of a shorter last block (a
// seq_len the block does not divide); every other entry is FULL.  Entries are ascending in
// j.  Three steps: count the entries of each row, scan the counts into row
// offsets (three small kernels), write each row's entries; then the same for
// the k-block columns the backward walks.  The per-query-block lists follow step
// three of "How Does Flash-MSA Sparse Attention Work?" and the precomputed
// block offsets of the FAQ on sparse kernels slower than dense ("How Do
// Sparse Attention Kernels Work in GPU Clusters?"); building them on the
// device serves masks that change per input (the dynamic-sparsity FAQ of the
// same page, the learned per-head block masks of "Flash-MSA" on "The Only
// Guide You Need for Sparse Attention Kernels in Long-Context LLMs").
#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

#include "internal.h"

namespace bsa {
namespace {

// Rows: one wave per row (layout head * nb + i), four rows per workgroup.
// With kVec = 16 (nb and the bitmap's address multiples of 16, so every row
// is 16-byte aligned) lane L reads bytes [16 L, 16 L + 16) of each 1 KB
// stretch of its row with one load; with kVec = 1 it reads byte L of each
// 64-byte stretch.  Only the bytes below the row's last column (the diagonal
// under the causal cut) count.
constexpr int kRowThreads = 256;
constexpr int kRowWaves = kRowThreads / 64;

// Bit v set iff byte v of the kVec bytes at p is nonzero, for v < lim (the
// bytes at or beyond lim are not read when kVec is 1, and are read but
// dropped when kVec is 16; the caller keeps all 16 inside the row).
template <int kVec>
__device__ __forceinline__ uint32_t nonzero_bits(const uint8_t* p, int lim) {
  if (lim <= 0) return 0;
  if constexpr (kVec == 1) {
    return p[0] != 0 ? 1u : 0u;
  } else {
    const uint4 x = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t bits = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      // Bit 7 of each byte: set iff the byte is nonzero (its low 7 bits
      // carry into bit 7 when any is set, or bit 7 is set already).
      const uint32_t hi = (((w[k] & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | w[k]) & 0x80808080u;
      bits |= (((hi >> 7) & 1u) | ((hi >> 14) & 2u) | ((hi >> 21) & 4u) | ((hi >> 28) & 8u)) << (4 * k);
    }
    return lim >= 16 ? bits : bits & ((1u << lim) - 1u);
  }
}

// counts[row] = entries of row.
template <int kVec>
__global__ __launch_bounds__(kRowThreads) void count_rows(const uint8_t* __restrict__ bm, int nb, int nrows,
                                                          int causal, int32_t* __restrict__ counts) {
  const int row = blockIdx.x * kRowWaves + (threadIdx.x >> 6);
  if (row >= nrows) return;                          // whole waves
  const int lane = threadIdx.x & 63;
  const int i = row % nb;
  const int jend = causal ? i + 1 : nb;
  const uint8_t* r = bm + size_t(row) * nb;
  int c = 0;
  for (int j0 = lane * kVec; j0 < jend; j0 += 64 * kVec) c += __popc(nonzero_bits<kVec>(r + j0, jend - j0));
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) c += __shfl_xor(c, w);
  if (lane == 0) counts[row] = c;
}

// rows[x] = {exclusive prefix of counts, counts[x]} over all n rows, and
// *d_nnz = the total: per-block sums of kScanBlock counts, one workgroup
// scanning those sums in place (sums[nblk] = total), and each block's local
// scan offset by its sum's prefix.
constexpr int kScanBlock = 1024;
constexpr int kScanWaves = kScanBlock / 64;
constexpr int kSmallScanBlocks = 8;     // up to this many blocks of rows: one-workgroup scan

// Inclusive scan of v over the workgroup (blockDim.x == kScanBlock); total
// receives the workgroup's sum.  wsum: kScanWaves values of LDS.
__device__ __forceinline__ long long block_scan(long long v, long long* wsum, long long& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const long long y = __shfl_up(v, d);
    if (lane >= d) v += y;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  if (wave == 0) {
    long long w = lane < kScanWaves ? wsum[lane] : 0;
#pragma unroll
    for (int d = 1; d < kScanWaves; d <<= 1) {
      const long long y = __shfl_up(w, d);
      if (lane >= d) w += y;
    }
    if (lane < kScanWaves) wsum[lane] = w;
  }
  __syncthreads();
  total = wsum[kScanWaves - 1];
  return v + (wave ? wsum[wave - 1] : 0);
}

__global__ __launch_bounds__(kScanBlock) void scan_block_sums(const int32_t* __restrict__ counts, int n,
                                                              int64_t* __restrict__ sums) {
  __shared__ long long wsum[kScanWaves];
  const int x = blockIdx.x * kScanBlock + threadIdx.x;
  long long total;
  block_scan(x < n ? counts[x] : 0, wsum, total);
  if (threadIdx.x == 0) sums[blockIdx.x] = total;
}

__global__ __launch_bounds__(kScanBlock) void scan_sums(int64_t* __restrict__ sums, int nblk) {
  __shared__ long long wsum[kScanWaves];
  long long carry = 0;
  for (int c0 = 0; c0 < nblk; c0 += kScanBlock) {
    const int x = c0 + threadIdx.x;
    const long long v = x < nblk ? sums[x] : 0;
    long long total;
    const long long inc = block_scan(v, wsum, total);
    __syncthreads();                                   // wsum is reused by the next chunk
    if (x < nblk) sums[x] = carry + inc - v;           // exclusive prefix
    carry += total;
  }
  if (threadIdx.x == 0) sums[nblk] = carry;
}

// The whole scan in one workgroup, chunk by chunk (few rows: one launch
// instead of three).
__global__ __launch_bounds__(kScanBlock) void scan_small(const int32_t* __restrict__ counts, int n,
                                                         RowDesc* __restrict__ rows, int64_t* d_nnz) {
  __shared__ long long wsum[kScanWaves];
  long long carry = 0;
  for (int c0 = 0; c0 < n; c0 += kScanBlock) {
    const int x = c0 + threadIdx.x;
    const int32_t c = x < n ? counts[x] : 0;
    long long total;
    const long long inc = block_scan(c, wsum, total);
    __syncthreads();                                   // wsum is reused by the next chunk
    if (x < n) rows[x] = {int32_t(carry + inc - c), c};
    carry += total;
  }
  if (d_nnz && threadIdx.x == 0) *d_nnz = carry;
}

__global__ __launch_bounds__(kScanBlock) void scan_apply(const int32_t* __restrict__ counts, int n,
                                                         const int64_t* __restrict__ sums, int nblk,
                                                         RowDesc* __restrict__ rows, int64_t* d_nnz) {
  __shared__ long long wsum[kScanWaves];
  const int x = blockIdx.x * kScanBlock + threadIdx.x;
  const int32_t c = x < n ? counts[x] : 0;
  long long total;
  const long long inc = block_scan(c, wsum, total);
  if (x < n) rows[x] = {int32_t(sums[blockIdx.x] + inc - c), c};
  if (d_nnz && blockIdx.x == 0 && threadIdx.x == 0) *d_nnz = sums[nblk];
}

// The entries of each row, ascending: entry = (j << 1) | partial.  Each
// stretch of the row: every lane's count, their exclusive prefix over the
// wave, and each lane writes its entries from there in column order.
template <int kVec>
__global__ __launch_bounds__(kRowThreads) void fill_rows(const uint8_t* __restrict__ bm, int nb, int nrows,
                                                         int causal, int tail, const RowDesc* __restrict__ rows,
                                                         int32_t* __restrict__ entries) {
  const int row = blockIdx.x * kRowWaves + (threadIdx.x >> 6);
  if (row >= nrows) return;                          // whole waves
  const int lane = threadIdx.x & 63;
  const int i = row % nb;
  const int jend = causal ? i + 1 : nb;
  const uint8_t* r = bm + size_t(row) * nb;
  int32_t* out = entries + rows[row].start;
  int base = 0;
  for (int p0 = 0; p0 < jend; p0 += 64 * kVec) {     // wave-uniform
    const int j0 = p0 + lane * kVec;
    uint32_t bits = j0 < jend ? nonzero_bits<kVec>(r + j0, jend - j0) : 0u;
    const int c = __popc(bits);
    int inc = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(inc, d);
      if (lane >= d) inc += y;
    }
    int pos = base + inc - c;
    while (bits) {
      const int j = j0 + __builtin_ctz(bits);
      bits &= bits - 1u;
      out[pos++] = (j << 1) | (((causal && j == i) || i == tail || j == tail) ? 1 : 0);
    }
    base += __shfl(inc, 63);
  }
}

// The transposed CSR for the backward: the q-blocks i of each k-block column
// (layout head * nb + j) with bitmap[hl][i][j] != 0 (and i >= j for a causal
// layout), ascending, entry = (i << 1) | partial.  One workgroup per strip of
// kStrip * kVec columns of one layout head: lane l of every wave owns the kVec
// columns j0 .. j0 + kVec - 1, j0 = strip start + kVec * l, and reads them
// with one load per row (kVec = 4 when nb is a multiple of 4, so every row
// of 4-byte groups is aligned; else 1), so each wave reads kStrip * kVec
// consecutive bytes of a row per load; wave w owns the contiguous row chunk
// [w * chunk, (w + 1) * chunk), loading kRowBatch rows at a time before it
// uses them (so each lane has that many loads in flight).  The count kernel adds the chunks' counts;
// the fill kernel recounts its chunk, takes the counts of the chunks above it
// as its offset in each column's list and writes its entries in row order,
// so every list comes out ascending.
constexpr int kStrip = 64;
constexpr int kChunks = 16;
constexpr int kStripThreads = kStrip * kChunks;
constexpr int64_t kWideMinStrips = 256;
constexpr int kRowBatch = 8;              // rows loaded together per lane   // 4-column lanes only with at least this many workgroups

struct StripCursor {
  const uint8_t* col;   // bitmap byte (row 0, this lane's first column)
  int j0, i0, i1;       // first column; rows [i0, i1) of this wave's chunk
  bool valid;
};

template <int kVec>
__device__ __forceinline__ int strips_of(int nb) {
  return (nb + kStrip * kVec - 1) / (kStrip * kVec);
}

template <int kVec>
__device__ __forceinline__ StripCursor strip_cursor(const uint8_t* bm, int nb, int causal) {
  const int strips = strips_of<kVec>(nb);
  const int hl = blockIdx.x / strips, s = blockIdx.x % strips;
  const int lane = threadIdx.x % kStrip, w = threadIdx.x / kStrip;
  const int chunk = (nb + kChunks - 1) / kChunks;
  StripCursor c;
  c.j0 = s * kStrip * kVec + lane * kVec;
  c.valid = c.j0 < nb;                 // all kVec columns, as kVec divides nb
  c.col = bm + size_t(hl) * nb * nb + (c.valid ? c.j0 : 0);
  c.i0 = min(nb, w * chunk);
  c.i1 = min(nb, c.i0 + chunk);
  // Under the causal cut, rows below the lane's first column hold none of its entries.
  if (causal && c.i0 < c.j0) c.i0 = min(c.j0, c.i1);
  return c;
}

// The bytes of row i of the lane's columns (byte v of the result = column j0 + v).
template <int kVec>
__device__ __forceinline__ uint32_t strip_row(const StripCursor& c, int nb, int i) {
  if constexpr (kVec == 4)
    return *reinterpret_cast<const uint32_t*>(c.col + size_t(i) * nb);
  else
    return c.col[size_t(i) * nb];
}

template <int kVec>
__device__ __forceinline__ bool strip_on(uint32_t x, int v, int i, int j0, int causal) {
  return ((x >> (8 * v)) & 255u) != 0 && (!causal || i >= j0 + v);
}

template <int kVec>
__device__ __forceinline__ void strip_count(const StripCursor& c, int nb, int causal, int (&n)[kVec]) {
#pragma unroll
  for (int v = 0; v < kVec; ++v) n[v] = 0;
  if (!c.valid) return;
  for (int i = c.i0; i < c.i1; i += kRowBatch) {
    uint32_t x[kRowBatch];
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u) x[u] = i + u < c.i1 ? strip_row<kVec>(c, nb, i + u) : 0u;
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u)
#pragma unroll
      for (int v = 0; v < kVec; ++v) n[v] += strip_on<kVec>(x[u], v, i + u, c.j0, causal);
  }
}

template <int kVec>
__global__ __launch_bounds__(kStripThreads) void count_cols(const uint8_t* __restrict__ bm, int nb, int causal,
                                                            int32_t* __restrict__ counts) {
  __shared__ int part[kChunks][kStrip * kVec];
  const StripCursor c = strip_cursor<kVec>(bm, nb, causal);
  const int lane = threadIdx.x % kStrip, w = threadIdx.x / kStrip;
  int n[kVec];
  strip_count<kVec>(c, nb, causal, n);
#pragma unroll
  for (int v = 0; v < kVec; ++v) part[w][lane * kVec + v] = n[v];
  __syncthreads();
  if (w == 0 && c.valid) {
    const int hl = blockIdx.x / strips_of<kVec>(nb);
#pragma unroll
    for (int v = 0; v < kVec; ++v) {
      int total = 0;
      for (int x = 0; x < kChunks; ++x) total += part[x][lane * kVec + v];
      counts[hl * nb + c.j0 + v] = total;
    }
  }
}

// kMasks: the wave's chunk has at most kMaskBatches * kRowBatch rows (nb at
// most kChunks times that), and the count pass keeps, per batch of
// kRowBatch rows, the lane's entry bits (bit u * kVec + v: row i0 + u,
// column j0 + v) in registers, so the write pass reads no bitmap byte again.
constexpr int kMaskBatches = 16;

template <int kVec, bool kMasks>
__global__ __launch_bounds__(kStripThreads) void fill_cols(const uint8_t* __restrict__ bm, int nb, int causal,
                                                           int tail, const RowDesc* __restrict__ cols,
                                                           int32_t* __restrict__ entries) {
  __shared__ int part[kChunks][kStrip * kVec];
  const StripCursor c = strip_cursor<kVec>(bm, nb, causal);
  const int lane = threadIdx.x % kStrip, w = threadIdx.x / kStrip;
  int n[kVec];
  uint32_t mk[kMasks ? kMaskBatches : 1];
  if constexpr (kMasks) {
    static_assert(kVec * kRowBatch <= 32, "one word of entry bits per batch");
#pragma unroll
    for (int v = 0; v < kVec; ++v) n[v] = 0;
#pragma unroll
    for (int bb = 0; bb < kMaskBatches; ++bb) {
      const int i0 = c.i0 + bb * kRowBatch;
      uint32_t m = 0;
      if (c.valid && i0 < c.i1) {
        uint32_t x[kRowBatch];
#pragma unroll
        for (int u = 0; u < kRowBatch; ++u) x[u] = i0 + u < c.i1 ? strip_row<kVec>(c, nb, i0 + u) : 0u;
#pragma unroll
        for (int u = 0; u < kRowBatch; ++u)
#pragma unroll
          for (int v = 0; v < kVec; ++v)
            if (strip_on<kVec>(x[u], v, i0 + u, c.j0, causal)) m |= 1u << (u * kVec + v);
      }
      mk[bb] = m;
#pragma unroll
      for (int v = 0; v < kVec; ++v) {
        uint32_t col = 0;
#pragma unroll
        for (int u = 0; u < kRowBatch; ++u) col |= 1u << (u * kVec + v);
        n[v] += __popc(m & col);
      }
    }
  } else {
    strip_count<kVec>(c, nb, causal, n);
  }
#pragma unroll
  for (int v = 0; v < kVec; ++v) part[w][lane * kVec + v] = n[v];
  __syncthreads();
  if (!c.valid) return;
  const int hl = blockIdx.x / strips_of<kVec>(nb);
  int off[kVec];
#pragma unroll
  for (int v = 0; v < kVec; ++v) {
    off[v] = cols[hl * nb + c.j0 + v].start;
    for (int x = 0; x < w; ++x) off[v] += part[x][lane * kVec + v];
  }
  auto put = [&](int i, int v) {
    entries[off[v]++] = (i << 1) | (((causal && i == c.j0 + v) || i == tail || c.j0 + v == tail) ? 1 : 0);
  };
  if constexpr (kMasks) {
#pragma unroll
    for (int bb = 0; bb < kMaskBatches; ++bb) {
      const uint32_t m = mk[bb];
      if (m == 0) continue;
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u)
#pragma unroll
        for (int v = 0; v < kVec; ++v)
          if ((m >> (u * kVec + v)) & 1u) put(c.i0 + bb * kRowBatch + u, v);
    }
  } else {
    for (int i0 = c.i0; i0 < c.i1; i0 += kRowBatch) {
      uint32_t x[kRowBatch];
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) x[u] = i0 + u < c.i1 ? strip_row<kVec>(c, nb, i0 + u) : 0u;
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u)
#pragma unroll
        for (int v = 0; v < kVec; ++v)
          if (strip_on<kVec>(x[u], v, i0 + u, c.j0, causal)) put(i0 + u, v);
    }
  }
}

// ---------------------------------------------------------------------------
// Cutting long dK/dV walks (bf16 backward of a dynamic plan).  The walk of
// item (b, hk, j) is the transposed lists of column j of the KV group's
// query heads, one after another: walk[hk * nb + j] entries, the same for
// every batch entry.  As the host planner does for static plans, a walk
// longer than the chunk length C = max(64, 2 * mean walk) becomes
// k = ceil(L / C) chunks [c * L / k, (c + 1) * L / k); here C doubles until
// the chunks fit the plan's partial-tile and slot budgets.  A wide kernel
// sums each column's walk over the group's lists; one workgroup then
// finds C and, per column, the exclusive prefixes of the extra chunks
// (beyond each split column's first), the partial tiles and the split
// columns, packed 21 bits each (the budgets keep every sum below 2^20); a
// wide kernel then writes the launch descriptors and the reduction list.
// ---------------------------------------------------------------------------
constexpr int kPackBits = 21;
constexpr long long kPackMask = (1ll << kPackBits) - 1;
constexpr int kWriteThreads = 256;

__device__ __forceinline__ long long split_pack(long long L, long long chunk) {
  if (L <= chunk) return 0;
  const long long k = (L + chunk - 1) / chunk;
  return (k - 1) | (k << kPackBits) | (1ll << (2 * kPackBits));
}

// walk[x] for every column x = hk * nb + j: one thread each.
__global__ __launch_bounds__(kWriteThreads) void kv_walks(const RowDesc* __restrict__ cols, int nb, int n,
                                                          int group, int per_head, int32_t* __restrict__ walk) {
  const int x = blockIdx.x * kWriteThreads + threadIdx.x;
  if (x >= n) return;
  const int hk = x / nb, j = x - hk * nb;
  int L = 0;
  for (int g = 0; g < group; ++g) L += cols[(per_head ? hk * group + g : 0) * nb + j].count;
  walk[x] = L;
}

// head: [0] chunk length, [1] extra chunks, [2] partial tiles, [3] split
// columns (each per batch entry), [4] split columns in all.
__global__ __launch_bounds__(kScanBlock) void kv_split_plan(int n, int batch, long long max_extra,
                                                            long long max_parts, const int32_t* __restrict__ walk,
                                                            int64_t* __restrict__ pre, int32_t* __restrict__ head) {
  __shared__ long long wsum[kScanWaves];
  // Sums run over columns x = t, t + kScanBlock, ... (coalesced reads).
  long long mine = 0;
  for (int x = threadIdx.x; x < n; x += kScanBlock) mine += walk[x];
  long long total;
  block_scan(mine, wsum, total);
  __syncthreads();
  long long chunk = n > 0 ? 2 * ((total + n - 1) / n) : 0;
  if (chunk < 64) chunk = 64;
  for (;;) {
    // Extra chunks (low 32 bits) and partial tiles (high 32 bits) at this chunk length.
    long long ep = 0;
    for (int x = threadIdx.x; x < n; x += kScanBlock) {
      const long long L = walk[x];
      if (L > chunk) {
        const long long k = (L + chunk - 1) / chunk;
        ep += (k - 1) + (k << 32);
      }
    }
    long long sum;
    block_scan(ep, wsum, sum);
    __syncthreads();
    if ((sum & 0xffffffffll) * batch <= max_extra && (sum >> 32) * batch <= max_parts) break;
    chunk *= 2;
  }
  // Exclusive prefix of the packed counts in column order, kScanBlock columns at a time.
  long long all = 0;
  for (int c0 = 0; c0 < n; c0 += kScanBlock) {
    const int x = c0 + threadIdx.x;
    const long long v = x < n ? split_pack(walk[x], chunk) : 0;
    long long part;
    const long long inc = block_scan(v, wsum, part);
    __syncthreads();                                   // wsum is reused by the next block of columns
    if (x < n) pre[x] = all + inc - v;
    all += part;
  }
  if (threadIdx.x == 0) {
    head[0] = int32_t(chunk < 0x7fffffffll ? chunk : 0x7fffffffll);
    head[1] = int32_t(all & kPackMask);
    head[2] = int32_t((all >> kPackBits) & kPackMask);
    head[3] = int32_t((all >> (2 * kPackBits)) & kPackMask);
    head[4] = batch * head[3];
  }
}

// One thread per item t = b * n + hk * nb + j (and per extra slot): the
// item's own slot runs its whole walk or its first chunk; the other chunks go
// to the extra slots, the split column to the reduction list; extra slots
// left over are idle.
__global__ __launch_bounds__(kWriteThreads) void kv_split_write(const int32_t* __restrict__ walk,
                                                                const int64_t* __restrict__ pre,
                                                                const int32_t* __restrict__ head,
                                                                const int32_t* __restrict__ slot_of, int n,
                                                                int64_t items, int64_t extra_slots,
                                                                int4* __restrict__ desc, int4* __restrict__ reduce) {
  const int64_t t = int64_t(blockIdx.x) * kWriteThreads + threadIdx.x;
  const int chunk = head[0], e_b = head[1], p_b = head[2], s_b = head[3];
  const int64_t b = t / n;
  if (t >= (items / n) * e_b && t < extra_slots) desc[t] = make_int4(-1, 0, 0, -1);
  if (t >= items) return;
  const int x = int(t - b * n);
  const int L = walk[x];
  const int s = slot_of[t];
  if (s < 0) return;
  int4* own = desc + extra_slots + s;
  if (L <= chunk) {
    *own = make_int4(int(t), 0, L, -1);
    return;
  }
  const long long pk = pre[x];
  const int e0 = int(pk & kPackMask), p0 = int((pk >> kPackBits) & kPackMask);
  const int r0 = int((pk >> (2 * kPackBits)) & kPackMask);
  const int k = (L + chunk - 1) / chunk;
  const int pb = int(b * p_b + p0);
  *own = make_int4(int(t), 0, L / k, pb);
  int4* ex = desc + b * e_b + e0 - 1;    // chunk c >= 1 at ex[c]
  for (int c = 1; c < k; ++c)
    ex[c] = make_int4(int(t), int(int64_t(c) * L / k), int(int64_t(c + 1) * L / k), pb + c);
  reduce[b * s_b + r0] = make_int4(int(t), pb, k, 0);
}

// Launch order of a dynamic plan without the causal cut, longest row first
// within each (KV head, batch entry) run, as the host planner orders the
// q-blocks of a static bitmap plan (the workgroups that run together on an
// XCD then have rows of about the same length and sweep the key blocks at
// the same pace).  order_rows: one workgroup per KV head ranks the q-blocks
// of its group's first query head's layout by descending row length, a
// counting sort over kOrderBuckets buckets (lengths from kOrderBuckets - 1 up
// share the last); the order inside a bucket is whatever the atomics give,
// which changes only which slot runs a q-block, not what it computes.
constexpr int kOrderThreads = 256;
constexpr int kOrderBuckets = 1024;
__global__ __launch_bounds__(kOrderThreads) void order_rows(const RowDesc* __restrict__ rows, int nb, int group,
                                                            int per_head, int32_t* __restrict__ order) {
  __shared__ int hist[kOrderBuckets];
  __shared__ int part[kOrderThreads];
  const int hk = blockIdx.x;
  const RowDesc* r = rows + size_t(per_head ? hk * group : 0) * nb;
  for (int x = threadIdx.x; x < kOrderBuckets; x += kOrderThreads) hist[x] = 0;
  __syncthreads();
  auto key = [](int c) { return kOrderBuckets - 1 - (c < kOrderBuckets - 1 ? c : kOrderBuckets - 1); };
  for (int i = threadIdx.x; i < nb; i += kOrderThreads) atomicAdd(&hist[key(r[i].count)], 1);
  __syncthreads();
  // Exclusive scan of the buckets: each thread sums its 4, the 256 partial
  // sums are scanned in place, then each thread writes its 4 offsets.
  constexpr int kPer = kOrderBuckets / kOrderThreads;
  const int t = threadIdx.x;
  int local = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) local += hist[t * kPer + u];
  part[t] = local;
  __syncthreads();
  for (int off = 1; off < kOrderThreads; off <<= 1) {
    const int v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int run = part[t] - local;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int c = hist[t * kPer + u];
    hist[t * kPer + u] = run;
    run += c;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nb; i += kOrderThreads) order[size_t(hk) * nb + atomicAdd(&hist[key(r[i].count)], 1)] = i;
}

// work[s] = work_base[s] with its q-block i replaced by the i-th of its KV
// head's order (idle slots stay idle).
__global__ __launch_bounds__(kOrderThreads) void reorder_work(const int32_t* __restrict__ base, int64_t slots,
                                                              int nb, int H, int group,
                                                              const int32_t* __restrict__ order,
                                                              int32_t* __restrict__ work) {
  const int64_t s = int64_t(blockIdx.x) * kOrderThreads + threadIdx.x;
  if (s >= slots) return;
  const int32_t item = base[s];
  if (item < 0) {
    work[s] = -1;
    return;
  }
  const int i = item % nb, bh = item / nb;
  const int hk = (bh % H) / group;
  work[s] = bh * nb + order[size_t(hk) * nb + i];
}

}  // namespace
}  // namespace bsa

extern "C" bsa_status_t bsa_plan_set_bitmap(bsa_plan_t plan, const uint8_t* d_bitmap, int64_t* d_nnz,
                                            void* stream) {
  using namespace bsa;
  clear_error();
  if (!plan || !d_bitmap) return fail(BSA_ERR_INVALID_ARGUMENT, "plan and d_bitmap must not be NULL");
  if (!plan->dynamic) return fail(BSA_ERR_INVALID_ARGUMENT, "plan was not made by bsa_plan_dynamic");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(BSA_ERR_DEVICE, "hipGetDevice failed");
  if (dev != plan->device)
    return fail(BSA_ERR_INVALID_ARGUMENT, "plan was built on device %d but device %d is current",
                plan->device, dev);
  for (const void* ptr : {static_cast<const void*>(d_bitmap), static_cast<const void*>(d_nnz)}) {
    if (!ptr) continue;
    hipPointerAttribute_t attr{};
    if (hipPointerGetAttributes(&attr, ptr) != hipSuccess || attr.type != hipMemoryTypeDevice ||
        attr.device != plan->device) {
      (void)hipGetLastError();
      return fail(BSA_ERR_INVALID_ARGUMENT, "d_bitmap and d_nnz must be device memory of device %d",
                  plan->device);
    }
  }
  const int nb = plan->nb;
  const int rows = plan->layout_heads * nb;
  if (rows == 0) return BSA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto* d_rows = const_cast<RowDesc*>(plan->d_rows);
  auto* d_entries = const_cast<int32_t*>(plan->d_entries);
  // 16-byte loads when every row of the bitmap is 16-byte aligned.
  const bool rows16 = nb % 16 == 0 && reinterpret_cast<uintptr_t>(d_bitmap) % 16 == 0;
  const unsigned row_groups = unsigned((rows + kRowWaves - 1) / kRowWaves);
  if (rows16)
    hipLaunchKernelGGL(count_rows<16>, dim3(row_groups), dim3(kRowThreads), 0, s, d_bitmap, nb, rows,
                       plan->causal, plan->d_counts);
  else
    hipLaunchKernelGGL(count_rows<1>, dim3(row_groups), dim3(kRowThreads), 0, s, d_bitmap, nb, rows,
                       plan->causal, plan->d_counts);
  const int nblk = (rows + kScanBlock - 1) / kScanBlock;
  auto scan = [&](RowDesc* out, int64_t* nnz_out) {
    if (nblk <= kSmallScanBlocks) {
      hipLaunchKernelGGL(scan_small, dim3(1), dim3(kScanBlock), 0, s, plan->d_counts, rows, out, nnz_out);
      return;
    }
    hipLaunchKernelGGL(scan_block_sums, dim3(unsigned(nblk)), dim3(kScanBlock), 0, s, plan->d_counts, rows,
                       plan->d_scan);
    hipLaunchKernelGGL(scan_sums, dim3(1), dim3(kScanBlock), 0, s, plan->d_scan, nblk);
    hipLaunchKernelGGL(scan_apply, dim3(unsigned(nblk)), dim3(kScanBlock), 0, s, plan->d_counts, rows,
                       plan->d_scan, nblk, out, nnz_out);
  };
  scan(d_rows, d_nnz);
  // The shorter last block of a seq_len the block does not divide: its tiles
  // are PARTIAL (-1: every block whole).
  const int tail = plan->prob.seq_len % plan->prob.block_size != 0 ? nb - 1 : -1;
  if (rows16)
    hipLaunchKernelGGL(fill_rows<16>, dim3(row_groups), dim3(kRowThreads), 0, s, d_bitmap, nb, rows,
                       plan->causal, tail, d_rows, d_entries);
  else
    hipLaunchKernelGGL(fill_rows<1>, dim3(row_groups), dim3(kRowThreads), 0, s, d_bitmap, nb, rows,
                       plan->causal, tail, d_rows, d_entries);
  if (plan->d_work_base) {
    // Longest row first within each (KV head, batch entry) run of the order.
    const int hkv = plan->prob.num_kv_heads, group = plan->prob.num_heads / hkv;
    const int64_t slots = int64_t(plan->work.size());
    hipLaunchKernelGGL(order_rows, dim3(unsigned(hkv)), dim3(kOrderThreads), 0, s, d_rows, nb, group,
                       plan->layout_heads > 1 ? 1 : 0, plan->d_order);
    hipLaunchKernelGGL(reorder_work, dim3(unsigned((slots + kOrderThreads - 1) / kOrderThreads)),
                       dim3(kOrderThreads), 0, s, plan->d_work_base, slots, nb, plan->prob.num_heads, group,
                       plan->d_order, const_cast<int32_t*>(plan->d_work));
  }
  // The same entries per k-block column, for the backward's dK/dV walk.
  auto* d_cols = const_cast<RowDesc*>(plan->d_cols);
  auto* d_entries_t = const_cast<int32_t*>(plan->d_entries_t);
  // 4-byte loads of 4 columns per lane when every row of the bitmap is 4-byte
  // aligned and the wider strips still give a workgroup per CU.
  const bool wide = nb % 4 == 0 && reinterpret_cast<uintptr_t>(d_bitmap) % 4 == 0 &&
                    int64_t(plan->layout_heads) * ((nb + 4 * kStrip - 1) / (4 * kStrip)) >= kWideMinStrips;
  const int vec = wide ? 4 : 1;
  const unsigned strips = unsigned(plan->layout_heads) * unsigned((nb + kStrip * vec - 1) / (kStrip * vec));
  if (vec == 4)
    hipLaunchKernelGGL(count_cols<4>, dim3(strips), dim3(kStripThreads), 0, s, d_bitmap, nb, plan->causal,
                       plan->d_counts);
  else
    hipLaunchKernelGGL(count_cols<1>, dim3(strips), dim3(kStripThreads), 0, s, d_bitmap, nb, plan->causal,
                       plan->d_counts);
  scan(d_cols, nullptr);
  // Entry bits kept in registers between the fill kernel's two passes when
  // each wave's chunk of rows fits them.
  const bool masks = (nb + kChunks - 1) / kChunks <= kMaskBatches * kRowBatch;
  if (vec == 4 && masks)
    hipLaunchKernelGGL((fill_cols<4, true>), dim3(strips), dim3(kStripThreads), 0, s, d_bitmap, nb, plan->causal,
                       tail, d_cols, d_entries_t);
  else if (vec == 4)
    hipLaunchKernelGGL((fill_cols<4, false>), dim3(strips), dim3(kStripThreads), 0, s, d_bitmap, nb, plan->causal,
                       tail, d_cols, d_entries_t);
  else if (masks)
    hipLaunchKernelGGL((fill_cols<1, true>), dim3(strips), dim3(kStripThreads), 0, s, d_bitmap, nb, plan->causal,
                       tail, d_cols, d_entries_t);
  else
    hipLaunchKernelGGL((fill_cols<1, false>), dim3(strips), dim3(kStripThreads), 0, s, d_bitmap, nb, plan->causal,
                       tail, d_cols, d_entries_t);
  if (plan->kv_extra_slots > 0) {
    // The dK/dV launch descriptors for the new walk lengths.
    const int hkv = plan->prob.num_kv_heads, group = plan->prob.num_heads / hkv;
    const int n = hkv * nb;
    const int64_t items = int64_t(plan->prob.batch) * n;
    hipLaunchKernelGGL(kv_walks, dim3(unsigned((n + kWriteThreads - 1) / kWriteThreads)), dim3(kWriteThreads), 0,
                       s, d_cols, nb, n, group, plan->layout_heads > 1 ? 1 : 0, plan->d_kv_walk);
    hipLaunchKernelGGL(kv_split_plan, dim3(1), dim3(kScanBlock), 0, s, n, plan->prob.batch,
                       (long long)plan->kv_extra_slots, (long long)plan->kv_partials, plan->d_kv_walk,
                       plan->d_kv_pre, plan->d_kv_head);
    const int64_t cover = items > plan->kv_extra_slots ? items : plan->kv_extra_slots;
    hipLaunchKernelGGL(kv_split_write, dim3(unsigned((cover + kWriteThreads - 1) / kWriteThreads)),
                       dim3(kWriteThreads), 0, s, plan->d_kv_walk, plan->d_kv_pre, plan->d_kv_head,
                       plan->d_kv_slot, n, items, plan->kv_extra_slots,
                       reinterpret_cast<int4*>(const_cast<int32_t*>(plan->d_work_kv)),
                       reinterpret_cast<int4*>(const_cast<int32_t*>(plan->d_kv_reduce)));
  }
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(BSA_ERR_DEVICE, "planner launch failed: %s", hipGetErrorString(err));
  return BSA_OK;
}

namespace bsa {
namespace {

// Copies layout head layout_head of a device CSR (descriptors d_desc, entries
// d_ent) to the host in the format of bsa_plan_csr.
bsa_status_t read_device_csr(bsa_plan_t plan, const RowDesc* d_desc, const int32_t* d_ent, int32_t layout_head,
                             int32_t* row_ptr, int32_t* col_idx, uint8_t* flags, int64_t capacity, int64_t* nnz) {
  if (!plan || !row_ptr || !nnz || (capacity > 0 && (!col_idx || !flags)))
    return fail(BSA_ERR_INVALID_ARGUMENT, "NULL argument to a device CSR read");
  if (!plan->dynamic) return fail(BSA_ERR_INVALID_ARGUMENT, "plan was not made by bsa_plan_dynamic");
  if (layout_head < 0 || layout_head >= plan->layout_heads)
    return fail(BSA_ERR_INVALID_ARGUMENT, "layout_head %d out of range [0, %d)", layout_head,
                plan->layout_heads);
  const int nb = plan->nb;
  std::vector<RowDesc> rd(nb);
  if (hipDeviceSynchronize() != hipSuccess ||
      (nb && hipMemcpy(rd.data(), d_desc + size_t(layout_head) * nb, nb * sizeof(RowDesc),
                       hipMemcpyDeviceToHost) != hipSuccess))
    return fail(BSA_ERR_DEVICE, "reading the device CSR failed: %s", hipGetErrorString(hipGetLastError()));
  const int64_t first = nb ? rd[0].start : 0;
  const int64_t count = nb ? int64_t(rd[nb - 1].start) + rd[nb - 1].count - first : 0;
  if (capacity < count)
    return fail(BSA_ERR_INVALID_ARGUMENT, "capacity %lld is below the head's %lld entries",
                (long long)capacity, (long long)count);
  std::vector<int32_t> en(static_cast<size_t>(count));
  if (count && hipMemcpy(en.data(), d_ent + first, size_t(count) * sizeof(int32_t), hipMemcpyDeviceToHost) !=
                   hipSuccess)
    return fail(BSA_ERR_DEVICE, "reading the device CSR failed: %s", hipGetErrorString(hipGetLastError()));
  row_ptr[0] = 0;
  for (int i = 0; i < nb; ++i) row_ptr[i + 1] = int32_t(rd[i].start - first + rd[i].count);
  for (int64_t e = 0; e < count; ++e) {
    col_idx[e] = en[size_t(e)] >> 1;
    flags[e] = uint8_t(en[size_t(e)] & 1);
  }
  *nnz = count;
  return BSA_OK;
}

}  // namespace
}  // namespace bsa

extern "C" bsa_status_t bsa_plan_read_csr(bsa_plan_t plan, int32_t layout_head, int32_t* row_ptr,
                                          int32_t* col_idx, uint8_t* flags, int64_t capacity, int64_t* nnz) {
  bsa::clear_error();
  return bsa::read_device_csr(plan, plan ? plan->d_rows : nullptr, plan ? plan->d_entries : nullptr, layout_head,
                              row_ptr, col_idx, flags, capacity, nnz);
}

extern "C" bsa_status_t bsa_plan_read_csr_transposed(bsa_plan_t plan, int32_t layout_head, int32_t* col_ptr,
                                                     int32_t* row_idx, uint8_t* flags, int64_t capacity,
                                                     int64_t* nnz) {
  bsa::clear_error();
  return bsa::read_device_csr(plan, plan ? plan->d_cols : nullptr, plan ? plan->d_entries_t : nullptr,
                              layout_head, col_ptr, row_idx, flags, capacity, nnz);
}

extern "C" bsa_status_t bsa_plan_read_work(bsa_plan_t plan, int32_t* work, int64_t capacity, int64_t* slots) {
  using namespace bsa;
  clear_error();
  if (!plan || !slots || (capacity > 0 && !work)) return fail(BSA_ERR_INVALID_ARGUMENT, "NULL argument to bsa_plan_read_work");
  if (!plan->info.on_device)
    return fail(BSA_ERR_INVALID_ARGUMENT, "plan was built by bsa_plan_host and has no device copy");
  const int64_t n = int64_t(plan->work.size());
  if (capacity < n)
    return fail(BSA_ERR_INVALID_ARGUMENT, "capacity %lld is below the plan's %lld launch slots", (long long)capacity,
                (long long)n);
  if (hipDeviceSynchronize() != hipSuccess ||
      (n && hipMemcpy(work, plan->d_work, size_t(n) * sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess))
    return fail(BSA_ERR_DEVICE, "reading the launch order failed: %s", hipGetErrorString(hipGetLastError()));
  *slots = n;
  return BSA_OK;
}

extern "C" bsa_status_t bsa_plan_read_work_kv(bsa_plan_t plan, int32_t* desc, int64_t capacity, int64_t* slots,
                                              int64_t* splits) {
  using namespace bsa;
  clear_error();
  if (!plan || !slots || !splits || (capacity > 0 && !desc))
    return fail(BSA_ERR_INVALID_ARGUMENT, "NULL argument to bsa_plan_read_work_kv");
  if (!plan->info.on_device)
    return fail(BSA_ERR_INVALID_ARGUMENT, "plan was built by bsa_plan_host and has no device copy");
  const int64_t n = int64_t(plan->kv_desc.size());
  if (capacity < n)
    return fail(BSA_ERR_INVALID_ARGUMENT, "capacity %lld is below the plan's %lld dK/dV slots",
                (long long)capacity, (long long)n);
  int32_t count = int32_t(plan->kv_reduce.size());
  if (hipDeviceSynchronize() != hipSuccess ||
      (n && hipMemcpy(desc, plan->d_work_kv, size_t(n) * 4 * sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess) ||
      (plan->dynamic && hipMemcpy(&count, plan->d_kv_count, sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess))
    return fail(BSA_ERR_DEVICE, "reading the dK/dV launch order failed: %s", hipGetErrorString(hipGetLastError()));
  *slots = n;
  *splits = count;
  return BSA_OK;
}
