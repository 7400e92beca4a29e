// Block-sparse flash attention backward kernels for gfx950 (CDNA4) and the
// bsa_backward launcher.
//
// The gradients of the forward (masked softmax attention over each query's
// allowed keys) given dO = dLoss/dO, the forward's O and its log-sum-exp:
//   p_qk  = exp(scale * <Q_q, K_k> - LSE_q)          (the forward's weights)
//   Delta_q = <dO_q, O_q>
//   ds_qk = p_qk * (<dO_q, V_k> - Delta_q)           (softmax Jacobian)
//   dQ_q  = scale * sum_k ds_qk K_k
//   dK_k  = scale * sum_q ds_qk Q_q,   dV_k = sum_q p_qk dO_q
// The pages discuss the backward only through its cost (training throughput
// of block-sparse vs dense attention in "Sparse Attention Kernels vs Full
// Attention Performance"); like the forward it visits only the active tiles
// and never stores a score matrix: every tile's scores are recomputed from Q
// and K and turned into weights with the saved LSE.
//
// Kernels:
//   bwd_dq_bf16_d128   one workgroup per (b, h, q-block): first Delta_q of
//                      its rows from O and dO (written for the dK/dV
//                      kernel), then a walk of the forward's CSR row: S^T
//                      and dP^T = V dO^T on MFMA, dS^T in registers,
//                      dQ^T += K^T dS^T.
//   bwd_dkdv_bf16_d128 one workgroup per (b, KV head, k-block), walking the
//                      transposed CSR over every query head of the GQA group:
//                      S and dP = dO V^T on MFMA, P and dS in registers,
//                      dV^T += dO^T P and dK^T += Q^T dS.
//   bwd_kv_reduce      sums the float32 partials of walks the plan split.
// Splitting dQ from dK/dV recomputes S and dP once more but needs no atomics,
// so results are deterministic.  Both tile kernels use the forward's MFMA
// layouts: a 32x32 accumulator tile gives each lane one column (a query in
// the dQ kernel, a key in the dK/dV kernel) and 16 rows, and accumulator
// registers 8c .. 8c+7 of tile t are exactly the 8 contraction elements that
// lane supplies for 16-element chunk 2t + c of the next product's B operand;
// the matching A operand comes from LDS through ds_read_b64_tr_b16.
// Both tile kernels walk their lists in 32-row steps whose rows (K and V in
// the dQ kernel; Q and dO in the dK/dV kernel, which keeps its block's V rows
// in LDS for the whole walk) are double-buffered in LDS and filled by direct
// HBM->LDS loads issued a step ahead, one barrier per step; two workgroups
// share a CU.  float32 kernels for fp32 inputs follow at the end.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "internal.h"
#include "queue.h"

namespace bsa {
namespace {

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const float* lse;
  const uint16_t* dout;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* delta;
  const RowDesc* rows;        // forward CSR rows [layout heads * nb]
  const int32_t* entries;     // (j << 1) | partial
  const int32_t* work;        // dQ launch order: (b * H + h) * nb + i
  const RowDesc* cols;        // transposed rows [layout heads * nb]
  const int32_t* entries_t;   // (i << 1) | partial
  const int32_t* kv_desc;     // dK/dV launch order: per slot {item (b * Hkv + hk) * nb + j,
                              // first and end entry of the group's walk, partial slot or -1}
  const int32_t* kv_reduce;   // per split column {item, first partial slot, count, 0}
  const int32_t* kv_reduce_count;   // device count of kv_reduce entries (dynamic plans), else NULL
  float* kv_scratch;          // float32 partials [slot][dK, dV][128 keys][128]
  int64_t N;
  int32_t H, Hkv, group, nb, per_head_layout;
  float scale, sl2;           // sl2 = scale * log2(e)
  int32_t N32;                // N as int32 (N <= 2^30)
  int32_t causal, token_rule, gk32, gq32;
  // Window and causal parts of the token predicate as one range of q - k:
  // allowed iff (uint32)(q - k - mlo) <= mspan.
  int32_t mlo;
  uint32_t mspan;
  // Variable-length batch (bsa_backward_varlen): device int32 [batch], entry b
  // uses its first seq_lens[b] positions; nullptr otherwise.
  const int32_t* seq_lens;
  // Launches of the bf16 tile kernels: slots run by one workgroup each, then
  // queue workgroups (queue.h); lq_dq over `work`, lq_kv over kv_desc.
  LaunchQueue lq_dq, lq_kv;
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kD = 128;
constexpr int kB = 128;           // layout block = tile height and width
constexpr int kThreads = 256;     // 4 waves of 64
constexpr int kTileBytes = kB * kD * 2;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;

// Token predicate inside a PARTIAL tile: the window/causal range of q - k, or
// a global key / global query row (still under the causal cut).  With
// token_rule == 0 the range is the causal cut alone.
// Positions at or beyond the sequence's length n do not exist (every tile of
// its last block is treated as PARTIAL).
__device__ __forceinline__ bool pair_ok(const BwdParams& p, int q, int k, int n) {
  const bool in_range = uint32_t(q - k) - uint32_t(p.mlo) <= p.mspan;
  const bool glob = p.token_rule && (k < p.gk32 || q < p.gq32) && (!p.causal || k <= q);
  return (in_range || glob) && q < n && k < n;
}

// Length of batch entry b's sequence: seq_lens[b] clamped to [0, N] in a
// variable-length batch, else N.
__device__ __forceinline__ int entry_length(const BwdParams& p, int b) {
  int n = p.N32;
  if (p.seq_lens) {
    const int x = p.seq_lens[b];
    n = x < 0 ? 0 : (x > n ? n : x);
  }
  return n;
}

// LDS tile layout for rows read both row-wise and transposed: row r (256
// bytes) with 16-byte chunk c at chunk c ^ tile_swz(r), tile_swz(r) =
// 4 (r & 3) + ((r >> 2) & 3).  Row reads of 16 bytes and the transposing
// 8-byte reads both stay inside one chunk, so either kind sees the logical
// layout; 16 consecutive rows read at one chunk land in 16 different chunks,
// and the 4 rows x 2 adjacent chunks of a transposing read in 8, so neither
// read has bank conflicts.
__device__ __forceinline__ int tile_swz(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }
__device__ __forceinline__ uint32_t tile_off(int r, int c) { return r * 256 + 16 * (c ^ tile_swz(r)); }

// LDS layout of K/V rows that are only read row-wise (B operands): chunk c of
// row r at c ^ (r & 15), which keeps 16-byte reads of 32 rows x 2 chunks free
// of bank conflicts.
__device__ __forceinline__ uint32_t rows_off(int r, int c) { return r * 256 + 16 * (c ^ (r & 15)); }

// Copy kRows contiguous rows of 128 bf16 (256 bytes) from global memory into
// LDS with either layout: coalesced 16-byte loads, kRows / 16 per thread,
// issued in groups of at most four before their stores.  Thread t moves
// chunk t % 16 of rows t / 16 + 16 u, so its global and LDS offsets are one
// base plus u * 4096 (the swizzles depend on the row only through r & 15).
// The thread index passes through an empty asm so its address arithmetic
// is redone per call instead of being hoisted out of the caller's loops and
// held in registers.
// Rows at or beyond valid_rows (the end of a ragged sequence) are loaded from
// row valid_rows - 1.
template <int kRows, bool kRowsOnly>
__device__ __forceinline__ void stage(lds_u8* dst, const unsigned char* __restrict__ src, int tid,
                                      int valid_rows = kRows) {
  constexpr int kPer = kRows / 16;
  constexpr int kGroup = kPer < 4 ? kPer : 4;
  int t = tid;
  __asm__ volatile("" : "+v"(t));
  const int r = t >> 4, c = t & 15;
  const u32x4* g = reinterpret_cast<const u32x4*>(src + c * 16);
  lds_u8* const l = dst + (kRowsOnly ? rows_off(r, c) : tile_off(r, c));
#pragma unroll
  for (int part = 0; part < kPer / kGroup; ++part) {
    u32x4 v[kGroup];
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      const int row = r + 16 * (part * kGroup + u);
      v[u] = g[(row < valid_rows ? row : valid_rows - 1) * 16];
    }
#pragma unroll
    for (int u = 0; u < kGroup; ++u)
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(l + (part * kGroup + u) * 4096) = v[u];
  }
}

// A operand (32 rows x 16 contraction elements) by a row read: row
// row0 + (lane & 31), elements 16 cc + 8 (lane >> 5) .. +7.
__device__ __forceinline__ bf16x8 read_rows(const lds_u8* base, uint32_t off) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(base + off);
}

// A operand by two transposing reads: lane l receives, for column
// d = 32 dt + (l & 31), the 8 rows 16 kc + 4 (l >> 5) + {0..3, 8..11} (the
// row order of a 16-element chunk of the accumulator layout).  off_lo and
// off_hi address rows 4 (l >> 5) + r4 and that + 8 (see cols_base); 16 kc
// rows add 16 kc * 256 bytes to both.
__device__ __forceinline__ bf16x8 read_cols(const lds_u8* base, uint32_t off_lo, uint32_t off_hi, int kc) {
  const bf16x4 lo = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) s16x4*>(const_cast<lds_u8*>(base) + off_lo + (16 * kc) * 256)));
  const bf16x4 hi = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) s16x4*>(const_cast<lds_u8*>(base) + off_hi + (16 * kc) * 256)));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// Sum of x over lanes l and l ^ 32 (v_permlane32_swap: one result holds the
// lane's own value, the other its partner's).
__device__ __forceinline__ float sum_with_partner(float x) {
  const uint32_t b = __float_as_uint(x);
  const auto sw = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// Store a wave's 32-column x 128-row transposed accumulator (acc[dt] row
// 32 dt + 8 (r / 4) + 4 hf + r % 4 of this lane's column, column r32) as 32
// bf16 rows of 128 values at dst0 (row r32 at dst0 + 128 r32), times mul;
// only the first nvalid rows are written.  The block is staged in 8 KB of
// LDS that no wave reads any more (16-byte chunk c of row r at c ^ (r & 15):
// no bank conflicts either way), then written as whole 256-byte rows, 16
// bytes per lane and four rows per store, instead of 16-byte pieces of 32
// rows per store.  The wave reads back only what it wrote.
__device__ __forceinline__ void store_block(uint16_t* dst0, const f32x16 (&acc)[4], float mul, int r32, int hf,
                                            int lane, lds_u8* stage, int nvalid) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 pk;
      pk[0] = uint32_t(bf16_bits(acc[dt][4 * g + 0] * mul)) | (uint32_t(bf16_bits(acc[dt][4 * g + 1] * mul)) << 16);
      pk[1] = uint32_t(bf16_bits(acc[dt][4 * g + 2] * mul)) | (uint32_t(bf16_bits(acc[dt][4 * g + 3] * mul)) << 16);
      *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(
          stage + r32 * 256 + 16 * ((4 * dt + g) ^ (r32 & 15)) + 8 * hf) = pk;
    }
  __asm__ volatile("" ::: "memory");
  const int sr = lane >> 4, sc = lane & 15;      // row within a group of 4, 16-byte chunk
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int r = 4 * s + sr;
    const u32x4 val = *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(stage + r * 256 + 16 * (sc ^ (r & 15)));
    if (r < nvalid) *reinterpret_cast<u32x4*>(dst0 + int64_t(r) * kD + 8 * sc) = val;
  }
  __asm__ volatile("" ::: "memory");
}

// Wait until at most N of this wave's vector-memory operations are pending,
// then a workgroup barrier.  The "memory" clobber keeps LDS accesses on their
// side of the barrier.
#define BSA_WAIT_BARRIER(N) \
  __asm__ volatile("s_waitcnt vmcnt(" #N ")\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")

// HBM->LDS load of 16 bytes per lane (1 KB per wave) from sbase + voff into
// LDS at lds_addr + 16 * lane, in inline assembly so that the compiler adds
// no waits of its own for it; each use is followed by BSA_WAIT_BARRIER before
// the data is read.  M0 is reserved for the compiler, which therefore does
// not honour it as a clobber; the compiled kernel has no other use of M0
// (checked on its assembly by a CPU test).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  __asm__ volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                   :: "v"(voff), "s"(sbase), "s"(lds_addr) : "memory", "m0");
}
#pragma clang diagnostic pop

constexpr int kStepRows = 32;
constexpr int kStepBytes = kStepRows * kD * 2;   // 8 KB

// Per-lane LDS operand offsets of a 32-row step buffer as one base XOR-ed
// with a constant per operand (the layouts' swizzles are XORs on the chunk
// bits; a CPU test checks these identities for every lane):
//   row reads, tile layout  tile_off(r32, 2cc + hf)           = tile_rows_base ^ 32 cc
//   row reads, row layout   rows_off(32w + r32, 2cc + hf)     = rows_rows_base(w) ^ 32 cc
//   transposed reads: in 16-lane group g, lane 4 r4 + c4 addresses row
//   4 hf + r4 + 8 s (s = 0 for the low half, 1 for the high half) and columns
//   32 dt + 16 (g & 1) + 4 c4 .. +3 in the tile layout    = cols_base(s) ^ 64 dt
__device__ __forceinline__ uint32_t tile_rows_base(int lane) {
  const int r32 = lane & 31, hf = lane >> 5, f = tile_swz(r32);
  return r32 * 256 + 16 * (hf ^ (f & 1)) + 16 * (f & 14);
}
__device__ __forceinline__ uint32_t rows_rows_base(int lane, int w) {
  const int r32 = lane & 31, hf = lane >> 5;
  return (32 * w + r32) * 256 + 16 * (hf ^ (r32 & 1)) + 16 * (r32 & 14);
}
__device__ __forceinline__ uint32_t cols_base(int lane, int s) {
  const int hf = lane >> 5, r4 = (lane & 15) >> 2, c4 = lane & 3, gp = (lane >> 4) & 1;
  return (4 * hf + r4 + 8 * s) * 256 + 16 * ((2 * gp + (c4 >> 1)) ^ (hf + 2 * s)) + 8 * (c4 & 1) + 64 * r4;
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (b, h, q-block); wave w owns query rows 32w .. +31
// and walks the forward's CSR row in steps of 32 keys.  Q^T and dO^T stay in
// registers as B operands, the row's LSE and Delta in one register each.
// Delta_q = <dO_q, O_q> is formed first, from O loaded in dO's register
// layout (each lane holds half of its row, lanes l and l ^ 32 the two
// halves), and written to p.delta for the dK/dV kernel, which runs after
// this one on the same stream; every launch slot of the plan is one q-block,
// so every row is written (0 for rows at or beyond the entry's length).  K
// rows (read row-wise for S^T and transposed for dQ^T) and V rows (row-wise
// for dP^T) of a step are double-buffered and filled by direct HBM->LDS
// loads issued a step ahead, interleaved with the S^T/dP^T MFMAs; one
// barrier per step, 32 KB of LDS.
// ---------------------------------------------------------------------------
// kRagged: the sequence ends inside its last block, or the batch entries
// have lengths of their own (seq_lens).  With Nb the entry's length, rows at
// or beyond Nb load row Nb - 1 and are masked; the walk stops at the entry's
// last block; rows in [Nb, N) get dQ = 0 and rows at or beyond N are not
// written.
template <bool kRagged>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_bf16_d128(BwdParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char K0[kStepBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char K1[kStepBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char V0[kStepBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char V1[kStepBytes];
  lds_u8* const Kb[2] = {(lds_u8*)K0, (lds_u8*)K1};
  lds_u8* const Vb[2] = {(lds_u8*)V0, (lds_u8*)V1};
  const uint32_t Ka[2] = {uint32_t(reinterpret_cast<uintptr_t>((lds_u8*)K0)),
                          uint32_t(reinterpret_cast<uintptr_t>((lds_u8*)K1))};
  const uint32_t Va[2] = {uint32_t(reinterpret_cast<uintptr_t>((lds_u8*)V0)),
                          uint32_t(reinterpret_cast<uintptr_t>((lds_u8*)V1))};

  __shared__ int s_slot;
  int done;
  const int slot = queue_slot(p.lq_dq, &s_slot, done);
  const int item = slot >= 0 ? p.work[slot] : -1;
  if (item < 0) {
    queue_release(p.lq_dq, done);
    return;
  }
  const int i = item % p.nb;
  const int bh = item / p.nb;
  const int h = bh % p.H, b = bh / p.H;
  const int hk = h / p.group;
  const RowDesc row = p.rows[(p.per_head_layout ? h : 0) * p.nb + i];
  const int Nb = kRagged ? entry_length(p, b) : p.N32;
  const int nbb = (Nb + kB - 1) / kB;
  // The CSR row lists ascending key blocks: the walk is its prefix below the
  // entry's last block (none for a q-block beyond it).
  int ne = row.count;
  if (kRagged) {
    ne = i >= nbb ? 0 : row.count;
    while (ne > 0 && (p.entries[row.start + ne - 1] >> 1) >= nbb) --ne;
  }

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, r32 = lane & 31, hf = lane >> 5;
  const int qg = i * kB + wave * 32 + r32;
  const int64_t qrow = (int64_t(b) * p.H + h) * p.N + qg;
  const int64_t qrow_ld = kRagged && qg >= Nb ? qrow - qg + (Nb > 0 ? Nb - 1 : 0) : qrow;   // row to load from

  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};

  // dO^T as a B operand: lane (row r32, half hf) holds d = 16c + 8hf .. +7;
  // O in the same layout gives Delta (float32 products of the bf16 values).
  bf16x8 df[8];
  float dlt;
  {
    bf16x8 of[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      df[c] = *reinterpret_cast<const bf16x8*>(p.dout + qrow_ld * kD + c * 16 + hf * 8);
      of[c] = *reinterpret_cast<const bf16x8*>(p.o + qrow_ld * kD + c * 16 + hf * 8);
    }
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        part[e & 3] = fmaf(static_cast<float>(of[c][e]), static_cast<float>(df[c][e]), part[e & 3]);
    dlt = sum_with_partner((part[0] + part[1]) + (part[2] + part[3]));
    if (hf == 0 && (!kRagged || qg < p.N32)) p.delta[qrow] = kRagged && qg >= Nb ? 0.f : dlt;
  }

  if (ne > 0) {
    // Q^T as a B operand, in dO's layout.
    bf16x8 qf[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(p.q + qrow_ld * kD + c * 16 + hf * 8);
    const float lse = p.lse[qrow_ld];
    // An empty row (LSE = -inf) has every score masked in every tile it meets.
    const float lse2 = lse == -INFINITY ? 0.f : lse * kLog2e;
    // Complete these loads before the first HBM->LDS load, so the pending
    // counts the barriers wait on only see those.
    __asm__ volatile("s_waitcnt vmcnt(0)" ::"v"(qf[0]), "v"(qf[1]), "v"(qf[2]), "v"(qf[3]), "v"(qf[4]),
                     "v"(qf[5]), "v"(qf[6]), "v"(qf[7]), "v"(df[0]), "v"(df[1]), "v"(df[2]), "v"(df[3]),
                     "v"(df[4]), "v"(df[5]), "v"(df[6]), "v"(df[7]), "v"(lse2), "v"(dlt) : "memory");

    const unsigned char* Kg = reinterpret_cast<const unsigned char*>(p.k + (int64_t(b) * p.Hkv + hk) * p.N * kD);
    const unsigned char* Vg = reinterpret_cast<const unsigned char*>(p.v + (int64_t(b) * p.Hkv + hk) * p.N * kD);
    // HBM->LDS loads of one step: wave w fills rows 8w .. 8w+7 of the K and V
    // buffers, 4 rows (1 KB) per instruction; lane L writes chunk L % 16 of
    // row R = 8w + 4u + L / 16 and reads the logical chunk the layout places
    // there (K: chunk ^ tile_swz(R); V: chunk ^ (R & 15)).
    const int l4 = lane >> 4, lc = lane & 15;
    auto dma_step = [&](int j, int st, int bf, int u) {
      const int R = wave * 8 + 4 * (u & 1) + l4;
      const uint32_t lds_off = (wave * 8 + 4 * (u & 1)) * 256;
      const uint32_t chunk = 16 * (u < 2 ? (lc ^ tile_swz(R)) : (lc ^ (R & 15)));
      // Source row relative to the key block's first row (below Nb); in the
      // entry's ragged last block rows at or beyond Nb read row Nb - 1.
      int rel = st * kStepRows + R;
      if (kRagged && j == nbb - 1) rel = rel < Nb - j * kB ? rel : Nb - j * kB - 1;
      const int64_t tile0 = int64_t(j) * kB;
      if (u < 2)
        dma16(Kg + tile0 * 256, rel * 256 + chunk, Ka[bf] + lds_off);
      else
        dma16(Vg + tile0 * 256, rel * 256 + chunk, Va[bf] + lds_off);
    };
    const uint32_t bq0 = tile_rows_base(lane), bv0 = rows_rows_base(lane, 0);
    const uint32_t bcl0 = cols_base(lane, 0), bch0 = cols_base(lane, 1);

    int e = 0;
    // Entries are wave-uniform; readfirstlane keeps the load addresses built
    // from them in scalar registers, as the HBM->LDS loads require.
    int ent = __builtin_amdgcn_readfirstlane(p.entries[row.start]);
#pragma unroll
    for (int u = 0; u < 4; ++u) dma_step(ent >> 1, 0, 0, u);
    while (true) {
      const int j = ent >> 1;
      // Tiles touching a short last block of the entry are masked whatever
      // the plan's flag.
      const bool partial = (ent & 1) || (kRagged && (Nb % kB) != 0 && (j == nbb - 1 || i == nbb - 1));
      const bool have_next = e + 1 < ne;
      const int ent_n = have_next ? __builtin_amdgcn_readfirstlane(p.entries[row.start + e + 1]) : 0;
#pragma unroll
      for (int st = 0; st < 4; ++st) {                 // keys 32st .. 32st+31 of key block j
        const int bf = st & 1;
        lds_u8* const Ks = Kb[bf];
        lds_u8* const Vs = Vb[bf];
        BSA_WAIT_BARRIER(0);                           // this step's rows landed; the other buffer is free
        uint32_t bq = bq0, bv = bv0, bcl = bcl0, bch = bch0;
        __asm__ volatile("" : "+v"(bq), "+v"(bv), "+v"(bcl), "+v"(bch));
        const bool pf = st < 3 || have_next;
        const int tj = st < 3 ? j : (ent_n >> 1);
        // S^T and dP^T: 16 MFMAs alternating between the two accumulators,
        // each A operand (a K or V row read) issued two MFMAs ahead, the next
        // step's loads one every other MFMA.
        f32x16 sc = f32x16{}, dp = f32x16{};
        auto lda = [&](int m) {
          return (m & 1) ? read_rows(Vs, bv ^ (32 * (m >> 1))) : read_rows(Ks, bq ^ (32 * (m >> 1)));
        };
        bf16x8 ab[4];
        ab[0] = lda(0);
        ab[1] = lda(1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < 16; ++m) {
          if (m + 2 < 16) ab[(m + 2) & 3] = lda(m + 2);
          if (pf && (m & 1) == 0 && m < 8) dma_step(tj, (st + 1) & 3, bf ^ 1, m >> 1);
          __builtin_amdgcn_sched_barrier(0);
          if (m & 1)
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab[m & 3], df[m >> 1], dp, 0, 0, 0);
          else
            sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab[m & 3], qf[m >> 1], sc, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        // Register r holds key 32st + 8 (r / 4) + 4 hf + r % 4 of block j, for
        // query qg.  The token mask runs only in PARTIAL tiles (the empty asm
        // keeps the branch a real, wave-uniform one).
        if (partial) {
          __asm__ volatile("");
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = j * kB + st * kStepRows + 8 * (r >> 2) + 4 * hf + (r & 3);
            sc[r] = pair_ok(p, qg, kk, Nb) ? sc[r] : -INFINITY;
          }
        }
        bf16x8 ds[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = __builtin_amdgcn_exp2f(fmaf(sc[r], p.sl2, -lse2));
          ds[r >> 3][r & 7] = static_cast<__bf16>(pr * (dp[r] - dlt));
        }
        // dQ^T += K^T dS^T: key chunk m >> 2 of the step, d-tile m & 3.
        auto ldc = [&](int m) { return read_cols(Ks, bcl ^ (64 * (m & 3)), bch ^ (64 * (m & 3)), m >> 2); };
        bf16x8 cb[4];
        cb[0] = ldc(0);
        cb[1] = ldc(1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          if (m + 2 < 8) cb[(m + 2) & 3] = ldc(m + 2);
          __builtin_amdgcn_sched_barrier(0);
          acc[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cb[m & 3], ds[m >> 2], acc[m & 3], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (!have_next) break;
      ++e;
      ent = ent_n;
    }
  }
  queue_release(p.lq_dq, done);
  // Every wave is past its last LDS read: the wave's 8 KB buffer stages dQ.
  BSA_WAIT_BARRIER(0);
  {
    const int row0 = i * kB + wave * 32;
    const int nvalid = kRagged ? (p.N32 - row0 < 0 ? 0 : (p.N32 - row0 > 32 ? 32 : p.N32 - row0)) : 32;
    lds_u8* const stage = wave == 0 ? Kb[0] : wave == 1 ? Kb[1] : wave == 2 ? Vb[0] : Vb[1];
    store_block(p.dq + (qrow - r32) * kD, acc, p.scale, r32, hf, lane, stage, nvalid);
  }
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (b, KV head, k-block); wave w owns keys
// 32w .. +31 and walks, for every query head of the group, the q-blocks of
// the transposed CSR in steps of 32 queries.  K^T stays in registers as a B
// operand; the block's V rows sit in LDS for the whole walk and give the B
// operand of dP by row reads.  Q and dO rows of a step (8 KB each) are
// double-buffered and filled by direct HBM->LDS loads issued a step ahead,
// interleaved with the S/dP MFMAs; one barrier per step.  The step's LSE and
// Delta are loaded a step ahead too (lane l < 32: LSE of query l, else Delta
// of query l - 32) and parked in a wave-private LDS row.  64 KB + 1 KB of LDS
// and at most 256 registers: two workgroups share a CU.
// ---------------------------------------------------------------------------
template <bool kRagged>
__global__ __launch_bounds__(kThreads, 2) void bwd_dkdv_bf16_d128(BwdParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char Vsh[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char Q0[kStepBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char Q1[kStepBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char dO0[kStepBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char dO1[kStepBytes];
  __shared__ __attribute__((aligned(16))) float priv[4 * 64];
  lds_u8* const Vs = (lds_u8*)Vsh;
  lds_u8* const Qb[2] = {(lds_u8*)Q0, (lds_u8*)Q1};
  lds_u8* const dOb[2] = {(lds_u8*)dO0, (lds_u8*)dO1};
  const uint32_t Qa[2] = {uint32_t(reinterpret_cast<uintptr_t>((lds_u8*)Q0)),
                          uint32_t(reinterpret_cast<uintptr_t>((lds_u8*)Q1))};
  const uint32_t dOa[2] = {uint32_t(reinterpret_cast<uintptr_t>((lds_u8*)dO0)),
                           uint32_t(reinterpret_cast<uintptr_t>((lds_u8*)dO1))};

  __shared__ int s_slot;
  int done;
  const int slot = queue_slot(p.lq_kv, &s_slot, done);
  const int item = slot >= 0 ? p.kv_desc[4 * slot] : -1;
  if (item < 0) {
    queue_release(p.lq_kv, done);
    return;
  }
  const int walk_begin = p.kv_desc[4 * slot + 1];
  const int walk_end = p.kv_desc[4 * slot + 2];
  const int partial_slot = p.kv_desc[4 * slot + 3];
  const int j = item % p.nb;
  const int bk = item / p.nb;
  const int hk = bk % p.Hkv, b = bk / p.Hkv;
  const int Nb = kRagged ? entry_length(p, b) : p.N32;
  const int nbb = (Nb + kB - 1) / kB;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, r32 = lane & 31, hf = lane >> 5;
  const int kg = j * kB + wave * 32 + r32;
  const int64_t kvbase = (int64_t(b) * p.Hkv + hk) * p.N;
  const int64_t krow = kvbase + kg;

  f32x16 dk[4], dv[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    dk[dt] = f32x16{};
    dv[dt] = f32x16{};
  }

  // Cursor over this slot's part [walk_begin, walk_end) of the walk: the
  // group's transposed lists one after another, as (query head of the group,
  // entry of its list); every value is wave-uniform.  The lists are ascending
  // in q-block, so under kRagged the first q-block beyond the entry's last
  // skips the rest of its list; a k-block beyond it has no walk.
  struct Entry {
    int h, i, partial;
  };
  int cg = 0, ce = walk_begin, left = walk_end - walk_begin;
  if (kRagged && j >= nbb) left = 0;
  RowDesc ccol = p.cols[(p.per_head_layout ? hk * p.group : 0) * p.nb + j];
  auto next_entry = [&](Entry& out) -> bool {
    int ent;
    while (true) {
      if (left <= 0) return false;
      while (ce >= ccol.count) {
        ce -= ccol.count;
        if (++cg >= p.group) return false;
        ccol = p.cols[(p.per_head_layout ? hk * p.group + cg : 0) * p.nb + j];
      }
      ent = __builtin_amdgcn_readfirstlane(p.entries_t[ccol.start + ce]);
      if (!kRagged || (ent >> 1) < nbb) break;
      left -= ccol.count - ce;
      ce = ccol.count;
    }
    ++ce;
    --left;
    out.h = hk * p.group + cg;
    out.i = ent >> 1;
    out.partial = ent & 1;
    return true;
  };

  Entry cur;
  bool have = next_entry(cur);
  if (have) {
    // K^T as a B operand: lane (key r32, half hf) holds d = 16c + 8hf .. +7.
    bf16x8 kf[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
      kf[c] = *reinterpret_cast<const bf16x8*>(p.k + (kRagged && kg >= Nb ? kvbase + Nb - 1 : krow) * kD +
                                               c * 16 + hf * 8);
    // V rows of this k-block; the first step's barrier publishes them.
    stage<kB, true>(Vs, reinterpret_cast<const unsigned char*>(p.v + (kvbase + int64_t(j) * kB) * kD), tid,
                    kRagged ? (Nb - j * kB < kB ? Nb - j * kB : kB) : kB);
    // Complete these loads before the first HBM->LDS load, so the pending
    // counts the barriers wait on only see those.
    __asm__ volatile("s_waitcnt vmcnt(0)" ::"v"(kf[0]), "v"(kf[1]), "v"(kf[2]), "v"(kf[3]), "v"(kf[4]),
                     "v"(kf[5]), "v"(kf[6]), "v"(kf[7]) : "memory");

    // HBM->LDS loads of one step: wave w fills rows 8w .. 8w+7 of the Q and
    // dO buffers, 4 rows (1 KB) per instruction; lane L writes chunk L % 16
    // of row R = 8w + 4u + L / 16 and reads the logical chunk the tile layout
    // places there (chunk ^ tile_swz(R)).
    auto dma_step = [&](const Entry& en, int st, int bf, int u) {
      // Source row relative to the q-block's first row (below Nb); in the
      // entry's ragged last block rows at or beyond Nb read row Nb - 1.
      const int64_t tile0 = (int64_t(b) * p.H + en.h) * p.N + int64_t(en.i) * kB;
      const int R = wave * 8 + 4 * (u & 1) + (lane >> 4);
      int rel = st * kStepRows + R;
      if (kRagged && en.i == nbb - 1) rel = rel < Nb - en.i * kB ? rel : Nb - en.i * kB - 1;
      const uint32_t voff = rel * 256 + 16 * ((lane & 15) ^ tile_swz(R));
      const uint32_t lds_off = (wave * 8 + 4 * (u & 1)) * 256;
      if (u < 2)
        dma16(p.q + tile0 * kD, voff, Qa[bf] + lds_off);
      else
        dma16(p.dout + tile0 * kD, voff, dOa[bf] + lds_off);
    };
    auto load_x = [&](const Entry& en, int st) {
      int qi = en.i * kB + st * kStepRows + (lane & 31);
      if (kRagged) qi = qi < Nb ? qi : Nb - 1;
      const int64_t r = (int64_t(b) * p.H + en.h) * p.N + qi;
      return lane < 32 ? p.lse[r] : p.delta[r];
    };
    // Operand offset bases (Q/dO row reads, V row reads, transposed reads);
    // they pass through an empty asm at every step, so the compiler
    // re-derives the operand addresses inside the step instead of holding
    // all of them in registers.
    const uint32_t bq0 = tile_rows_base(lane), bv0 = rows_rows_base(lane, wave);
    const uint32_t bcl0 = cols_base(lane, 0), bch0 = cols_base(lane, 1);
    float* const my = priv + wave * 64;

    float x = load_x(cur, 0);
#pragma unroll
    for (int u = 0; u < 4; ++u) dma_step(cur, 0, 0, u);

    while (have) {
      Entry nxt;
      const bool have_next = next_entry(nxt);
#pragma unroll
      for (int st = 0; st < 4; ++st) {                 // queries 32st .. 32st+31 of q-block cur.i
        const int bf = st & 1;
        lds_u8* const Qs = Qb[bf];
        lds_u8* const dOs = dOb[bf];
        BSA_WAIT_BARRIER(0);                           // this step's rows landed; the other buffer is free
        // This step's LSE (lanes < 32, as LSE * log2 e, 0 for an empty row:
        // every score of such a row is masked in this tile) and Delta.
        my[lane] = lane < 32 ? (x == -INFINITY ? 0.f : x * kLog2e) : x;
        uint32_t bq = bq0, bv = bv0, bcl = bcl0, bch = bch0;
        __asm__ volatile("" : "+v"(bq), "+v"(bv), "+v"(bcl), "+v"(bch));
        const bool pf = st < 3 || have_next;
        const Entry& te = st < 3 ? cur : nxt;
        if (pf) x = load_x(te, (st + 1) & 3);
        // S and dP: 16 MFMAs alternating between the two accumulators; the
        // operands of MFMA m (a Q or dO row read, and for dP a V row read)
        // are issued two MFMAs ahead, the next step's loads one every other
        // MFMA.
        f32x16 s = f32x16{}, dp = f32x16{};
        auto lda = [&](int m) { return read_rows((m & 1) ? dOs : Qs, bq ^ (32 * (m >> 1))); };
        auto ldb = [&](int m) { return read_rows(Vs, bv ^ (32 * (m >> 1))); };
        bf16x8 ab[4], bb[4];
        ab[0] = lda(0);
        ab[1] = lda(1);
        bb[1] = ldb(1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < 16; ++m) {
          if (m + 2 < 16) {
            ab[(m + 2) & 3] = lda(m + 2);
            if ((m + 2) & 1) bb[(m + 2) & 3] = ldb(m + 2);
          }
          if (pf && (m & 1) == 0 && m < 8) dma_step(te, (st + 1) & 3, bf ^ 1, m >> 1);
          __builtin_amdgcn_sched_barrier(0);
          if (m & 1)
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab[m & 3], bb[m & 3], dp, 0, 0, 0);
          else
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab[m & 3], kf[m >> 1], s, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        // Register r holds query 32st + 8 (r / 4) + 4 hf + r % 4 of q-block
        // cur.i, for key kg.  The token mask runs only in PARTIAL tiles.
        const int qbase = cur.i * kB + st * kStepRows;
        if (cur.partial || (kRagged && (Nb % kB) != 0 && (cur.i == nbb - 1 || j == nbb - 1))) {
          __asm__ volatile("");
#pragma unroll
          for (int r = 0; r < 16; ++r)
            s[r] = pair_ok(p, qbase + 8 * (r >> 2) + 4 * hf + (r & 3), kg, Nb) ? s[r] : -INFINITY;
        }
        bf16x8 pb[2], db[2];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int q0 = 8 * g4 + 4 * hf;
          const f32x4 L = *reinterpret_cast<const f32x4*>(my + q0);
          const f32x4 Dl = *reinterpret_cast<const f32x4*>(my + 32 + q0);
#pragma unroll
          for (int r3 = 0; r3 < 4; ++r3) {
            const int r = 4 * g4 + r3;
            const float pr = __builtin_amdgcn_exp2f(fmaf(s[r], p.sl2, -L[r3]));
            pb[r >> 3][r & 7] = static_cast<__bf16>(pr);
            db[r >> 3][r & 7] = static_cast<__bf16>(pr * (dp[r] - Dl[r3]));
          }
        }
        // dV^T += dO^T P and dK^T += Q^T dS: 16 MFMAs; operand m is query
        // chunk m >> 3 of the step, d-tile (m >> 1) & 3, dV for even m, dK
        // for odd m.
        auto ldc = [&](int m) {
          const int dt = (m >> 1) & 3;
          return read_cols((m & 1) ? Qs : dOs, bcl ^ (64 * dt), bch ^ (64 * dt), m >> 3);
        };
        bf16x8 cb[4];
        cb[0] = ldc(0);
        cb[1] = ldc(1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < 16; ++m) {
          if (m + 2 < 16) cb[(m + 2) & 3] = ldc(m + 2);
          __builtin_amdgcn_sched_barrier(0);
          const int dt = (m >> 1) & 3;
          if (m & 1)
            dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cb[m & 3], db[m >> 3], dk[dt], 0, 0, 0);
          else
            dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cb[m & 3], pb[m >> 3], dv[dt], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      cur = nxt;
      have = have_next;
    }
  }
  queue_release(p.lq_kv, done);
  if (partial_slot < 0) {
    // Every wave is past its last LDS read: 8 KB of the V block per wave
    // stages dK, then dV.
    BSA_WAIT_BARRIER(0);
    const int row0 = j * kB + wave * 32;
    const int nvalid = kRagged ? (p.N32 - row0 < 0 ? 0 : (p.N32 - row0 > 32 ? 32 : p.N32 - row0)) : 32;
    lds_u8* const stage = Vs + wave * (32 * 256);
    store_block(p.dk + (krow - r32) * kD, dk, p.scale, r32, hf, lane, stage, nvalid);
    store_block(p.dv + (krow - r32) * kD, dv, 1.f, r32, hf, lane, stage, nvalid);
  } else {
    // One chunk of a split column: float32 partial sums, unscaled.
    float* const part = p.kv_scratch + int64_t(partial_slot) * 2 * kB * kD + (wave * 32 + r32) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = dt * 32 + 8 * g4 + 4 * hf;
        *reinterpret_cast<f32x4*>(part + d) =
            f32x4{dk[dt][4 * g4], dk[dt][4 * g4 + 1], dk[dt][4 * g4 + 2], dk[dt][4 * g4 + 3]};
        *reinterpret_cast<f32x4*>(part + kB * kD + d) =
            f32x4{dv[dt][4 * g4], dv[dt][4 * g4 + 1], dv[dt][4 * g4 + 2], dv[dt][4 * g4 + 3]};
      }
  }
}

// ---------------------------------------------------------------------------
// Split columns: dK = scale * sum of the chunks' partials, dV = their sum, in
// chunk order (deterministic); kReduceParts workgroups per split column
// (blockIdx.y), 4 values per thread.  A dynamic plan's list length is known
// only on the device: its workgroups stride over the list by gridDim.x.
// ---------------------------------------------------------------------------
constexpr int kReduceParts = 2 * kB * kD / 4 / kThreads;   // 32

__global__ __launch_bounds__(kThreads) void bwd_kv_reduce(BwdParams p) {
  const int splits = p.kv_reduce_count ? *p.kv_reduce_count : int(gridDim.x);
  const int v = blockIdx.y * kThreads + threadIdx.x;
  const int tensor = v / (kB * kD / 4);              // 0: dK, 1: dV
  const int e = 4 * (v % (kB * kD / 4));             // element (key * 128 + d) of the tile
  const float mul = tensor == 0 ? p.scale : 1.f;
  for (int r = blockIdx.x; r < splits; r += gridDim.x) {
    const int item = p.kv_reduce[4 * r];
    const int first = p.kv_reduce[4 * r + 1];
    const int count = p.kv_reduce[4 * r + 2];
    const int j = item % p.nb;
    const int bk = item / p.nb;
    const int hk = bk % p.Hkv, b = bk / p.Hkv;
    const int64_t row0 = (int64_t(b) * p.Hkv + hk) * p.N + int64_t(j) * kB;
    if (int64_t(j) * kB + e / kD >= p.N) continue;    // beyond a ragged sequence's end
    f32x4 acc = f32x4{};
    for (int c = 0; c < count; ++c)
      acc += *reinterpret_cast<const f32x4*>(p.kv_scratch + (int64_t(first + c) * 2 + tensor) * kB * kD + e);
    u32x2 pk;
    pk[0] = uint32_t(bf16_bits(acc[0] * mul)) | (uint32_t(bf16_bits(acc[1] * mul)) << 16);
    pk[1] = uint32_t(bf16_bits(acc[2] * mul)) | (uint32_t(bf16_bits(acc[3] * mul)) << 16);
    uint16_t* const dst = (tensor == 0 ? p.dk : p.dv) + row0 * kD + e;
    *reinterpret_cast<u32x2*>(dst) = pk;
  }
}

// ---------------------------------------------------------------------------
// float32 backward (head_dim 64 | 128, block 64 | 128): exact fp32 FMAs on the
// VALU, for fp32 inputs (the exact-precision path; small problems).  As in the
// fp32 forward, 4 consecutive lanes share one row, each holding a quarter of
// the head dimension, and a dot product is their partial sums combined by two
// butterfly exchanges.  dQ: one workgroup per (b, h, q-block) over its CSR
// row, K and V staged through LDS in stages of up to 64 keys.  dK/dV: one
// workgroup per (b, KV head, k-block) over its transposed lists (whole walks;
// the fp32 path does not split them), Q, dO, LSE and Delta staged likewise.
// ---------------------------------------------------------------------------
constexpr int kF32Lanes = 4;

// Sum over the kF32Lanes (4) lanes of each aligned lane quad: butterfly
// exchanges with lanes l ^ 1 and l ^ 2 through DPP quad permutations, which
// move values between lanes inside the VALU instead of through LDS.
__device__ __forceinline__ float quad_sum(float a) {
  a += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, a), 0xB1, 0xF, 0xF, false));
  a += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, a), 0x4E, 0xF, 0xF, false));
  return a;
}

// Delta_q = <dO_q, O_q> for float32 rows of D values, 16 lanes per row.
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_delta_f32(const float* __restrict__ o, const float* __restrict__ dout,
                                                        float* __restrict__ delta, int64_t rows, BwdParams p) {
  const int64_t row = int64_t(blockIdx.x) * (kThreads / 16) + (threadIdx.x >> 4);
  const int c = threadIdx.x & 15;
  float s = 0.f;
  // Rows at or beyond their entry's length (variable-length batches) are
  // padding: not read, and their Delta is 0.
  const bool inside = row < rows && (!p.seq_lens || row % p.N < entry_length(p, int(row / p.N / p.H)));
  if (inside) {
#pragma unroll
    for (int d = c; d < D; d += 16) s = fmaf(o[row * D + d], dout[row * D + d], s);
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) s += __shfl_xor(s, m);
  if (c == 0 && row < rows) delta[row] = s;
}

template <int D, int BS>
__global__ __launch_bounds__(BS * kF32Lanes) void bwd_dq_f32(BwdParams p) {
  constexpr int KT = BS < 64 ? BS : 64;  // keys per LDS stage
  constexpr int DL = D / kF32Lanes;      // head-dimension slice per lane
  constexpr int NT = BS * kF32Lanes;     // threads
  extern __shared__ float smem[];
  float* Ks = smem;                      // [KT][D]
  float* Vs = Ks + KT * D;               // [KT][D]

  const int item = p.work[blockIdx.x];
  if (item < 0) return;
  const int i = item % p.nb;
  const int bh = item / p.nb;
  const int h = bh % p.H, b = bh / p.H;
  const int hk = h / p.group;
  const RowDesc row = p.rows[(p.per_head_layout ? h : 0) * p.nb + i];
  const int t = threadIdx.x;
  const int r = t / kF32Lanes, sl = t % kF32Lanes;
  const int qg = i * BS + r;
  // The entry's length and block count: the walk is the prefix of the
  // ascending CSR row below block nbb, tiles of a shorter last block are
  // masked token by token, and rows at or beyond Nb load row Nb - 1.
  const int Nb = entry_length(p, b);
  const int nbb = (Nb + BS - 1) / BS;
  const bool short_tail = Nb % BS != 0;
  int ne = i >= nbb ? 0 : row.count;
  while (ne > 0 && (p.entries[row.start + ne - 1] >> 1) >= nbb) --ne;
  const int64_t hb = (int64_t(b) * p.H + h) * p.N;
  const int64_t qld = hb + (qg < Nb ? qg : (Nb > 0 ? Nb - 1 : 0));
  const float* fq = reinterpret_cast<const float*>(p.q);
  const float* fdo = reinterpret_cast<const float*>(p.dout);
  const float* Kb = reinterpret_cast<const float*>(p.k) + (int64_t(b) * p.Hkv + hk) * p.N * D;
  const float* Vb = reinterpret_cast<const float*>(p.v) + (int64_t(b) * p.Hkv + hk) * p.N * D;
  float qv[DL], dov[DL], acc[DL];
#pragma unroll
  for (int d = 0; d < DL; ++d) {
    qv[d] = fq[qld * D + sl * DL + d];
    dov[d] = fdo[qld * D + sl * DL + d];
    acc[d] = 0.f;
  }
  const float lse = p.lse[qld];
  const float lse2 = lse == -INFINITY ? 0.f : lse * kLog2e;   // empty rows: every score is masked
  const float dlt = p.delta[qld];

  for (int e = 0; e < ne; ++e) {
    const int ent = p.entries[row.start + e];
    const int j = ent >> 1;
    const bool partial = (ent & 1) || (short_tail && (j == nbb - 1 || i == nbb - 1));
    for (int st = 0; st < BS / KT; ++st) {
      const int k0 = j * BS + st * KT;
      __syncthreads();
      for (int x = t; x < KT * D / 4; x += NT) {
        const int64_t kr = k0 + x / (D / 4) < Nb ? k0 + x / (D / 4) : Nb - 1;
        const int64_t src = kr * D + (x % (D / 4)) * 4;
        reinterpret_cast<float4*>(Ks)[x] = *reinterpret_cast<const float4*>(Kb + src);
        reinterpret_cast<float4*>(Vs)[x] = *reinterpret_cast<const float4*>(Vb + src);
      }
      __syncthreads();
      for (int kk = 0; kk < KT; ++kk) {
        // This lane's slices of the key's K and V rows, 16 bytes per LDS read.
        float kr[DL], vr[DL];
#pragma unroll
        for (int d4 = 0; d4 < DL / 4; ++d4) {
          *reinterpret_cast<float4*>(kr + 4 * d4) = reinterpret_cast<const float4*>(Ks + kk * D + sl * DL)[d4];
          *reinterpret_cast<float4*>(vr + 4 * d4) = reinterpret_cast<const float4*>(Vs + kk * D + sl * DL)[d4];
        }
        float a = 0.f, c = 0.f;
#pragma unroll
        for (int d = 0; d < DL; ++d) {
          a = fmaf(qv[d], kr[d], a);
          c = fmaf(dov[d], vr[d], c);
        }
        a = quad_sum(a);
        c = quad_sum(c);
        const float pr = (partial && !pair_ok(p, qg, k0 + kk, Nb)) ? 0.f : __builtin_amdgcn_exp2f(fmaf(a, p.sl2, -lse2));
        const float ds = pr * (c - dlt);
#pragma unroll
        for (int d = 0; d < DL; ++d) acc[d] = fmaf(ds, kr[d], acc[d]);
      }
    }
  }
  if (qg >= p.N) return;
  float* dq = reinterpret_cast<float*>(p.dq) + (hb + qg) * D + sl * DL;
#pragma unroll
  for (int d = 0; d < DL; ++d) dq[d] = acc[d] * p.scale;
}

template <int D, int BS>
__global__ __launch_bounds__(BS * kF32Lanes) void bwd_dkdv_f32(BwdParams p) {
  constexpr int QT = BS < 64 ? BS : 64;  // queries per LDS stage
  constexpr int DL = D / kF32Lanes;
  constexpr int NT = BS * kF32Lanes;
  extern __shared__ float smem[];
  float* Qs = smem;                      // [QT][D]
  float* dOs = Qs + QT * D;              // [QT][D]
  float* Ls = dOs + QT * D;              // [QT] LSE * log2(e) (0 for empty rows)
  float* Dls = Ls + QT;                  // [QT] Delta

  const int item = blockIdx.x;           // (b * Hkv + hk) * nb + j, every item once
  const int j = item % p.nb;
  const int bk = item / p.nb;
  const int hk = bk % p.Hkv, b = bk / p.Hkv;
  const int t = threadIdx.x;
  const int r = t / kF32Lanes, sl = t % kF32Lanes;
  const int kg = j * BS + r;
  // As in dQ: a k-block at or beyond block nbb has no walk, each list stops
  // below block nbb, and rows at or beyond Nb load row Nb - 1.
  const int Nb = entry_length(p, b);
  const int nbb = (Nb + BS - 1) / BS;
  const bool short_tail = Nb % BS != 0;
  const int64_t kvb = (int64_t(b) * p.Hkv + hk) * p.N;
  const int64_t kld = kvb + (kg < Nb ? kg : (Nb > 0 ? Nb - 1 : 0));
  const float* fk = reinterpret_cast<const float*>(p.k);
  const float* fv = reinterpret_cast<const float*>(p.v);
  float kv[DL], vv[DL], dk[DL], dv[DL];
#pragma unroll
  for (int d = 0; d < DL; ++d) {
    kv[d] = fk[kld * D + sl * DL + d];
    vv[d] = fv[kld * D + sl * DL + d];
    dk[d] = 0.f;
    dv[d] = 0.f;
  }
  for (int g = 0; g < (j < nbb ? p.group : 0); ++g) {
    const int h = hk * p.group + g;
    const RowDesc col = p.cols[(p.per_head_layout ? h : 0) * p.nb + j];
    const int64_t hb = (int64_t(b) * p.H + h) * p.N;
    const float* Qb = reinterpret_cast<const float*>(p.q) + hb * D;
    const float* dOb = reinterpret_cast<const float*>(p.dout) + hb * D;
    for (int e = 0; e < col.count; ++e) {
      const int ent = p.entries_t[col.start + e];
      const int i = ent >> 1;
      if (i >= nbb) break;                        // the lists ascend in q-block
      const bool partial = (ent & 1) || (short_tail && (j == nbb - 1 || i == nbb - 1));
      for (int st = 0; st < BS / QT; ++st) {
        const int q0 = i * BS + st * QT;
        __syncthreads();
        for (int x = t; x < QT * D / 4; x += NT) {
          const int64_t qr = q0 + x / (D / 4) < Nb ? q0 + x / (D / 4) : Nb - 1;
          const int64_t src = qr * D + (x % (D / 4)) * 4;
          reinterpret_cast<float4*>(Qs)[x] = *reinterpret_cast<const float4*>(Qb + src);
          reinterpret_cast<float4*>(dOs)[x] = *reinterpret_cast<const float4*>(dOb + src);
        }
        for (int x = t; x < QT; x += NT) {
          const int64_t qr = hb + (q0 + x < Nb ? q0 + x : Nb - 1);
          const float l = p.lse[qr];
          Ls[x] = l == -INFINITY ? 0.f : l * kLog2e;
          Dls[x] = p.delta[qr];
        }
        __syncthreads();
        for (int qq = 0; qq < QT; ++qq) {
          // This lane's slices of the query's Q and dO rows, 16 bytes per LDS read.
          float qr[DL], dr[DL];
#pragma unroll
          for (int d4 = 0; d4 < DL / 4; ++d4) {
            *reinterpret_cast<float4*>(qr + 4 * d4) = reinterpret_cast<const float4*>(Qs + qq * D + sl * DL)[d4];
            *reinterpret_cast<float4*>(dr + 4 * d4) = reinterpret_cast<const float4*>(dOs + qq * D + sl * DL)[d4];
          }
          float a = 0.f, c = 0.f;
#pragma unroll
          for (int d = 0; d < DL; ++d) {
            a = fmaf(qr[d], kv[d], a);
            c = fmaf(dr[d], vv[d], c);
          }
          a = quad_sum(a);
          c = quad_sum(c);
          const float pr =
              (partial && !pair_ok(p, q0 + qq, kg, Nb)) ? 0.f : __builtin_amdgcn_exp2f(fmaf(a, p.sl2, -Ls[qq]));
          const float ds = pr * (c - Dls[qq]);
#pragma unroll
          for (int d = 0; d < DL; ++d) {
            dv[d] = fmaf(pr, dr[d], dv[d]);
            dk[d] = fmaf(ds, qr[d], dk[d]);
          }
        }
      }
    }
  }
  if (kg >= p.N) return;
  float* dkp = reinterpret_cast<float*>(p.dk) + (kvb + kg) * D + sl * DL;
  float* dvp = reinterpret_cast<float*>(p.dv) + (kvb + kg) * D + sl * DL;
#pragma unroll
  for (int d = 0; d < DL; ++d) {
    dkp[d] = dk[d] * p.scale;
    dvp[d] = dv[d];
  }
}

template <int D, int BS>
hipError_t launch_f32_backward(const BwdParams& prm, const Plan& plan, hipStream_t s) {
  constexpr int T = (BS < 64 ? BS : 64);
  constexpr size_t smem_dq = size_t(2 * T * D) * sizeof(float);
  constexpr size_t smem_kv = size_t(2 * T * D + 2 * T) * sizeof(float);
  // Set on every launch (a host-side call): the attribute is per device, and
  // a process may launch on several.
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_dq_f32<D, BS>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, int(smem_dq));
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_dkdv_f32<D, BS>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(smem_kv));
  if (e != hipSuccess) return e;
  const bsa_problem_t& pr = plan.prob;
  const int64_t rows = int64_t(pr.batch) * pr.num_heads * pr.seq_len;
  const int64_t rows_per_block = kThreads / 16;
  hipLaunchKernelGGL(bwd_delta_f32<D>, dim3(unsigned((rows + rows_per_block - 1) / rows_per_block)), dim3(kThreads),
                     0, s, static_cast<const float*>(static_cast<const void*>(prm.o)),
                     static_cast<const float*>(static_cast<const void*>(prm.dout)), prm.delta, rows, prm);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((bwd_dq_f32<D, BS>), dim3(unsigned(plan.info.launch_slots)), dim3(BS * kF32Lanes), smem_dq, s,
                     prm);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t kv_items = int64_t(pr.batch) * pr.num_kv_heads * plan.nb;
  if (kv_items > 0) {
    hipLaunchKernelGGL((bwd_dkdv_f32<D, BS>), dim3(unsigned(kv_items)), dim3(BS * kF32Lanes), smem_kv, s, prm);
    err = hipGetLastError();
  }
  return err;
}

bsa_status_t backward_impl(const void* q, const void* k, const void* v, const void* out, const float* lse,
                           const void* dout, bsa_plan_t plan, const int32_t* seq_lens, void* dq, void* dk, void* dv,
                           float* delta, void* stream) {
  if (!plan) return fail(BSA_ERR_INVALID_ARGUMENT, "plan must not be NULL");
  if (!plan->info.on_device)
    return fail(BSA_ERR_INVALID_ARGUMENT, "plan was built by bsa_plan_host and has no device copy");
  const bsa_problem_t& pr = plan->prob;
  const bool bf16 = pr.dtype == BSA_BF16 && pr.head_dim == 128 && pr.block_size == 128;
  const bool f32 = pr.dtype == BSA_F32 && (pr.head_dim == 64 || pr.head_dim == 128) &&
                   (pr.block_size == 64 || pr.block_size == 128);
  if (!bf16 && !f32)
    return fail(BSA_ERR_UNSUPPORTED, "no backward kernel for this (dtype, head_dim, block_size)");
  if (plan->info.work_items == 0) return BSA_OK;
  if (bf16 && plan->kv_partials > 0 && !plan->d_kv_scratch)
    return fail(BSA_ERR_DEVICE, "plan has split dK/dV columns but no partial-sum scratch");
  if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv || !delta)
    return fail(BSA_ERR_INVALID_ARGUMENT, "q, k, v, out, lse, dout, dq, dk, dv and delta must all be non-NULL");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(BSA_ERR_DEVICE, "hipGetDevice failed");
  if (dev != plan->device)
    return fail(BSA_ERR_INVALID_ARGUMENT, "plan was built on device %d but device %d is current",
                plan->device, dev);
  BwdParams prm;
  prm.q = static_cast<const uint16_t*>(q);
  prm.k = static_cast<const uint16_t*>(k);
  prm.v = static_cast<const uint16_t*>(v);
  prm.o = static_cast<const uint16_t*>(out);
  prm.lse = lse;
  prm.dout = static_cast<const uint16_t*>(dout);
  prm.dq = static_cast<uint16_t*>(dq);
  prm.dk = static_cast<uint16_t*>(dk);
  prm.dv = static_cast<uint16_t*>(dv);
  prm.delta = delta;
  prm.rows = plan->d_rows;
  prm.entries = plan->d_entries;
  prm.work = plan->d_work;
  prm.cols = plan->d_cols;
  prm.entries_t = plan->d_entries_t;
  prm.kv_desc = plan->d_work_kv;
  prm.kv_reduce = plan->d_kv_reduce;
  prm.kv_reduce_count = plan->dynamic ? plan->d_kv_count : nullptr;
  prm.kv_scratch = plan->d_kv_scratch;
  prm.N = pr.seq_len;
  prm.N32 = int32_t(pr.seq_len);
  prm.seq_lens = seq_lens;
  prm.H = pr.num_heads;
  prm.Hkv = pr.num_kv_heads;
  prm.group = pr.num_heads / pr.num_kv_heads;
  prm.nb = plan->nb;
  prm.per_head_layout = plan->layout_heads > 1 ? 1 : 0;
  prm.scale = pr.scale;
  prm.sl2 = pr.scale * kLog2e;
  prm.causal = plan->causal;
  prm.token_rule = plan->token_rule;
  auto clamp32 = [&](int64_t x) { return int32_t(x < 0 ? -1 : (x > pr.seq_len ? pr.seq_len : x)); };
  prm.gk32 = clamp32(plan->gk);
  prm.gq32 = clamp32(plan->gq);
  {
    // Range of q - k allowed by the window and the causal cut (|q - k| < N).
    const int64_t big = pr.seq_len + 1;
    int64_t lo = -big, hi = big;
    if (plan->token_rule) {
      if (plan->wr >= 0) lo = -plan->wr;
      if (plan->wl >= 0) hi = plan->wl;
    }
    if (plan->causal) lo = lo > 0 ? lo : 0;
    if (lo < -big) lo = -big;
    if (hi > big) hi = big;
    prm.mlo = int32_t(lo);
    prm.mspan = uint32_t(hi - lo);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (f32) {
    hipError_t e = hipSuccess;
    if (pr.head_dim == 64 && pr.block_size == 64) e = launch_f32_backward<64, 64>(prm, *plan, s);
    else if (pr.head_dim == 64) e = launch_f32_backward<64, 128>(prm, *plan, s);
    else if (pr.block_size == 64) e = launch_f32_backward<128, 64>(prm, *plan, s);
    else e = launch_f32_backward<128, 128>(prm, *plan, s);
    if (e != hipSuccess) return fail(BSA_ERR_DEVICE, "backward kernel launch failed: %s", hipGetErrorString(e));
    return BSA_OK;
  }
  const bool ragged = pr.seq_len % kB != 0 || seq_lens;
  prm.lq_dq = launch_queue(*plan, 0);
  prm.lq_kv = launch_queue(*plan, 1);
  const unsigned grid_dq = unsigned(int64_t(prm.lq_dq.static_slots) + prm.lq_dq.dyn_total);
  const unsigned grid_kv = unsigned(int64_t(prm.lq_kv.static_slots) + prm.lq_kv.dyn_total);
  if (ragged)
    hipLaunchKernelGGL(bwd_dq_bf16_d128<true>, dim3(grid_dq), dim3(kThreads), 0, s, prm);
  else
    hipLaunchKernelGGL(bwd_dq_bf16_d128<false>, dim3(grid_dq), dim3(kThreads), 0, s, prm);
  hipError_t err = hipGetLastError();
  if (err == hipSuccess && !plan->work_kv.empty()) {
    if (ragged)
      hipLaunchKernelGGL(bwd_dkdv_bf16_d128<true>, dim3(grid_kv), dim3(kThreads), 0, s, prm);
    else
      hipLaunchKernelGGL(bwd_dkdv_bf16_d128<false>, dim3(grid_kv), dim3(kThreads), 0, s, prm);
    err = hipGetLastError();
  }
  if (err == hipSuccess && plan->kv_reduce_launch > 0) {
    hipLaunchKernelGGL(bwd_kv_reduce, dim3(unsigned(plan->kv_reduce_launch), kReduceParts), dim3(kThreads), 0, s,
                       prm);
    err = hipGetLastError();
  }
  if (err != hipSuccess) return fail(BSA_ERR_DEVICE, "backward kernel launch failed: %s", hipGetErrorString(err));
  return BSA_OK;
}

// Workspace of bsa_backward_noalloc: Delta (one float per query row) in a
// file-scope device array instead of a caller buffer, for callers that cannot
// allocate (graph capture, allocation-free loops).  Each GPU the library runs
// on holds its own copy for the life of the process.  Host code never uses
// the array's name as an address: the per-device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr int64_t kScratchFloats = int64_t(16) << 20;   // 64 MiB: batch * heads * seq_len <= 16,777,216
static __device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxScratchDevices] = {};

// Address of `scratch` on device `dev` (the current device) into *out.
bsa_status_t scratch_on(int dev, float** out) {
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(BSA_ERR_UNSUPPORTED, "device ordinal %d is beyond the %d devices this entry point serves", dev,
                kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(BSA_ERR_DEVICE, "hipGetSymbolAddress of the backward workspace failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<float*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return BSA_OK;
}

}  // namespace
}  // namespace bsa

extern "C" bsa_status_t bsa_backward_noalloc(const void* q, const void* k, const void* v, const void* out,
                                             const float* lse, const void* dout, bsa_plan_t plan, void* dq,
                                             void* dk, void* dv, void* stream) {
  using namespace bsa;
  clear_error();
  if (!plan) return fail(BSA_ERR_INVALID_ARGUMENT, "plan must not be NULL");
  if (!plan->info.on_device)
    return fail(BSA_ERR_INVALID_ARGUMENT, "plan was built by bsa_plan_host and has no device copy");
  const bsa_problem_t& pr = plan->prob;
  const int64_t rows = int64_t(pr.batch) * pr.num_heads * pr.seq_len;
  if (rows > kScratchFloats)
    return fail(BSA_ERR_INVALID_ARGUMENT,
                "batch * heads * seq_len = %lld exceeds the %lld rows of the static workspace; use bsa_backward",
                (long long)rows, (long long)kScratchFloats);
  if (plan->info.work_items == 0) return BSA_OK;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(BSA_ERR_DEVICE, "hipGetDevice failed");
  if (dev != plan->device)
    return fail(BSA_ERR_INVALID_ARGUMENT, "plan was built on device %d but device %d is current",
                plan->device, dev);
  float* delta = nullptr;
  const bsa_status_t st = scratch_on(dev, &delta);
  if (st != BSA_OK) return st;
  return backward_impl(q, k, v, out, lse, dout, plan, nullptr, dq, dk, dv, delta, stream);
}

extern "C" bsa_status_t bsa_backward(const void* q, const void* k, const void* v, const void* out,
                                     const float* lse, const void* dout, bsa_plan_t plan, void* dq,
                                     void* dk, void* dv, float* delta, void* stream) {
  bsa::clear_error();
  return bsa::backward_impl(q, k, v, out, lse, dout, plan, nullptr, dq, dk, dv, delta, stream);
}

extern "C" bsa_status_t bsa_backward_varlen(const void* q, const void* k, const void* v, const void* out,
                                            const float* lse, const void* dout, bsa_plan_t plan,
                                            const int32_t* seq_lens, void* dq, void* dk, void* dv, float* delta,
                                            void* stream) {
  using namespace bsa;
  clear_error();
  if (!plan) return fail(BSA_ERR_INVALID_ARGUMENT, "plan must not be NULL");
  if (plan->info.work_items == 0) return BSA_OK;
  if (!seq_lens) return fail(BSA_ERR_INVALID_ARGUMENT, "seq_lens must not be NULL");
  hipPointerAttribute_t attr{};
  if (hipPointerGetAttributes(&attr, seq_lens) != hipSuccess || attr.type != hipMemoryTypeDevice ||
      attr.device != plan->device) {
    (void)hipGetLastError();
    return fail(BSA_ERR_INVALID_ARGUMENT, "seq_lens must be device memory of device %d", plan->device);
  }
  return backward_impl(q, k, v, out, lse, dout, plan, seq_lens, dq, dk, dv, delta, stream);
}
