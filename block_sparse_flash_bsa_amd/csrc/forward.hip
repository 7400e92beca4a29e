// Block-sparse flash attention forward kernels for gfx950 (CDNA4) and the
// bsa_forward launcher.
//
// One workgroup owns one (batch, head, q-block) item of the plan's launch
// order and walks that q-block's CSR list of key blocks: fetch K/V block j,
// scores on the tile, online-softmax update, accumulate P.V; finally write
// O = acc / l and LSE = m + ln l.  That is the block-sparse FlashAttention
// procedure of "How Does Flash-MSA Sparse Attention Work?" (How Do Sparse
// Attention Kernels Work in GPU Clusters?) with the running max / running sum
// recurrence of "The Mechanics" (Flash MSA Sparse Attention vs Full
// Attention); only the active tiles are ever computed and no score matrix is
// stored.  Token masks are evaluated only in tiles the plan flags PARTIAL.
//
// bf16 kernel (head_dim 128, block 128): 4 waves x 32 query rows.  Scores are
// computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16, so that
// each lane holds one query row: the row max and row sum are in-lane plus a
// single exchange between lanes l and l + 32.  O^T = V^T P^T keeps that
// layout, so the per-row rescale is a per-lane scalar.  K and V are staged in
// LDS row-major (with an XOR swizzle); the V^T operand of P.V is read with
// ds_read_b64_tr_b16, which transposes 4x4 blocks of 16-bit elements across
// each group of 16 lanes, so no transpose is done in registers.  The key order
// inside each 16-key chunk of P follows the S^T accumulator layout, and the V
// reads use the same order.  The softmax runs in the exp2 domain against a
// reference max that moves only when some P would reach 2^8 (so the
// accumulator is rarely rescaled and, in the common case, no row max is
// computed at all), in passes over independent registers: on gfx950 the VALU
// work per tile is about as large as the matrix work, and dependent
// instruction chains would leave it latency-bound.
//
// Each 128-key tile is processed as two 64-key halves, one barrier per half.
// A half's phase runs the P.V product of the previous half first (its V half
// landed at this barrier), then the scores of this half, then its softmax; the
// P of this half is kept in registers until the next phase.  So each phase is
// one block of 32 MFMAs followed by one block of VALU work, and the HBM->LDS
// loads issued in a phase (the next K half and this half's V) land by the next
// barrier.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "internal.h"
#include "queue.h"

namespace bsa {
namespace {

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const RowDesc* rows;
  const int32_t* entries;
  const int32_t* work;
  int64_t N;
  int32_t H, Hkv, group, nb, per_head_layout;
  float sl2;  // scale * log2(e)
  int32_t causal, token_rule;
  int64_t wl, wr, gk, gq;
  // The same window/global bounds clamped to [-1, N] so tile-local masks use
  // 32-bit arithmetic (N < 2^30 is enforced by the planner).
  int32_t wl32, wr32, gk32, gq32;
  // Window and causal parts of the token predicate as one range of q - k:
  // allowed iff (uint32)(q - k - mlo) <= mspan (mlo <= 0, mspan >= 0).
  int32_t mlo;
  uint32_t mspan;
  // Variable-length batch (bsa_forward_varlen): device int32 [batch], entry b
  // uses its first seq_lens[b] positions; nullptr otherwise.
  const int32_t* seq_lens;
  // Launch of the bf16 kernel: slots of `work` run by one workgroup each,
  // then queue workgroups (queue.h).
  LaunchQueue lq;
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Token-level predicate inside a PARTIAL tile.  With token_rule == 0 the
// window/global part is uniform over the tile and already true for every
// planned tile, so only causality remains.
__device__ __forceinline__ bool allowed(const FwdParams& p, int64_t q, int64_t k) {
  if (k >= p.N) return false;                     // beyond a ragged sequence's end
  if (p.causal && k > q) return false;
  if (!p.token_rule) return true;
  const bool in_w = (p.wl < 0 || q - k <= p.wl) && (p.wr < 0 || k - q <= p.wr);
  return in_w || k < p.gk || q < p.gq;
}

__device__ __forceinline__ void decode(const FwdParams& p, int item, int& b, int& h, int& i) {
  i = item % p.nb;
  const int bh = item / p.nb;
  h = bh % p.H;
  b = bh / p.H;
}

// ---------------------------------------------------------------------------
// bf16, head_dim 128, block 128: MFMA kernel
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 128;        // query rows per workgroup (= layout block)
constexpr int kBN = 128;        // keys per CSR entry (= layout block)
constexpr int kD = 128;         // head dim
constexpr int kThreads = 256;   // 4 waves of 64

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Max of x over lanes l and l ^ 32 (v_permlane32_swap: one result holds the
// lane's own value, the other its partner's).
__device__ __forceinline__ float max_with_partner(float x) {
  const uint32_t b = __float_as_uint(x);
  const auto sw = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

__device__ __forceinline__ float sum_with_partner(float x) {
  const uint32_t b = __float_as_uint(x);
  const auto sw = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// Max of the 16 values of an MFMA accumulator tile as a tree of v_max3.
__device__ __forceinline__ float max3_tree(const f32x16& v) {
  const float a = fmaxf(fmaxf(v[0], v[1]), v[2]), b = fmaxf(fmaxf(v[3], v[4]), v[5]);
  const float c = fmaxf(fmaxf(v[6], v[7]), v[8]), d = fmaxf(fmaxf(v[9], v[10]), v[11]);
  const float e = fmaxf(fmaxf(v[12], v[13]), v[14]);
  return fmaxf(fmaxf(fmaxf(a, b), c), fmaxf(fmaxf(d, e), v[15]));
}

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// One workgroup of 4 waves per (b, h, q-block) work item; wave w owns query
// rows 32w .. 32w+31.  Two workgroups share a CU (64 KB of LDS each), so each
// SIMD interleaves two independent waves whose matrix and softmax phases
// overlap.  K and V are each held as two 16 KB halves (keys 0-63 and 64-127
// of the current tile), all filled by direct HBM->LDS loads
// (global_load_lds_dwordx4; no staging registers, no LDS stores); the item's
// Q tile arrives the same way, through the K and V buffers of half 1, before
// the first tile.  A tile is
// processed in two 64-key halves, each after one workgroup barrier:
//   barrier 1: K and V half 0 of tile e have landed, and every wave is done
//     with half 1 of tile e-1: load K and V half 1 of tile e, then S^T,
//     softmax and P.V of keys 0-63;
//   barrier 2: half 1 of tile e has landed, and every wave is done with half
//     0: load K and V half 0 of tile e+1, then S^T, softmax and P.V of keys
//     64-127.
// Every load has a whole half-tile of work to land, and each barrier issues
// the same 8 loads per wave, interleaved with the S^T MFMAs that follow it
// (issued in one burst they stall the wave until the CU's load path has
// accepted them).  LDS rows are 256 bytes with their 16-byte chunks
// XOR-swizzled (K chunk c of row r at c ^ (r & 15), V chunk c at
// c ^ 4*(r & 3)), which keeps the 16-byte K reads and the transposed V reads
// free of bank conflicts.
constexpr int kHalfBytes = 64 * kD * 2;   // one 64-key half of K or V: 16 KB
typedef __attribute__((address_space(3))) unsigned char lds_u8;

// Wait until at most N of this wave's vector-memory operations are pending,
// then a workgroup barrier.  The "memory" clobber keeps LDS accesses on their
// side of the barrier; vector-memory loads issued later are not waited for.
#define BSA_WAIT_BARRIER(N) \
  __asm__ volatile("s_waitcnt vmcnt(" #N ")\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")

// HBM->LDS load of 16 bytes per lane (1 KB per wave) from sbase + voff into
// LDS at lds_addr + 16 * lane.  Inline assembly, so the compiler adds no
// waits of its own for it (its alias tracking of such loads is coarse and
// would make unrelated LDS reads wait for every load in flight); each use is
// followed by an explicit s_waitcnt vmcnt and a barrier before the data is
// read.
// M0 is reserved for the compiler, which therefore does not honour it as a
// clobber (hence the silenced warning); the compiled kernel has no other use
// of M0, which a CPU test checks in its assembly.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  __asm__ volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                   :: "v"(voff), "s"(sbase), "s"(lds_addr) : "memory", "m0");
}
#pragma clang diagnostic pop

// kRagged: the sequence of this batch entry ends inside a block: N % 128 != 0,
// or a variable-length batch whose entry b has Nb = seq_lens[b] <= N
// positions.  The walk stops at the last key block below Nb; tiles of the
// last block (row or column) are masked token by token (keys and queries at
// or beyond Nb do not exist; rows beyond Nb come out as empty rows, O = 0 and
// LSE = -inf); loads of rows at or beyond Nb read row Nb - 1 instead (padding
// is never read, so it may hold anything), and no row at or beyond N is
// written.  The instance for whole blocks compiles to the same code as
// without the flag.
template <bool kRagged>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_d128(FwdParams p, const int32_t* __restrict__ ents) {
  // Separate arrays per half, so the compiler can tell the halves apart.
  __shared__ __attribute__((aligned(1024))) unsigned char K0[kHalfBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char K1[kHalfBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char V0[kHalfBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char V1[kHalfBytes];
  __shared__ int s_slot;

  // The slot: the workgroup's own, or one claimed from the queues.
  int done;
  const int slot = queue_slot(p.lq, &s_slot, done);
  const int item = slot >= 0 ? p.work[slot] : -1;
  if (item < 0) {
    queue_release(p.lq, done);
    return;
  }
  int b, h, i;
  decode(p, item, b, h, i);
  const int hk = h / p.group;
  const RowDesc row = p.rows[(p.per_head_layout ? h : 0) * p.nb + i];
  // Length of this batch entry's sequence and its block count (kRagged).
  int Nb = int(p.N);
  if (kRagged && p.seq_lens) {
    const int x = p.seq_lens[b];
    Nb = x < 0 ? 0 : (x > Nb ? Nb : x);
  }
  const int nbb = (Nb + kBM - 1) / kBM;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, r32 = lane & 31, hf = lane >> 5;
  const int qrow = wave * 32 + r32;                       // row within the q-block
  const int64_t qg = int64_t(i) * kBM + qrow;             // global query index

  const unsigned char* Kg =
      reinterpret_cast<const unsigned char*>(static_cast<const uint16_t*>(p.k) + (int64_t(b) * p.Hkv + hk) * p.N * kD);
  const unsigned char* Vg =
      reinterpret_cast<const unsigned char*>(static_cast<const uint16_t*>(p.v) + (int64_t(b) * p.Hkv + hk) * p.N * kD);

  // Q^T operand: lane (row r32, half hf) holds d = 16c + 8hf .. +7 for c = 0..7
  // (read from LDS before the first tile, below).
  bf16x8 qf[8];

  // HBM->LDS loads of one 64-key half of K or V tile j: wave w fills rows
  // 16w .. 16w+15 of the half, 4 rows (1 KB) per instruction; lane L writes
  // chunk L % 16 of row 4u + L / 16 and reads the logical chunk the swizzle
  // places there (K: chunk ^ (row & 15), V: chunk ^ 4*(row & 3)).
  const int lr = lane >> 4, lc = lane & 15;
  uint32_t dko[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) dko[u] = (4 * u + lr) * 256 + 16 * (lc ^ (4 * u + lr));
  const uint32_t dvo = lr * 256 + 16 * (lc ^ (4 * lr));
  const uint32_t Ka[2] = {uint32_t(reinterpret_cast<uintptr_t>((lds_u8*)K0)),
                          uint32_t(reinterpret_cast<uintptr_t>((lds_u8*)K1))};
  const uint32_t Va[2] = {uint32_t(reinterpret_cast<uintptr_t>((lds_u8*)V0)),
                          uint32_t(reinterpret_cast<uintptr_t>((lds_u8*)V1))};
  // Instruction u (0..7) of the 8 loads for half hh of tile j: u < 4 K rows,
  // u >= 4 V rows.
  // clamp_c (compile time): the loads may reach rows at or beyond Nb, i.e.
  // the entry ends inside block j; only the ragged instance uses it.
  auto dma_half_part = [&](int j, int hh, int u, auto clamp_c) {
    const int64_t row0 = int64_t(j) * kBN + hh * 64 + wave * 16;
    if constexpr (kRagged && decltype(clamp_c)::value) {
      // Rows relative to the tile's first row (below Nb), clamped to the
      // last row of the sequence in its last block; one code path.
      const int64_t tile0 = int64_t(j) * kBN;
      const int lim = j == nbb - 1 ? Nb - j * kBN - 1 : kBN - 1;
      const int rl = hh * 64 + wave * 16 + 4 * (u & 3) + lr;
      const int rc = rl < lim ? rl : lim;
      const uint32_t chunk = (u < 4 ? dko[u] : dvo) & 255u;
      const uint32_t voff = uint32_t(rc) * 256u + chunk;
      if (u < 4)
        dma16(Kg + tile0 * (kD * 2), voff, Ka[hh] + wave * 16 * 256 + u * 1024);
      else
        dma16(Vg + tile0 * (kD * 2), voff, Va[hh] + wave * 16 * 256 + (u - 4) * 1024);
      return;
    }
    if (u < 4)
      dma16(Kg + row0 * (kD * 2), dko[u], Ka[hh] + wave * 16 * 256 + u * 1024);
    else
      dma16(Vg + row0 * (kD * 2), dvo + (u - 4) * 1024, Va[hh] + wave * 16 * 256 + (u - 4) * 1024);
  };

  // Per-lane LDS operand offsets (swizzle folded in).
  // K (A operand of S^T): row 32t + r32 of a half, logical chunk 2cc + hf.
  uint32_t koff[8];
#pragma unroll
  for (int cc = 0; cc < 8; ++cc) koff[cc] = r32 * 256 + 16 * ((2 * cc + hf) ^ (r32 & 15));
  // V^T operand by transposed reads: in 16-lane group g, lane 4*r4 + c4
  // addresses key row 16*cq + 8*s + 4*hf + r4 of a half and columns
  // 32*dt + 16*(g & 1) + 4*c4 .. +3; lane l then receives the 4 keys of
  // column d = 32*dt + (l & 31).
  const int r4 = (lane & 15) >> 2, c4 = lane & 3, gp = (lane >> 4) & 1;
  uint32_t voff[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
    voff[dt] = (4 * hf + r4) * 256 + 16 * ((4 * dt + 2 * gp + (c4 >> 1)) ^ (4 * r4)) + 8 * (c4 & 1);
  lds_u8* const K3[2] = {(lds_u8*)K0, (lds_u8*)K1};
  lds_u8* const V3[2] = {(lds_u8*)V0, (lds_u8*)V1};

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  float m_ref = -INFINITY;   // reference max (log2 domain, scaled)
  float l_part = 0.f;        // this lane's share of the row sum
  const float c = p.sl2;
  float cv;                  // c in a VGPR (see exp_pass)
  uint32_t span_v;           // mspan in a VGPR (the mask compares read only VGPRs)
  __asm__("v_mov_b32 %0, %1" : "=v"(cv) : "s"(c));
  __asm__("v_mov_b32 %0, %1" : "=v"(span_v) : "s"(p.mspan));
  const bool q_global = qg < p.gq32;

  // S^T for the 64 keys of half hh: two 32x32 tiles; lane holds row r32,
  // keys 64*hh + 32*t + 8*(r/4) + 4*hf + r%4 in accumulator register r of
  // tile t.  The 16 MFMAs alternate between the two tiles' accumulators
  // (operand k: tile k % 2, d chunk k / 2); each K operand is read from LDS
  // two MFMAs ahead of its use (the scheduling barriers keep that order), and
  // dma(u) issues the barrier's loads, one every other MFMA.
  auto qk_half = [&](int hh, f32x16 (&sq)[2], auto&& dma) {
    lds_u8* const kh = hh ? K3[1] : K3[0];
    auto ld = [&](int k) {
      return *reinterpret_cast<__attribute__((address_space(3))) bf16x8*>(kh + koff[k >> 1] + (k & 1) * 32 * 256);
    };
    sq[0] = f32x16{};
    sq[1] = f32x16{};
    bf16x8 kb[4];
    kb[0] = ld(0);
    kb[1] = ld(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k + 2 < 16) kb[(k + 2) & 3] = ld(k + 2);
      if ((k & 1) == 0) dma(k >> 1);
      __builtin_amdgcn_sched_barrier(0);
      sq[k & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[k & 3], qf[k >> 1], sq[k & 1], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Token mask of half hh of tile j (PARTIAL tiles only), in place.
  auto apply_mask = [&](f32x16 (&sq)[2], int hh, int j) {
    __asm__ volatile("");
    // Window and causal bounds: one unsigned range test of q - k per score
    // (key offsets within the half are compile-time constants).  Global
    // keys and global query rows, when this half or this wave has any, are
    // or-ed in per score, still under the causal bound.
    const int k0 = j * kBN + hh * 64;                            // first key of the half
    const int dq = int(qg) - k0;                                 // q - k at offset 0
    const uint32_t dql = uint32_t(dq) - uint32_t(p.mlo);
    // Every key of the half allowed for every row of the wave: no mask.
    if (__all(dql >= 63u && dql <= p.mspan) && !(kRagged && (j == nbb - 1 || i == nbb - 1))) return;
    if (p.token_rule && (k0 < p.gk32 || __any(q_global))) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ko = t * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
          const bool ok = (dql - uint32_t(ko) <= p.mspan) |
                          (((k0 + ko < p.gk32) | q_global) & (!p.causal | (dq - ko >= 0)));
          sq[t][r] = ok ? sq[t][r] : -INFINITY;
        }
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ko = t * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
          sq[t][r] = dql - uint32_t(ko) <= span_v ? sq[t][r] : -INFINITY;
        }
    }
    if (kRagged && (j == nbb - 1 || i == nbb - 1)) {
      // Keys and queries at or beyond the end of the sequence do not exist.
      const bool row_ok = qg < Nb;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ko = t * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
          sq[t][r] = ((k0 + ko < Nb) & row_ok) ? sq[t][r] : -INFINITY;
        }
    }
  };
  // P = exp2(c*S + nm) (nm = -reference), its bf16 copy, and four partial
  // row sums; S is left as it is.  Every operand is a VGPR: on gfx950 a VALU
  // instruction that reads an SGPR issues at half the rate of one that reads
  // only VGPRs, so the scale is kept in a VGPR copy (cv).
  auto exp_pass = [&](const f32x16 (&sq)[2], float nm, bf16x8 (&pq)[4], float (&ls)[4]) {
    f32x16 pe[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) pe[t][r] = fmaf(sq[t][r], cv, nm);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) pe[t][r] = __builtin_amdgcn_exp2f(pe[t][r]);
    ls[0] = pe[0][0]; ls[1] = pe[0][1]; ls[2] = pe[0][2]; ls[3] = pe[0][3];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) {
          if (t > 0 || q2 > 0 || ii >= 4) ls[ii & 3] += pe[t][q2 * 8 + ii];
          pq[t * 2 + q2][ii] = static_cast<__bf16>(pe[t][q2 * 8 + ii]);
        }
  };
  // Softmax of half hh of tile j: token mask (PARTIAL tiles only), P =
  // exp2(c*S - m_ref) in bf16, and the row sums.  The reference max m_ref
  // stays put while every P is below 2^8, which each lane checks through the
  // sum of its 32 values; otherwise (and until every row of the wave has a
  // finite reference) the row max is formed (in-lane, then with lane l ^ 32),
  // the reference moves to it when some row max exceeds it by more than 2^8
  // (a wave-uniform decision), and O and l are rescaled to match.  The
  // scores survive the fast attempt (its exponentials go to registers of
  // their own), so the fallback needs no second S^T product.  Accumulator
  // registers 8q .. 8q+7 of S^T tile t are exactly the 8 keys this lane
  // supplies for 16-key chunk 2t + q of the P.V product.  The empty volatile
  // asm keeps the conditional blocks real branches.
  auto softmax_half = [&](f32x16 (&sq)[2], int hh, int j, bool partial, bf16x8 (&pq)[4]) {
    if (partial) {
      __asm__ volatile("");
      apply_mask(sq, hh, j);
    }
    float ls[4];
    if (!__any(m_ref == -INFINITY)) {
      // Common case: keep the reference max (no inf/NaN and every P < 2^8).
      exp_pass(sq, -m_ref, pq, ls);
      const float ts = (ls[0] + ls[1]) + (ls[2] + ls[3]);
      if (!__any(!(ts < 256.f))) {
        l_part += ts;
        return;
      }
      __asm__ volatile("");
    }
    float mx = fmaxf(max3_tree(sq[0]), max3_tree(sq[1]));
    mx = max_with_partner(mx);
    const float m_new = mx * c;
    const bool moved = __any(m_new > m_ref + 8.f);
    const float m_use = moved ? fmaxf(m_ref, m_new) : m_ref;
    const float alpha = (m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_use);
    const float msub = (m_use == -INFINITY) ? 0.f : m_use;
    exp_pass(sq, -msub, pq, ls);
    l_part = fmaf(l_part, alpha, (ls[0] + ls[1]) + (ls[2] + ls[3]));
    // Rows whose reference was -inf have O = 0 still (every P so far was 0):
    // no rescale unless some row of the wave had a finite one.
    if (moved && __any(m_ref != -INFINITY)) {
      __asm__ volatile("");
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    }
    m_ref = m_use;
  };
  // O^T += V^T P^T over the four 16-key chunks of V half hh.
  auto pv_half = [&](int hh, const bf16x8 (&pq)[4]) {
    lds_u8* const vh = hh ? V3[1] : V3[0];
    // Operand k = 4*cq + dt; its two reads are issued two MFMAs ahead (a
    // deeper window is faster on short runs but draws enough power on long
    // dense ones to lower the sustained clock).
    auto ld = [&](int k) {
      const int cq = k >> 2, dt = k & 3;
      const bf16x4 lo = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          reinterpret_cast<__attribute__((address_space(3))) s16x4*>(vh + voff[dt] + (16 * cq) * 256)));
      const bf16x4 hi = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          reinterpret_cast<__attribute__((address_space(3))) s16x4*>(vh + voff[dt] + (16 * cq + 8) * 256)));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    bf16x8 vb[4];
    vb[0] = ld(0);
    vb[1] = ld(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k + 2 < 16) vb[(k + 2) & 3] = ld(k + 2);
      __builtin_amdgcn_sched_barrier(0);
      o[k & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb[k & 3], pq[k >> 2], o[k & 3], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int e0 = row.start;
  // kRagged: the walk ends at the last key block below Nb (entries ascend).
  auto walk_length = [&]() {
    int n = i >= nbb ? 0 : row.count;
    while (n > 0 && (ents[e0 + n - 1] >> 1) >= nbb) --n;
    return n;
  };
  const int ne = kRagged ? walk_length() : row.count;
  // One CSR entry (two phases); the last one (no next tile to load) is peeled
  // off so the loop body issues its loads unconditionally.
  bf16x8 pq[4];
  // clamp_c: this tile's loads reach the entry's last block and the entry
  // ends inside it (a uniform choice per tile, so the other tiles' loads take
  // no address arithmetic).
  auto tile = [&](int e, auto next_c, auto clamp_c) {
    constexpr bool has_next = decltype(next_c)::value;
    const int ent = ents[e0 + e];
    const int j = ent >> 1;
    // Tiles of the sequence's last block are masked token by token even where
    // the plan (made for N) calls them FULL.
    const bool partial = (ent & 1) || (kRagged && (Nb % kBN) != 0 && (j == nbb - 1 || i == nbb - 1));
    const int jn = has_next ? ents[e0 + e + 1] >> 1 : 0;
    f32x16 sq[2];
    BSA_WAIT_BARRIER(0);                 // K half 0 of e and V half 1 of e-1 landed
    if (e > 0) pv_half(1, pq);
    qk_half(0, sq, [&](int u) {
      if (u < 4) dma_half_part(j, 1, u, clamp_c);       // K half 1 of e
      else dma_half_part(j, 0, u, clamp_c);             // V half 0 of e
    });
    softmax_half(sq, 0, j, partial, pq);
    BSA_WAIT_BARRIER(0);                 // K half 1 and V half 0 of e landed
    pv_half(0, pq);
    qk_half(1, sq, [&](int u) {
      if (u < 4) {
        if constexpr (has_next) dma_half_part(jn, 0, u, clamp_c);   // K half 0 of e+1
      } else {
        dma_half_part(j, 1, u, clamp_c);                            // V half 1 of e
      }
    });
    softmax_half(sq, 1, j, partial, pq);
  };
  // The entry ends inside its last block (only then do loads need a clamp).
  const bool ctail = kRagged && (Nb % kBN) != 0;
  if (ne > 0) {
    // Q arrives by HBM->LDS loads as well, into K1 (rows 0-63 of the q-block)
    // and V1 (rows 64-127) with K's swizzle, issued together with K half 0 of
    // the first tile; after one barrier each wave reads its Q^T operand from
    // there.  The first tile's barrier then orders those reads before the
    // loads of half 1 into K1 and V1.  Rows at or beyond Nb (kRagged) load
    // row Nb - 1.
    {
      const int64_t R0 = int64_t(i) * kBM + wave * 32;          // the wave's first row
      const int64_t last = kRagged ? (Nb > 0 ? Nb - 1 : 0) : R0 + 31;
      const int64_t Rb = R0 < last ? R0 : last;
      const unsigned char* Qg = reinterpret_cast<const unsigned char*>(
          static_cast<const uint16_t*>(p.q) + ((int64_t(b) * p.H + h) * p.N + Rb) * kD);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        int64_t src = R0 + 4 * u + lr;
        if (kRagged) src = src < last ? src : last;
        const uint32_t voff = uint32_t(src - Rb) * 256u + 16u * (lc ^ ((4 * u + lr) & 15));
        dma16(Qg, voff, ((wave >> 1) ? Va[1] : Ka[1]) + (wave & 1) * (32 * 256) + u * 1024);
      }
    }
    const int j0 = ents[e0] >> 1;
#pragma unroll
    for (int u = 0; u < 4; ++u) dma_half_part(j0, 0, u, std::true_type{});
    BSA_WAIT_BARRIER(0);
    lds_u8* const qs = ((wave >> 1) ? V3[1] : K3[1]) + (wave & 1) * (32 * 256) + r32 * 256;
#pragma unroll
    for (int c = 0; c < 8; ++c)
      qf[c] = *reinterpret_cast<__attribute__((address_space(3))) bf16x8*>(qs + 16 * ((2 * c + hf) ^ (r32 & 15)));
  }
  // Entries ascend and the walk ends at block nbb - 1, so only the last tile
  // and the one before it (through its next entry) can reach that block:
  // every earlier tile takes the unclamped loads.
  if constexpr (kRagged) {
    const int nfast = ctail && ne >= 2 && (ents[e0 + ne - 1] >> 1) == nbb - 1 ? ne - 2 : ne - 1;
    int e = 0;
    for (; e < nfast; ++e) tile(e, std::true_type{}, std::false_type{});
    for (; e + 1 < ne; ++e) tile(e, std::true_type{}, std::true_type{});
  } else {
    for (int e = 0; e + 1 < ne; ++e) tile(e, std::true_type{}, std::false_type{});
  }
  if (ne > 0) {
    tile(ne - 1, std::false_type{}, std::bool_constant<kRagged>{});
    BSA_WAIT_BARRIER(0);
    pv_half(1, pq);
  }

  // Epilogue: O = acc / l (0 for an empty row), LSE = ln2 * (m_ref + log2 l).
  // Each wave stages its 32 x 128 block of O (bf16) in 8 KB of the K buffers,
  // which no wave reads after the last barrier (and which no load fills when
  // the walk is empty), then writes whole 256-byte rows: 16 bytes per lane,
  // four rows per store, instead of 16-byte pieces of 32 rows per store.
  // 16-byte chunk c of row r sits at chunk c ^ (r & 15), so both passes are
  // free of bank conflicts; each wave reads back only what it wrote.
  const float l = sum_with_partner(l_part);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  lds_u8* const stage = ((wave >> 1) ? K3[1] : K3[0]) + (wave & 1) * (32 * 256);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 pk;
      pk[0] = uint32_t(bf16_bits(o[dt][4 * g + 0] * inv)) | (uint32_t(bf16_bits(o[dt][4 * g + 1] * inv)) << 16);
      pk[1] = uint32_t(bf16_bits(o[dt][4 * g + 2] * inv)) | (uint32_t(bf16_bits(o[dt][4 * g + 3] * inv)) << 16);
      *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(
          stage + r32 * 256 + 16 * ((4 * dt + g) ^ (r32 & 15)) + 8 * hf) = pk;
    }
  __asm__ volatile("" ::: "memory");
  const int sr = lane >> 4, sc = lane & 15;      // row within a group of 4, 16-byte chunk
  uint16_t* const Ow = static_cast<uint16_t*>(p.o) + ((int64_t(b) * p.H + h) * p.N + int64_t(i) * kBM + wave * 32) * kD;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int r = 4 * s + sr;
    const u32x4 val = *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(stage + r * 256 + 16 * (sc ^ (r & 15)));
    if (!kRagged || int64_t(i) * kBM + wave * 32 + r < p.N)   // no row beyond a ragged sequence's end
      *reinterpret_cast<u32x4*>(Ow + r * kD + 8 * sc) = val;
  }
  queue_release(p.lq, done);
  if (kRagged && qg >= p.N) return;
  if (hf == 0)
    p.lse[(int64_t(b) * p.H + h) * p.N + qg] = l > 0.f ? (m_ref + log2f(l)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// float32 kernel (head_dim 64/128, block 64/128): exact fp32 FMA on the VALU.
// kF32Lanes consecutive lanes share one query row, each holding a slice of
// the head dimension of Q and of the accumulator; a score is the sum of their
// partial dot products, formed by butterfly exchanges.  K/V tiles are staged through LDS in
// 64-key stages.
// ---------------------------------------------------------------------------
constexpr int kF32Lanes = 4;   // lanes per query row
static_assert(kF32Lanes == 4, "quad_sum reduces over lane quads");

// Sum over the kF32Lanes (4) lanes of each aligned lane quad: butterfly
// exchanges with lanes l ^ 1 and l ^ 2 through DPP quad permutations, which
// move values between lanes inside the VALU instead of through LDS.
__device__ __forceinline__ float quad_sum(float a) {
  a += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, a), 0xB1, 0xF, 0xF, false));
  a += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, a), 0x4E, 0xF, 0xF, false));
  return a;
}

template <int D, int BS>
__global__ __launch_bounds__(BS * kF32Lanes) void fwd_f32(FwdParams p) {
  constexpr int KT = BS < 64 ? BS : 64;  // keys per LDS stage
  constexpr int DL = D / kF32Lanes;      // head-dimension slice per lane
  constexpr int NT = BS * kF32Lanes;     // threads
  extern __shared__ float smem[];
  float* Ks = smem;                      // [KT][D]
  float* Vs = Ks + KT * D;               // [KT][D]

  const int item = p.work[blockIdx.x];
  if (item < 0) return;
  int b, h, i;
  decode(p, item, b, h, i);
  const int hk = h / p.group;
  const RowDesc row = p.rows[(p.per_head_layout ? h : 0) * p.nb + i];
  const int t = threadIdx.x;
  const int r = t / kF32Lanes, sl = t % kF32Lanes;
  const int64_t q0 = int64_t(i) * BS;
  const int64_t qg = q0 + r;
  // This entry's length Nb (seq_lens[b] clamped to [0, N] in a variable-length
  // batch, else N) and block count; the walk is the prefix of the ascending
  // CSR row below block nbb (none for a q-block at or beyond it), and the
  // tiles of a shorter last block are masked token by token.
  int64_t Nb = p.N;
  if (p.seq_lens) {
    const int64_t x = p.seq_lens[b];
    Nb = x < 0 ? 0 : (x > Nb ? Nb : x);
  }
  const int64_t nbb = (Nb + BS - 1) / BS;
  const bool short_tail = Nb % BS != 0;
  int ne = i >= nbb ? 0 : row.count;
  while (ne > 0 && (p.entries[row.start + ne - 1] >> 1) >= nbb) --ne;

  const int64_t qld = qg < Nb ? qg : (Nb > 0 ? Nb - 1 : 0);   // rows at or beyond Nb load row Nb - 1
  const float* Qp = static_cast<const float*>(p.q) + ((int64_t(b) * p.H + h) * p.N + qld) * D + sl * DL;
  const float* Kb = static_cast<const float*>(p.k) + (int64_t(b) * p.Hkv + hk) * p.N * D;
  const float* Vb = static_cast<const float*>(p.v) + (int64_t(b) * p.Hkv + hk) * p.N * D;
  float qv[DL], acc[DL];
#pragma unroll
  for (int d = 0; d < DL; ++d) {
    qv[d] = Qp[d];
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const float c = p.sl2;

  for (int e = 0; e < ne; ++e) {
    const int ent = p.entries[row.start + e];
    const int j = ent >> 1;
    const bool partial = (ent & 1) || (short_tail && (j == nbb - 1 || i == nbb - 1));
    for (int st = 0; st < BS / KT; ++st) {
      const int64_t k0 = int64_t(j) * BS + st * KT;
      __syncthreads();
      for (int x = t; x < KT * D / 4; x += NT) {
        // Keys at or beyond Nb load row Nb - 1; the mask removes them.
        const int64_t kr = k0 + x / (D / 4) < Nb ? k0 + x / (D / 4) : Nb - 1;
        const int64_t src = kr * D + (x % (D / 4)) * 4;
        reinterpret_cast<float4*>(Ks)[x] = *reinterpret_cast<const float4*>(Kb + src);
        reinterpret_cast<float4*>(Vs)[x] = *reinterpret_cast<const float4*>(Vb + src);
      }
      __syncthreads();
      for (int kc = 0; kc < KT; kc += 16) {
        float s[16];
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
          const float4* kr = reinterpret_cast<const float4*>(Ks + (kc + kk) * D + sl * DL);   // 16-byte aligned
          float a = 0.f;
#pragma unroll
          for (int d4 = 0; d4 < DL / 4; ++d4) {
            const float4 kx = kr[d4];
            a = fmaf(qv[4 * d4], kx.x, a);
            a = fmaf(qv[4 * d4 + 1], kx.y, a);
            a = fmaf(qv[4 * d4 + 2], kx.z, a);
            a = fmaf(qv[4 * d4 + 3], kx.w, a);
          }
          a = quad_sum(a);
          const int64_t kk_g = k0 + kc + kk;
          s[kk] = (partial && (kk_g >= Nb || qg >= Nb || !allowed(p, qg, kk_g))) ? -INFINITY : a * c;
        }
        float mx = m;
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) mx = fmaxf(mx, s[kk]);
        if (mx > m) {
          const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mx);
          l *= alpha;
#pragma unroll
          for (int d = 0; d < DL; ++d) acc[d] *= alpha;
          m = mx;
        }
        const float msub = (m == -INFINITY) ? 0.f : m;
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
          const float pv = __builtin_amdgcn_exp2f(s[kk] - msub);
          l += pv;
          const float4* vr = reinterpret_cast<const float4*>(Vs + (kc + kk) * D + sl * DL);
#pragma unroll
          for (int d4 = 0; d4 < DL / 4; ++d4) {
            const float4 vx = vr[d4];
            acc[4 * d4] = fmaf(pv, vx.x, acc[4 * d4]);
            acc[4 * d4 + 1] = fmaf(pv, vx.y, acc[4 * d4 + 1]);
            acc[4 * d4 + 2] = fmaf(pv, vx.z, acc[4 * d4 + 2]);
            acc[4 * d4 + 3] = fmaf(pv, vx.w, acc[4 * d4 + 3]);
          }
        }
      }
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;     // rows at or beyond Nb: O = 0, LSE = -inf
  if (qg >= p.N) return;                          // beyond a ragged sequence's end
  float* Op = static_cast<float*>(p.o) + ((int64_t(b) * p.H + h) * p.N + qg) * D + sl * DL;
#pragma unroll
  for (int d = 0; d < DL; ++d) Op[d] = acc[d] * inv;
  if (sl == 0) p.lse[(int64_t(b) * p.H + h) * p.N + qg] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
}

template <int D, int BS>
constexpr size_t f32_smem_bytes() {
  return size_t(2 * (BS < 64 ? BS : 64) * D) * sizeof(float);
}

template <int D, int BS>
hipError_t launch_f32(const FwdParams& prm, int64_t slots, hipStream_t stream) {
  constexpr size_t smem = f32_smem_bytes<D, BS>();
  // Set on every launch (a host-side call): the attribute is per device, and
  // a process may launch on several.
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&fwd_f32<D, BS>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fwd_f32<D, BS>), dim3(unsigned(slots)), dim3(BS * kF32Lanes), smem, stream, prm);
  return hipGetLastError();
}

}  // namespace
}  // namespace bsa

namespace bsa {
namespace {

bsa_status_t forward_impl(const void* q, const void* k, const void* v, bsa_plan_t plan, const int32_t* seq_lens,
                          void* out, float* lse, void* stream) {
  using namespace bsa;
  clear_error();
  if (!plan) return fail(BSA_ERR_INVALID_ARGUMENT, "plan must not be NULL");
  if (!plan->info.on_device)
    return fail(BSA_ERR_INVALID_ARGUMENT, "plan was built by bsa_plan_host and has no device copy");
  const int64_t slots = plan->info.launch_slots;
  if (plan->info.work_items == 0) return BSA_OK;
  if (!q || !k || !v || !out || !lse)
    return fail(BSA_ERR_INVALID_ARGUMENT, "q, k, v, out and lse must all be non-NULL");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(BSA_ERR_DEVICE, "hipGetDevice failed");
  if (dev != plan->device)
    return fail(BSA_ERR_INVALID_ARGUMENT, "plan was built on device %d but device %d is current",
                plan->device, dev);
  const bsa_problem_t& pr = plan->prob;
  FwdParams prm;
  prm.q = q;
  prm.k = k;
  prm.v = v;
  prm.o = out;
  prm.lse = lse;
  prm.seq_lens = seq_lens;
  prm.rows = plan->d_rows;
  prm.entries = plan->d_entries;
  prm.work = plan->d_work;
  prm.N = pr.seq_len;
  prm.H = pr.num_heads;
  prm.Hkv = pr.num_kv_heads;
  prm.group = pr.num_heads / pr.num_kv_heads;
  prm.nb = plan->nb;
  prm.per_head_layout = plan->layout_heads > 1 ? 1 : 0;
  prm.sl2 = pr.scale * kLog2e;
  prm.causal = plan->causal;
  prm.token_rule = plan->token_rule;
  prm.wl = plan->wl;
  prm.wr = plan->wr;
  prm.gk = plan->gk;
  prm.gq = plan->gq;
  auto clamp32 = [&](int64_t x) { return int32_t(x < 0 ? -1 : (x > pr.seq_len ? pr.seq_len : x)); };
  prm.wl32 = clamp32(plan->wl);
  prm.wr32 = clamp32(plan->wr);
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
  hipError_t err = hipSuccess;
  prm.lq = launch_queue(*plan, 0);
  if (pr.dtype == BSA_BF16 && pr.head_dim == 128 && pr.block_size == 128) {
    const int64_t grid = int64_t(prm.lq.static_slots) + prm.lq.dyn_total;
    if (pr.seq_len % kBN != 0 || seq_lens)
      hipLaunchKernelGGL(fwd_bf16_d128<true>, dim3(unsigned(grid)), dim3(kThreads), 0, s, prm, prm.entries);
    else
      hipLaunchKernelGGL(fwd_bf16_d128<false>, dim3(unsigned(grid)), dim3(kThreads), 0, s, prm, prm.entries);
    err = hipGetLastError();
  } else if (pr.dtype == BSA_F32 && pr.head_dim == 64 && pr.block_size == 64) {
    err = launch_f32<64, 64>(prm, slots, s);
  } else if (pr.dtype == BSA_F32 && pr.head_dim == 64 && pr.block_size == 128) {
    err = launch_f32<64, 128>(prm, slots, s);
  } else if (pr.dtype == BSA_F32 && pr.head_dim == 128 && pr.block_size == 64) {
    err = launch_f32<128, 64>(prm, slots, s);
  } else if (pr.dtype == BSA_F32 && pr.head_dim == 128 && pr.block_size == 128) {
    err = launch_f32<128, 128>(prm, slots, s);
  } else {
    return fail(BSA_ERR_UNSUPPORTED, "no kernel for this (dtype, head_dim, block_size)");
  }
  if (err != hipSuccess) return fail(BSA_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(err));
  return BSA_OK;
}

}  // namespace
}  // namespace bsa

extern "C" bsa_status_t bsa_forward(const void* q, const void* k, const void* v, bsa_plan_t plan,
                                    void* out, float* lse, void* stream) {
  return bsa::forward_impl(q, k, v, plan, nullptr, out, lse, stream);
}

extern "C" bsa_status_t bsa_forward_varlen(const void* q, const void* k, const void* v, bsa_plan_t plan,
                                           const int32_t* seq_lens, void* out, float* lse, void* stream) {
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
  return forward_impl(q, k, v, plan, seq_lens, out, lse, stream);
}
