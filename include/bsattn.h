/*
 * libbsattn -- block-sparse flash attention forward for AMD Instinct MI355X
 * (gfx950 / CDNA4).  C ABI: plain structs, plain pointers, status codes.
 *
 * The operation (forward; the backward is declared with bsa_backward):
 *   For every batch b, query head h and query q, with hk = h / (H / Hkv):
 *     A(q)  = { k : allowed(h, q, k) }                 (the sparse layout)
 *     s_k   = scale * dot(Q[b,h,q,:], K[b,hk,k,:])      k in A(q)
 *     O[b,h,q,:] = sum_k softmax(s)_k * V[b,hk,k,:]
 *     LSE[b,h,q] = log(sum_k exp(s_k))                  (natural log)
 *   An empty A(q) gives O = 0 and LSE = -inf.
 *   Sources: the attention formula softmax(QK^T / sqrt(d_k)) V, section "The
 *   Mechanics: How Flash MSA Sparse Attention Works Under the Hood" of the page
 *   "Flash MSA Sparse Attention vs Full Attention"; the five-step block-sparse
 *   procedure (tile the sequence, block-level mask, fetch only active K/V
 *   blocks, flash tiling over them, online-softmax accumulation), section "How
 *   Does Flash-MSA Sparse Attention Work?" of "How Do Sparse Attention Kernels
 *   Work in GPU Clusters?"; the (batch, heads, seq_len, d_head) inputs and a
 *   mask given as bits or as block indices, section "The Architecture of Flash
 *   MSA Sparse Attention Kernels" of "Flash MSA Sparse Attention Kernels
 *   Explained".  The score matrix is never materialised.  The log-sum-exp
 *   output is this library's addition: merging partial results by online
 *   softmax and a backward pass both need it.
 *
 * Layout predicate (which (q, k) pairs are allowed), with u = units of the
 * window/global fields (tokens: q, k; blocks: q / block, k / block):
 *   allowed = causal_ok && (bitmap ? bitmap[hl][q/bs][k/bs]
 *                                  : in_window || key_global || query_global)
 *   causal_ok    = !causal || k <= q                (always token-exact)
 *   in_window    = (wl < 0 || qu - ku <= wl) && (wr < 0 || ku - qu <= wr)
 *   key_global   = ku < global_keys
 *   query_global = qu < global_queries
 * Sliding window |i - j| <= W and the causal window: section "The Mechanics"
 * of "Flash MSA Sparse Attention vs Full Attention"; global tokens that both
 * see and are seen by every position: "Global Tokens" under "Sparse Patterns
 * Beyond Sliding Windows" on the same page; a window counted in blocks plus
 * a few global blocks: "The Real Deal: Block-Sparse FlashAttention" of "The
 * Only Guide You Need for Sparse Attention Kernels in Long-Context LLMs".
 *
 * Threading: calls on different plans may run concurrently; a plan may be
 * used by several streams at once (the forwards only read it), except that
 * bsa_plan_set_bitmap rewrites a dynamic plan and must not overlap a forward
 * or backward that uses it on another stream (nor another set_bitmap: the
 * plan's count and scan scratch is shared), and backward calls
 * (bsa_backward, bsa_backward_varlen) with one plan must not overlap each
 * other (they share the plan's partial-sum scratch).  The last error string
 * is thread-local.
 */
#ifndef BSATTN_H
#define BSATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSA_ABI_VERSION 7

/* Status codes.  Every entry point that can fail returns one; no exception
 * crosses the ABI.  Out-parameters are written only on BSA_OK. */
typedef int32_t bsa_status_t;
#define BSA_OK                   0
#define BSA_ERR_INVALID_ARGUMENT 1  /* bad shape, pointer, field or plan state */
#define BSA_ERR_UNSUPPORTED      2  /* valid but not built: (dtype, head_dim, block) */
#define BSA_ERR_OUT_OF_MEMORY    3  /* host or device allocation failed */
#define BSA_ERR_DEVICE           4  /* HIP runtime error (launch, copy, device) */

/* Element type of Q, K, V and O.  LSE is always float32. */
#define BSA_F32  0
#define BSA_BF16 1

/* Units of the window/global fields of bsa_layout_t. */
#define BSA_UNIT_TOKENS 0
#define BSA_UNIT_BLOCKS 1

/* Work-order policy for the plan (which workgroup runs which q-block). */
#define BSA_SCHEDULE_DEFAULT  0  /* = BSA_SCHEDULE_XCD */
#define BSA_SCHEDULE_XCD      1  /* locality runs per XCD, cost-balanced, LPT tail */
#define BSA_SCHEDULE_LPT      2  /* global longest-first */
#define BSA_SCHEDULE_ROWMAJOR 3  /* (b, h, q-block) order */

/* The attention problem a plan is prepared for.
 *   batch >= 0, num_heads >= 1, num_kv_heads >= 1, num_heads % num_kv_heads == 0
 *     (query head h reads KV head h / (num_heads / num_kv_heads)).
 *   seq_len in [0, 2^30].  When block_size does not divide it, the last block
 *     is shorter: positions at or beyond seq_len neither attend nor are
 *     attended (the kernels pad virtually: they read row seq_len - 1 in place
 *     of missing rows, mask them, and write no row beyond seq_len - 1), and
 *     every tile touching that block is PARTIAL.  The FAQ of "The Only Guide
 *     You Need for Sparse Attention Kernels in Long-Context LLMs" answers the
 *     variable-length question by padding to the block size; this does that
 *     padding inside the kernels, for static and dynamic plans alike.
 *   block_size: layout block = kernel tile height and width.
 *   Supported (dtype, head_dim, block_size):
 *     BSA_BF16: (128, 128)                    -- MFMA kernel
 *     BSA_F32 : (64 | 128, 64 | 128)          -- exact fp32 kernel
 *   scale: 0 means 1/sqrt(head_dim); otherwise finite and > 0.
 *   schedule: one of BSA_SCHEDULE_*.
 *   batch * num_heads * (seq_len / block_size) must stay below 2^30.
 */
typedef struct {
  int32_t batch;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int64_t seq_len;
  int32_t block_size;
  int32_t dtype;
  float   scale;
  int32_t schedule;
} bsa_problem_t;

/* Which (q, k) pairs are allowed (see the predicate above).
 *   causal: 0 or 1.  unit: BSA_UNIT_TOKENS or BSA_UNIT_BLOCKS.
 *   window_left, window_right >= -1 (-1 = unbounded), inclusive distances.
 *   global_keys, global_queries >= 0.
 *   bitmap: NULL, or a HOST array uint8 [bitmap_heads][nb][nb] (nb =
 *     ceil(seq_len / block_size)), nonzero = block active, row = q-block, column =
 *     k-block; it replaces window/global (causal still applies).  The plan
 *     copies what it needs; the caller keeps ownership.  bitmap_heads is 1
 *     (shared by every head) or num_heads (one layout per query head); the
 *     bitmap is shared across the batch.
 */
typedef struct {
  int32_t causal;
  int32_t unit;
  int64_t window_left;
  int64_t window_right;
  int64_t global_keys;
  int64_t global_queries;
  const uint8_t* bitmap;
  int32_t bitmap_heads;
} bsa_layout_t;

/* Opaque plan: owns its host CSR arrays and, when built by bsa_plan, their
 * device copy on the HIP device that was current at creation. */
typedef struct bsa_plan* bsa_plan_t;

/* Summary of a plan (all counts exact). */
typedef struct {
  int32_t layout_heads;      /* 1 or num_heads */
  int32_t num_blocks;        /* nb = ceil(seq_len / block_size) */
  int64_t nnz;               /* CSR entries over all layout heads */
  int64_t nnz_partial;       /* of which PARTIAL (token mask applied) */
  int64_t active_blocks;     /* sum over (b, h) of the row lengths: tiles computed per forward */
  int64_t allowed_pairs;     /* sum over (b, h) of allowed (q, k) pairs */
  int64_t work_items;        /* batch * num_heads * nb */
  int64_t launch_slots;      /* workgroups launched (>= work_items; idle slots exit) */
  int32_t max_row_entries;   /* longest q-block row */
  int32_t on_device;         /* 1 if the plan has a device copy */
} bsa_plan_info_t;

/* Build a plan: validate the problem and layout, turn the layout into a
 * per-q-block CSR list of key blocks (ascending, each flagged FULL or PARTIAL
 * from its exact allowed-pair count), build the work order, and upload it to
 * the current HIP device (synchronous hipMalloc + hipMemcpy).
 * Per-query-block lists of key blocks: step three of "How Does Flash-MSA
 * Sparse Attention Work?" (each query block fetches only its active K/V
 * blocks) and the precomputed block offsets recommended in the FAQ entry on
 * sparse kernels slower than dense, both on "How Do Sparse Attention Kernels
 * Work in GPU Clusters?".
 * Errors: INVALID_ARGUMENT (NULL pointers, bad fields), UNSUPPORTED,
 * OUT_OF_MEMORY, DEVICE.  *out_plan is written only on BSA_OK. */
bsa_status_t bsa_plan(const bsa_problem_t* problem, const bsa_layout_t* layout,
                      bsa_plan_t* out_plan);

/* Same as bsa_plan but host-only: no HIP call is made, so it works without a
 * GPU.  Such a plan can be inspected but not passed to bsa_forward. */
bsa_status_t bsa_plan_host(const bsa_problem_t* problem, const bsa_layout_t* layout,
                           bsa_plan_t* out_plan);

/* Free a plan and its device copy.  NULL is ignored.  The caller must make
 * sure no forward using the plan is still running (synchronise first). */
void bsa_plan_destroy(bsa_plan_t plan);

/* The CSR of one layout head: row_ptr [nb + 1] (head-local offsets), col_idx
 * [nnz] ascending within each row, flags [nnz] (0 = FULL, 1 = PARTIAL).  The
 * pointers are owned by the plan and valid until bsa_plan_destroy.
 * Errors: INVALID_ARGUMENT for a NULL plan/out pointer or a layout_head out
 * of range. */
bsa_status_t bsa_plan_csr(bsa_plan_t plan, int32_t layout_head, const int32_t** row_ptr,
                          const int32_t** col_idx, const uint8_t** flags, int64_t* nnz);

/* Plan summary.  Errors: INVALID_ARGUMENT for NULL pointers. */
bsa_status_t bsa_plan_get_info(bsa_plan_t plan, bsa_plan_info_t* info);

/* The launch order: slot s of the grid runs item work[s] = (b * H + h) * nb + i,
 * or -1 for an idle slot.  Owned by the plan.  Errors: INVALID_ARGUMENT. */
bsa_status_t bsa_plan_work(bsa_plan_t plan, const int32_t** work, int64_t* slots);

/* Sum over (b, h) of CSR entries: the tiles one forward computes (the
 * numerator of the active-block FLOP count 4 * block^2 * head_dim per tile).
 * Returns -1 for a NULL plan. */
int64_t bsa_plan_active_blocks(bsa_plan_t plan);

/* ---------------------------------------------------------------------------
 * Dynamic plans: the block bitmap lives in device memory and may change from
 * one forward to the next (for instance the per-head block mask a router or a
 * top-k block selector produces on the GPU), so the CSR is derived on the
 * device instead of on the host.  Motivation: rebuilding masks on the host
 * costs milliseconds per change (FAQ on dynamic sparsity of "How Do Sparse
 * Attention Kernels Work in GPU Clusters?"); the learned per-head block masks
 * are those of "Flash-MSA" on "The Only Guide You Need for Sparse Attention
 * Kernels in Long-Context LLMs".  The predicate is the bitmap branch of the
 * one above: tile (i, j) of layout head hl is active iff bitmap[hl][i][j] != 0
 * and (!causal || j <= i); it is PARTIAL iff causal and j == i, or i or j is
 * the shorter last block of a seq_len that block_size does not divide
 * (nb = ceil(seq_len / block_size) blocks per side, as for bsa_plan).
 * ------------------------------------------------------------------------- */

/* Create a dynamic plan on the current HIP device.  layout->bitmap must be
 * NULL; layout->bitmap_heads (1 or num_heads) is the head count of the
 * bitmaps that bsa_plan_set_bitmap will take; layout->causal applies; the
 * window and global fields must be -1 and 0 (unit is ignored).  Device memory
 * for the largest possible CSR is allocated here (bitmap_heads * nb * nb
 * four-byte entries, nb * (nb + 1) / 2 per head when causal; for the bf16
 * backward also min(batch * num_kv_heads * nb, 1024) float32 partial dK/dV
 * tiles of 128 KiB for the chunks of long walks) together with a
 * fixed launch order of every (b, h, q-block) item, locality runs per XCD as
 * in BSA_SCHEDULE_XCD but with equal item counts (row lengths are not known
 * on the host), and the same for the backward's transposed lists and its
 * (b, KV head, k-block) items.  The CSR starts empty: until the first bsa_plan_set_bitmap a
 * forward writes O = 0 and LSE = -inf.  Count fields of bsa_plan_info_t that
 * depend on the bitmap (nnz, nnz_partial, active_blocks, allowed_pairs,
 * max_row_entries) are -1 and bsa_plan_active_blocks returns -1;
 * bsa_plan_work returns the launch order at creation, bsa_plan_csr fails
 * with INVALID_ARGUMENT (bsa_plan_read_csr copies the device CSR back).
 * Errors: INVALID_ARGUMENT, UNSUPPORTED, OUT_OF_MEMORY, DEVICE, as bsa_plan. */
bsa_status_t bsa_plan_dynamic(const bsa_problem_t* problem, const bsa_layout_t* layout,
                              bsa_plan_t* out_plan);

/* Rebuild a dynamic plan's device CSR from d_bitmap, device memory holding
 * [bitmap_heads][nb][nb] bytes (nonzero = active), asynchronously on `stream`
 * (a hipStream_t; NULL = default stream): kernels count each row, scan the
 * counts and write the ascending entries, then do the same per k-block
 * column (the transposed lists bsa_backward walks).  A later bsa_forward on the
 * same stream (or after synchronisation) uses the new CSR.  If d_nnz is not
 * NULL it is a device pointer to one int64_t that receives the total number
 * of entries over all layout heads (multiply by batch, and by num_heads when
 * bitmap_heads == 1, for the tiles one forward computes).  For a plan without
 * the causal cut on the default (XCD) schedule it also re-sorts the launch
 * order: within each (KV head, batch entry) run, q-blocks go longest row
 * first (row lengths of the group's first query head's layout, bucketed, in
 * no fixed order within a bucket), as bsa_plan orders the q-blocks of a
 * static bitmap plan; results do not depend on the order
 * (bsa_plan_read_work copies it back).  The bitmap is read only during the
 * call's kernels; the caller keeps ownership.  Nothing is allocated.
 * Errors (before anything is launched): INVALID_ARGUMENT for a NULL plan or
 * bitmap, a plan that is not dynamic, a bitmap or plan on another device, or
 * a bitmap pointer that is not device memory; DEVICE if a launch fails. */
bsa_status_t bsa_plan_set_bitmap(bsa_plan_t plan, const uint8_t* d_bitmap, int64_t* d_nnz,
                                 void* stream);

/* Copy layout head `layout_head` of a dynamic plan's device CSR to the host
 * (synchronous: waits for the device): row_ptr [nb + 1] head-local offsets,
 * col_idx and flags (0 = FULL, 1 = PARTIAL) of up to `capacity` entries, and
 * the head's entry count in *nnz.  Same format as bsa_plan_csr.
 * Errors: INVALID_ARGUMENT for NULL pointers, a plan that is not dynamic, a
 * layout_head out of range or capacity < the head's entry count; DEVICE if a
 * copy fails. */
bsa_status_t bsa_plan_read_csr(bsa_plan_t plan, int32_t layout_head, int32_t* row_ptr,
                               int32_t* col_idx, uint8_t* flags, int64_t capacity, int64_t* nnz);

/* The same for the transposed lists a dynamic plan builds on the device for
 * the backward (per k-block column, the q-blocks that attend to it,
 * ascending), in the format of bsa_plan_csr_transposed: col_ptr [nb + 1],
 * row_idx and flags [capacity].  Synchronous; errors as bsa_plan_read_csr. */
bsa_status_t bsa_plan_read_csr_transposed(bsa_plan_t plan, int32_t layout_head, int32_t* col_ptr,
                                          int32_t* row_idx, uint8_t* flags, int64_t capacity, int64_t* nnz);

/* Run the forward pass asynchronously on `stream` (a hipStream_t; NULL = the
 * default stream) of the plan's device.
 *   q   : device, [batch][num_heads][seq_len][head_dim], contiguous, dtype
 *   k, v: device, [batch][num_kv_heads][seq_len][head_dim], contiguous, dtype
 *   out : device, [batch][num_heads][seq_len][head_dim], contiguous, dtype
 *         (bf16 rounded to nearest even from float32 accumulators)
 *   lse : device, float32 [batch][num_heads][seq_len]; natural log of the sum
 *         of exp(scaled scores) over the allowed keys; -inf for empty rows
 * All buffers are caller-owned; out and lse must not alias the inputs.  Every
 * element of out and lse is written.  Nothing is allocated or freed.
 * Launch: one workgroup per slot of the plan's order (bsa_plan_work); for the
 * bf16 kernel on a static plan of the XCD order whose rows average 16 tiles
 * or more, the last eighth of each XCD's rows is instead a queue that extra
 * workgroups drain, claiming from any XCD's queue as they free up (XCDs of
 * one chip run a few percent apart).  Its claim counters are plan memory, in
 * 64 sets that successive queued launches take in turn (each launch's last
 * workgroup clears its set): calls with one plan may run concurrently, on any
 * streams, as long as at most 64 queued launches (a forward is one, a
 * backward two) are in flight at once.  Results do not depend on which
 * workgroup runs an item.
 * Errors (returned before anything is launched): INVALID_ARGUMENT for NULL
 * pointers, a host-only plan, or a plan made on another device; DEVICE if
 * the launch fails.  Faults during execution surface at the caller's next
 * synchronisation.  A problem with no work items returns BSA_OK at once. */
bsa_status_t bsa_forward(const void* q, const void* k, const void* v, bsa_plan_t plan,
                         void* out, float* lse, void* stream);

/* ---------------------------------------------------------------------------
 * Backward pass: the gradients of a scalar loss through the forward above,
 * given its upstream gradient dO = dLoss/dO.  With p_qk = exp(s_qk - LSE_q)
 * over k in A(q) (zero elsewhere) and Delta_q = <dO_q, O_q>:
 *   dV_k = sum_q p_qk dO_q
 *   ds_qk = p_qk * (<dO_q, V_k> - Delta_q)          (softmax Jacobian)
 *   dQ_q = scale * sum_k ds_qk K_k,   dK_k = scale * sum_q ds_qk Q_q
 * where keys sum over every query head of their GQA group.  The pages treat
 * the backward through its cost (training throughput of block-sparse vs
 * dense attention in "Sparse Attention Kernels vs Full Attention
 * Performance"; forward and backward timings in the FAQ of "How Do Sparse
 * Attention Kernels Work in GPU Clusters?"); it reuses the forward's LSE, so
 * no score matrix is stored here either.  The q-block walk for dQ is the
 * forward's CSR; the k-block walk for dK and dV is the CSR transposed, which
 * bsa_plan builds with the plan.
 * ------------------------------------------------------------------------- */

/* The transposed CSR of one layout head: col_ptr [nb + 1] (head-local
 * offsets), row_idx [nnz] = the ascending q-blocks whose lists hold k-block
 * j, flags [nnz] as in bsa_plan_csr.  Plan-owned, valid until
 * bsa_plan_destroy.  Errors: INVALID_ARGUMENT for NULL pointers, a dynamic
 * plan, or a layout_head out of range. */
bsa_status_t bsa_plan_csr_transposed(bsa_plan_t plan, int32_t layout_head, const int32_t** col_ptr,
                                     const int32_t** row_idx, const uint8_t** flags, int64_t* nnz);

/* Launch order of the dK/dV kernel: slot s runs item work[s] =
 * (b * num_kv_heads + hk) * nb + j, or -1 for an idle slot.  An item whose
 * walk (the transposed lists of its group's query heads, one after another)
 * is longer than the chunk length C = max(64, 2 * mean walk), such as the
 * k-block of a global key, is cut into k = ceil(walk / C) chunks that occupy
 * several slots; their float32 partial sums live in plan-owned device scratch
 * and a reduction kernel adds them in chunk order.  For a dynamic plan's bf16
 * backward the cut is made on the device by bsa_plan_set_bitmap, by the same
 * rule (so the results equal a static plan's of the same bitmap bit for bit),
 * except that C doubles while the chunks would exceed the plan's budget of
 * min(items, 1024) partial tiles of 128 KiB; its first slots (that budget,
 * rounded up to a multiple of 8) are reserved for those chunks and show here
 * as idle, the other slots as the items' fixed order.  Plan-owned.
 * Errors: INVALID_ARGUMENT for NULL pointers. */
bsa_status_t bsa_plan_work_kv(bsa_plan_t plan, const int32_t** work, int64_t* slots);

/* The forward's (and dQ's) launch order as the device holds it
 * (synchronous: waits for the device): work [slots] in the format of
 * bsa_plan_work.  For a dynamic plan this is the order the last
 * bsa_plan_set_bitmap left (see there).  capacity is the room in work, in
 * slots (bsa_plan_work gives the count).
 * Errors: INVALID_ARGUMENT for NULL pointers, a host-only plan or too small a
 * capacity; DEVICE if the copy fails. */
bsa_status_t bsa_plan_read_work(bsa_plan_t plan, int32_t* work, int64_t capacity, int64_t* slots);

/* The dK/dV launch descriptors as the device holds them (synchronous: waits
 * for the device): desc [slots][4] int32 = {item, first walk entry, end
 * entry, partial tile or -1 for a whole walk}, item -1 for an idle slot;
 * *splits = the number of split columns the reduction sums.  For a dynamic
 * plan these are what the last bsa_plan_set_bitmap wrote.  capacity is the
 * room in desc, in slots (bsa_plan_work_kv gives the count).
 * Errors: INVALID_ARGUMENT for NULL pointers, a host-only plan or too small a
 * capacity; DEVICE if the copy fails. */
bsa_status_t bsa_plan_read_work_kv(bsa_plan_t plan, int32_t* desc, int64_t capacity, int64_t* slots,
                                   int64_t* splits);

/* Run the backward pass asynchronously on `stream` (a hipStream_t; NULL =
 * the default stream) of the plan's device.
 *   q, k, v : the forward's inputs (layouts as in bsa_forward)
 *   out, lse: the forward's outputs for exactly these inputs and this plan
 *   dout    : device, [batch][num_heads][seq_len][head_dim], dtype: dLoss/dO
 *   dq      : device, like q;   dk, dv: device, like k and v (dtype; bf16
 *             is rounded to nearest even from float32 accumulators)
 *   delta   : device, float32 [batch][num_heads][seq_len]: caller-owned
 *             workspace; receives Delta_q = <dO_q, O_q> (computed from the
 *             rounded out), which the dK/dV kernel reads
 * Kernels run in order on the stream: dQ (one workgroup per q-block: it
 * first forms Delta for the block's rows and writes it to delta, then walks
 * the block's CSR row; the float32 path forms Delta in a kernel of its own
 * before dQ), dK/dV (one workgroup per KV head and
 * k-block, walking its transposed list over the group's query heads, or per
 * chunk of a long walk) and, if the plan split any walk, the reduction of
 * the chunks' partial sums.  The bf16 dQ and dK/dV launches of a static
 * plan whose walks average 16 tiles or more end in launch queues as the
 * forward does (see bsa_forward), each taking one of the plan's 64 counter
 * sets.  Every
 * element of dq, dk, dv and delta is written (zero rows where nothing
 * attends).  Outputs must not alias inputs or each other.  Nothing is
 * allocated or freed.
 * Supported: every (dtype, head_dim, block_size) bsa_plan accepts, static or
 * dynamic: BSA_BF16 (128, 128) on MFMA; BSA_F32 (64 | 128, 64 | 128) with
 * exact fp32 FMAs (outputs float32; the fp32 path walks long k-block lists
 * whole instead of splitting them).
 * Errors (before anything is launched): INVALID_ARGUMENT for NULL pointers, a
 * host-only plan or a plan made on another device; UNSUPPORTED as above;
 * DEVICE if a launch fails.  A problem with no work items returns BSA_OK. */
bsa_status_t bsa_backward(const void* q, const void* k, const void* v, const void* out,
                          const float* lse, const void* dout, bsa_plan_t plan, void* dq, void* dk,
                          void* dv, float* delta, void* stream);

/* bsa_backward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving or training loops, harnesses that forbid
 * hipMalloc.  It computes exactly what bsa_backward computes (the same
 * kernels), but keeps Delta in a workspace of the library's own -- a static
 * device array of 64 MiB per GPU, held until the process ends -- instead of a
 * caller buffer, and calls no allocating routine.  The caller still passes
 * every input and output; the plan (made beforehand) keeps the float32
 * partial sums of split dK/dV walks as for bsa_backward.
 *   Limit: batch * num_heads * seq_len <= 16,777,216 query rows.
 *   Concurrency: every call on one GPU shares that GPU's workspace, so calls
 *   that overlap on one GPU (other streams, other threads) race; serialise
 *   them.  The workspace keeps the last call's contents, all of which the
 *   next call overwrites before reading.
 * Errors (before anything is launched): as bsa_backward, plus
 * INVALID_ARGUMENT when the problem exceeds the limit and UNSUPPORTED on a
 * device ordinal of 64 or more; DEVICE if the workspace address cannot be
 * obtained on first use on a device. */
bsa_status_t bsa_backward_noalloc(const void* q, const void* k, const void* v, const void* out,
                                  const float* lse, const void* dout, bsa_plan_t plan, void* dq, void* dk,
                                  void* dv, void* stream);

/* Variable-length batch: the same forward, where batch entry b uses only its
 * first seq_lens[b] positions of the padded [batch][heads][seq_len][head_dim]
 * buffers.  Its positions at or beyond seq_lens[b] neither attend nor are
 * attended, and their rows of out and lse are written as empty rows (O = 0,
 * LSE = -inf).  Padding is never read, so it may hold anything.  The layout
 * rule applies to each entry as to a sequence of seq_lens[b] positions; the
 * plan is the one for seq_len (the maximum), and its tiles beyond an entry's
 * length are skipped, its last partial block masked token by token.  This is
 * the variable-length counterpart of padding to the block size (FAQ of "The
 * Only Guide You Need for Sparse Attention Kernels in Long-Context LLMs";
 * variable-length sequences in production kernels, "Sparse Attention
 * Kernels vs Full Attention Performance").
 *   seq_lens: device int32 [batch]; values are clamped to [0, seq_len].
 * Other arguments as bsa_forward.  Every kernel of bsa_forward has a
 * variable-length form (bf16 128/128 on MFMA; float32 with head_dim and block
 * 64 or 128), for static and dynamic plans.
 * Errors: as bsa_forward, plus INVALID_ARGUMENT for a NULL seq_lens or one
 * that is not device memory of the plan's device. */
bsa_status_t bsa_forward_varlen(const void* q, const void* k, const void* v, bsa_plan_t plan,
                                const int32_t* seq_lens, void* out, float* lse, void* stream);

/* Variable-length batch: the backward of bsa_forward_varlen.  Batch entry b
 * uses its first seq_lens[b] positions; the gradients of those positions are
 * the ones of a sequence of seq_lens[b] positions under the same layout
 * (the dQ walks stop at the entry's last block, the dK/dV walks skip q-blocks
 * beyond it, and its last partial block is masked token by token).  Rows of
 * dq, dk, dv and delta at or beyond seq_lens[b] are written as zeros.
 * Padding of q, k, v, out, lse and dout is never read, so it may hold
 * anything.
 *   seq_lens: device int32 [batch]; values are clamped to [0, seq_len]; the
 *             same array that produced out and lse.
 * Other arguments as bsa_backward.  Every kernel of bsa_backward has a
 * variable-length form (bf16 128/128; float32 with head_dim and block 64 or
 * 128), for static and dynamic plans.
 * Errors: as bsa_backward, plus INVALID_ARGUMENT for a NULL seq_lens or one
 * that is not device memory of the plan's device. */
bsa_status_t bsa_backward_varlen(const void* q, const void* k, const void* v, const void* out,
                                 const float* lse, const void* dout, bsa_plan_t plan, const int32_t* seq_lens,
                                 void* dq, void* dk, void* dv, float* delta, void* stream);

/* Merge P partial attention results of the same R query rows over disjoint
 * key sets into the result over their union.  Softmax attention over
 * A_1 U ... U A_P is the partial softmaxes weighted by their normalisers, so
 * per row, with m = max_p L_p:
 *   lse_out = m + ln sum_p e^{L_p - m},
 *   out     = sum_p e^{L_p - m} O_p / sum_p e^{L_p - m};
 * a part with L_p = -inf (no key) carries no weight, and a row empty in every
 * part gets out = 0, lse_out = -inf.  This is the online-softmax combination
 * of local and remote partial attention in "How Do Sparse Attention Kernels
 * Work in GPU Clusters?" (its distributed forward): what rows split into key
 * ranges, or attention sharded by keys, need afterwards.  Asynchronous on
 * `stream` (NULL = default stream) of the current device; float32 arithmetic.
 *   parts    : P >= 1
 *   rows     : R >= 0 query rows (batch * heads * seq_len for forward outputs)
 *   head_dim : D, with D * element size a multiple of 16 bytes
 *   dtype    : BSA_BF16 or BSA_F32, of o_parts and out
 *   o_parts  : device, [P][R][D] contiguous (the parts' O, stacked)
 *   lse_parts: device, float32 [P][R] (the parts' LSE, natural log)
 *   out      : device, [R][D] dtype (bf16 rounded to nearest even)
 *   lse_out  : device, float32 [R]
 * out and lse_out must not alias the inputs.  Nothing is allocated.
 * Errors (before anything is launched): INVALID_ARGUMENT for P < 1, R < 0, a
 * bad dtype or head_dim, NULL pointers (R > 0), or pointers that are not
 * device memory of the current device; DEVICE if the launch fails. */
bsa_status_t bsa_lse_merge(int32_t parts, int64_t rows, int32_t head_dim, int32_t dtype, const void* o_parts,
                           const float* lse_parts, void* out, float* lse_out, void* stream);

/* Static description of a status code (never NULL). */
const char* bsa_status_string(bsa_status_t status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* bsa_last_error(void);

/* BSA_ABI_VERSION of the built library. */
int32_t bsa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSATTN_H */
