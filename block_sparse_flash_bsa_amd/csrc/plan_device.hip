// Device-side planner for dynamic plans: a block bitmap in device memory ->
// the per-q-block CSR of key blocks the forward walks, with FULL/PARTIAL
// flags, without a round trip through the host.
//
// The CSR is the same as the host planner's for a bitmap layout: tile (i, j)
// of layout head hl is an entry iff bitmap[hl][i][j] != 0 and, for a causal
// layout, j <= i; the diagonal tile of a causal layout is PARTIAL (the
// token-exact causal cut), every other entry FULL.  Entries are ascending in
// j.  Three kernels: count the entries of each row, scan the counts into row
// offsets, write each row's entries.  The per-query-block lists follow step
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

constexpr int kRowThreads = 256;    // threads per row (4 waves)
constexpr int kScanThreads = 1024;

// Sum of v over the workgroup (blockDim.x == kRowThreads); all threads get it.
__device__ __forceinline__ int block_sum(int v, int* red) {
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) v += __shfl_xor(v, w);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  const int total = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return total;
}

// counts[row] = entries of row (layout head * nb + i).
__global__ __launch_bounds__(kRowThreads) void count_rows(const uint8_t* __restrict__ bm, int nb, int causal,
                                                          int32_t* __restrict__ counts) {
  __shared__ int red[kRowThreads / 64];
  const int row = blockIdx.x;
  const int i = row % nb;
  const int jend = causal ? i + 1 : nb;
  const uint8_t* r = bm + size_t(row) * nb;
  int c = 0;
  for (int j = threadIdx.x; j < jend; j += kRowThreads) c += r[j] != 0;
  const int total = block_sum(c, red);
  if (threadIdx.x == 0) counts[row] = total;
}

// rows[row] = {exclusive prefix of counts, counts[row]}; *d_nnz = total.
// One workgroup; thread t owns a contiguous run of rows.
__global__ __launch_bounds__(kScanThreads) void scan_rows(const int32_t* __restrict__ counts, int n,
                                                          RowDesc* __restrict__ rows, int64_t* d_nnz) {
  __shared__ int64_t part[kScanThreads];
  const int t = threadIdx.x;
  const int per = (n + kScanThreads - 1) / kScanThreads;
  const int a = min(n, t * per), b = min(n, a + per);
  int64_t s = 0;
  for (int x = a; x < b; ++x) s += counts[x];
  part[t] = s;
  __syncthreads();
  // Inclusive Hillis-Steele scan of the per-thread sums.
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int64_t add = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += add;
    __syncthreads();
  }
  int64_t start = part[t] - s;
  for (int x = a; x < b; ++x) {
    const int32_t c = counts[x];
    rows[x] = {int32_t(start), c};
    start += c;
  }
  if (t == kScanThreads - 1 && d_nnz) *d_nnz = part[t];
}

// The entries of each row, ascending: entry = (j << 1) | partial.
__global__ __launch_bounds__(kRowThreads) void fill_rows(const uint8_t* __restrict__ bm, int nb, int causal,
                                                         const RowDesc* __restrict__ rows,
                                                         int32_t* __restrict__ entries) {
  __shared__ int wsum[kRowThreads / 64];
  const int row = blockIdx.x;
  const int i = row % nb;
  const int jend = causal ? i + 1 : nb;
  const uint8_t* r = bm + size_t(row) * nb;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t* out = entries + rows[row].start;
  int base = 0;
  for (int j0 = 0; j0 < jend; j0 += kRowThreads) {
    const int j = j0 + threadIdx.x;
    const bool on = j < jend && r[j] != 0;
    const uint64_t m = __ballot(on);
    const int below = __popcll(m & ((uint64_t(1) << lane) - 1));
    if (lane == 0) wsum[wave] = __popcll(m);
    __syncthreads();
    int off = base;
    for (int w = 0; w < wave; ++w) off += wsum[w];
    if (on) out[off + below] = (j << 1) | ((causal && j == i) ? 1 : 0);
    base += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
}

// The transposed CSR for the backward: counts[col] = entries of column
// (layout head * nb + j), i.e. the q-blocks i with bitmap[hl][i][j] != 0 (and
// i >= j for a causal layout).  The column is read with stride nb.
__global__ __launch_bounds__(kRowThreads) void count_cols(const uint8_t* __restrict__ bm, int nb, int causal,
                                                          int32_t* __restrict__ counts) {
  __shared__ int red[kRowThreads / 64];
  const int col = blockIdx.x;
  const int j = col % nb;
  const uint8_t* c0 = bm + size_t(col / nb) * nb * nb + j;
  int c = 0;
  for (int i = (causal ? j : 0) + threadIdx.x; i < nb; i += kRowThreads) c += c0[size_t(i) * nb] != 0;
  const int total = block_sum(c, red);
  if (threadIdx.x == 0) counts[col] = total;
}

// The entries of each column, ascending in i: entry = (i << 1) | partial.
__global__ __launch_bounds__(kRowThreads) void fill_cols(const uint8_t* __restrict__ bm, int nb, int causal,
                                                         const RowDesc* __restrict__ cols,
                                                         int32_t* __restrict__ entries) {
  __shared__ int wsum[kRowThreads / 64];
  const int col = blockIdx.x;
  const int j = col % nb;
  const uint8_t* c0 = bm + size_t(col / nb) * nb * nb + j;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t* out = entries + cols[col].start;
  int base = 0;
  for (int i0 = causal ? j : 0; i0 < nb; i0 += kRowThreads) {
    const int i = i0 + threadIdx.x;
    const bool on = i < nb && c0[size_t(i) * nb] != 0;
    const uint64_t m = __ballot(on);
    const int below = __popcll(m & ((uint64_t(1) << lane) - 1));
    if (lane == 0) wsum[wave] = __popcll(m);
    __syncthreads();
    int off = base;
    for (int w = 0; w < wave; ++w) off += wsum[w];
    if (on) out[off + below] = (i << 1) | ((causal && i == j) ? 1 : 0);
    base += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
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
  hipLaunchKernelGGL(count_rows, dim3(unsigned(rows)), dim3(kRowThreads), 0, s, d_bitmap, nb, plan->causal,
                     plan->d_counts);
  hipLaunchKernelGGL(scan_rows, dim3(1), dim3(kScanThreads), 0, s, plan->d_counts, rows, d_rows, d_nnz);
  hipLaunchKernelGGL(fill_rows, dim3(unsigned(rows)), dim3(kRowThreads), 0, s, d_bitmap, nb, plan->causal,
                     d_rows, d_entries);
  // The same entries per k-block column, for the backward's dK/dV walk.
  auto* d_cols = const_cast<RowDesc*>(plan->d_cols);
  auto* d_entries_t = const_cast<int32_t*>(plan->d_entries_t);
  hipLaunchKernelGGL(count_cols, dim3(unsigned(rows)), dim3(kRowThreads), 0, s, d_bitmap, nb, plan->causal,
                     plan->d_counts);
  hipLaunchKernelGGL(scan_rows, dim3(1), dim3(kScanThreads), 0, s, plan->d_counts, rows, d_cols, nullptr);
  hipLaunchKernelGGL(fill_cols, dim3(unsigned(rows)), dim3(kRowThreads), 0, s, d_bitmap, nb, plan->causal,
                     d_cols, d_entries_t);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(BSA_ERR_DEVICE, "planner launch failed: %s", hipGetErrorString(err));
  return BSA_OK;
}

extern "C" bsa_status_t bsa_plan_read_csr(bsa_plan_t plan, int32_t layout_head, int32_t* row_ptr,
                                          int32_t* col_idx, uint8_t* flags, int64_t capacity, int64_t* nnz) {
  using namespace bsa;
  clear_error();
  if (!plan || !row_ptr || !nnz || (capacity > 0 && (!col_idx || !flags)))
    return fail(BSA_ERR_INVALID_ARGUMENT, "NULL argument to bsa_plan_read_csr");
  if (!plan->dynamic) return fail(BSA_ERR_INVALID_ARGUMENT, "plan was not made by bsa_plan_dynamic");
  if (layout_head < 0 || layout_head >= plan->layout_heads)
    return fail(BSA_ERR_INVALID_ARGUMENT, "layout_head %d out of range [0, %d)", layout_head,
                plan->layout_heads);
  const int nb = plan->nb;
  std::vector<RowDesc> rd(nb);
  if (hipDeviceSynchronize() != hipSuccess ||
      (nb && hipMemcpy(rd.data(), plan->d_rows + size_t(layout_head) * nb, nb * sizeof(RowDesc),
                       hipMemcpyDeviceToHost) != hipSuccess))
    return fail(BSA_ERR_DEVICE, "reading the device CSR failed: %s", hipGetErrorString(hipGetLastError()));
  const int64_t first = nb ? rd[0].start : 0;
  const int64_t count = nb ? int64_t(rd[nb - 1].start) + rd[nb - 1].count - first : 0;
  if (capacity < count)
    return fail(BSA_ERR_INVALID_ARGUMENT, "capacity %lld is below the head's %lld entries",
                (long long)capacity, (long long)count);
  std::vector<int32_t> en(static_cast<size_t>(count));
  if (count && hipMemcpy(en.data(), plan->d_entries + first, size_t(count) * sizeof(int32_t),
                         hipMemcpyDeviceToHost) != hipSuccess)
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
