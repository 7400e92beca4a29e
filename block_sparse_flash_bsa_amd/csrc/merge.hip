// Merging partial attention results over disjoint key sets of the same
// queries (bsa_lse_merge).  Softmax attention over A_1 U ... U A_P is the
// partial softmaxes over each A_p weighted by their normalisers, so with the
// parts' natural-log LSEs L_p:
//   LSE = m + ln sum_p e^{L_p - m}  (m = max_p L_p),
//   O   = sum_p e^{L_p - m} O_p / sum_p e^{L_p - m};
// a part with L_p = -inf (no key) carries no weight, and a row empty in every
// part is O = 0, LSE = -inf, as the forward writes it.  This is the
// online-softmax combination of local and remote partial attention in "How Do
// Sparse Attention Kernels Work in GPU Clusters?" (its distributed forward),
// and what split rows or key-sharded attention need.
//
// HBM-bound: each part's O is read once and the result written once.  One
// thread per 16-byte chunk of an output row (8 bf16 or 4 float32 values),
// consecutive threads on consecutive chunks, so every load and store is a
// whole 16 bytes and a wave covers whole rows; the row's P LSEs are read by
// every thread of the row (cache hits after the first).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "internal.h"

namespace bsa {
namespace {

constexpr int kMergeThreads = 256;
constexpr float kMergeLog2e = 1.4426950408889634f;
constexpr float kMergeLn2 = 0.6931471805599453f;
typedef uint32_t m_u32x4 __attribute__((ext_vector_type(4)));
typedef float m_f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const uint16_t x = __builtin_bit_cast(uint16_t, static_cast<__bf16>(a));
  const uint16_t y = __builtin_bit_cast(uint16_t, static_cast<__bf16>(b));
  return uint32_t(x) | (uint32_t(y) << 16);
}

template <bool kBf16>
__global__ __launch_bounds__(kMergeThreads) void lse_merge_kernel(const unsigned char* __restrict__ o_parts,
                                                                  const float* __restrict__ lse_parts,
                                                                  unsigned char* __restrict__ out,
                                                                  float* __restrict__ lse_out, int parts,
                                                                  int64_t rows, int cpr) {
  const int64_t c = int64_t(blockIdx.x) * kMergeThreads + threadIdx.x;
  if (c >= rows * cpr) return;
  const int64_t r = c / cpr;
  float m = -INFINITY;
  for (int q = 0; q < parts; ++q) m = fmaxf(m, lse_parts[int64_t(q) * rows + r]);
  constexpr int kE = kBf16 ? 8 : 4;
  float acc[kE];
#pragma unroll
  for (int e = 0; e < kE; ++e) acc[e] = 0.f;
  float s = 0.f;
  if (m > -INFINITY) {
    for (int q = 0; q < parts; ++q) {
      const float w = __builtin_amdgcn_exp2f((lse_parts[int64_t(q) * rows + r] - m) * kMergeLog2e);
      s += w;
      const m_u32x4 x = *reinterpret_cast<const m_u32x4*>(o_parts + (int64_t(q) * rows * cpr + c) * 16);
      if constexpr (kBf16) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          acc[2 * u] = fmaf(w, __uint_as_float(x[u] << 16), acc[2 * u]);
          acc[2 * u + 1] = fmaf(w, __uint_as_float(x[u] & 0xffff0000u), acc[2 * u + 1]);
        }
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u] = fmaf(w, __uint_as_float(x[u]), acc[u]);
      }
    }
  }
  const float inv = s > 0.f ? 1.f / s : 0.f;
  if constexpr (kBf16) {
    m_u32x4 y;
#pragma unroll
    for (int u = 0; u < 4; ++u) y[u] = pack_bf16(acc[2 * u] * inv, acc[2 * u + 1] * inv);
    *reinterpret_cast<m_u32x4*>(out + c * 16) = y;
  } else {
    *reinterpret_cast<m_f32x4*>(out + c * 16) = m_f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
  }
  if (c == r * cpr) lse_out[r] = s > 0.f ? m + log2f(s) * kMergeLn2 : -INFINITY;
}

bool on_device(const void* ptr, int dev) {
  hipPointerAttribute_t attr{};
  if (hipPointerGetAttributes(&attr, ptr) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return attr.type == hipMemoryTypeDevice && attr.device == dev;
}

}  // namespace
}  // namespace bsa

extern "C" bsa_status_t bsa_lse_merge(int32_t parts, int64_t rows, int32_t head_dim, int32_t dtype,
                                      const void* o_parts, const float* lse_parts, void* out, float* lse_out,
                                      void* stream) {
  using namespace bsa;
  clear_error();
  if (parts < 1) return fail(BSA_ERR_INVALID_ARGUMENT, "parts must be >= 1 (got %d)", parts);
  if (rows < 0) return fail(BSA_ERR_INVALID_ARGUMENT, "rows must be >= 0 (got %lld)", (long long)rows);
  if (dtype != BSA_BF16 && dtype != BSA_F32)
    return fail(BSA_ERR_INVALID_ARGUMENT, "dtype must be BSA_BF16 or BSA_F32 (got %d)", dtype);
  const int64_t esize = dtype == BSA_BF16 ? 2 : 4;
  if (head_dim < 1 || (int64_t(head_dim) * esize) % 16 != 0)
    return fail(BSA_ERR_INVALID_ARGUMENT, "head_dim * element size must be a positive multiple of 16 bytes (got %d)",
                head_dim);
  const int cpr = int(int64_t(head_dim) * esize / 16);
  const int64_t chunks = rows * cpr;
  if (rows > 0 && chunks / cpr != rows) return fail(BSA_ERR_INVALID_ARGUMENT, "rows * head_dim overflows");
  if ((chunks + kMergeThreads - 1) / kMergeThreads > int64_t(INT32_MAX))
    return fail(BSA_ERR_INVALID_ARGUMENT, "problem too large: %lld chunks", (long long)chunks);
  if (rows == 0) return BSA_OK;
  if (!o_parts || !lse_parts || !out || !lse_out)
    return fail(BSA_ERR_INVALID_ARGUMENT, "o_parts, lse_parts, out and lse_out must all be non-NULL");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(BSA_ERR_DEVICE, "hipGetDevice failed");
  for (const void* ptr : {o_parts, static_cast<const void*>(lse_parts), static_cast<const void*>(out),
                          static_cast<const void*>(lse_out)})
    if (!on_device(ptr, dev))
      return fail(BSA_ERR_INVALID_ARGUMENT, "o_parts, lse_parts, out and lse_out must be device memory of device %d",
                  dev);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned grid = unsigned((chunks + kMergeThreads - 1) / kMergeThreads);
  if (dtype == BSA_BF16)
    hipLaunchKernelGGL(lse_merge_kernel<true>, dim3(grid), dim3(kMergeThreads), 0, s,
                       static_cast<const unsigned char*>(o_parts), lse_parts, static_cast<unsigned char*>(out),
                       lse_out, parts, rows, cpr);
  else
    hipLaunchKernelGGL(lse_merge_kernel<false>, dim3(grid), dim3(kMergeThreads), 0, s,
                       static_cast<const unsigned char*>(o_parts), lse_parts, static_cast<unsigned char*>(out),
                       lse_out, parts, rows, cpr);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(BSA_ERR_DEVICE, "merge launch failed: %s", hipGetErrorString(err));
  return BSA_OK;
}
