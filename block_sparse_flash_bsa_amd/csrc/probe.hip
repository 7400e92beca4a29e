// MFMA throughput probe for the benchmark's roofline: the sustained bf16
// matrix rate of this GPU under its power limit, measured with the same
// instruction the attention kernels use (v_mfma_f32_32x32x16_bf16) and no
// memory traffic.  Each wave runs 4 independent accumulator chains, two waves
// per SIMD, on every CU.  Built into libbsattn_probe.so, separate from the
// attention library; only the benchmark calls it.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "bsattn_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256, 2) void mfma_probe(int64_t iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  // Operands with varied, non-zero bits (the matrix unit's power depends on
  // the data, so zeros would flatter the rate).
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(0.25f + 0.01f * float((lane * 7 + e * 3) & 31));
    b[e] = static_cast<__bf16>(-0.5f + 0.02f * float((lane * 5 + e * 11) & 31));
  }
  f32x16 c0 = f32x16{}, c1 = f32x16{}, c2 = f32x16{}, c3 = f32x16{};
  for (int64_t it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;   // keeps the chains live
}

}  // namespace

extern "C" int32_t bsa_probe_mfma(int64_t iters, int32_t workgroups, float* out, void* stream) {
  if (iters < 1 || workgroups < 1 || !out) return 1;
  hipLaunchKernelGGL(mfma_probe, dim3(unsigned(workgroups)), dim3(256), 0, static_cast<hipStream_t>(stream), iters,
                     out);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" double bsa_probe_mfma_flops(int64_t iters, int32_t workgroups) {
  // 4 waves per workgroup, 4 MFMAs per iteration, 2 * 32 * 32 * 16 FLOPs each.
  return double(workgroups) * 4.0 * 4.0 * double(iters) * 32768.0;
}
