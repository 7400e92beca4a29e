/*
 * libbsattn_probe -- measurement helper for the benchmark, separate from the
 * attention library: the sustained bf16 MFMA rate of the GPU under its power
 * limit, for the roofline that the attention kernels are reported against
 * beside the published peak.
 */
#ifndef BSATTN_PROBE_H
#define BSATTN_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Launch `workgroups` workgroups of 4 waves on `stream` (a hipStream_t; NULL =
 * default), each wave running `iters` iterations of 4 independent
 * v_mfma_f32_32x32x16_bf16 chains on register operands (no memory traffic),
 * and writing one float per thread to the device buffer `out` (at least
 * workgroups * 256 floats, caller-owned) so the chains are not removed.
 * Asynchronous.  Returns 0, 1 for a bad argument, 4 if the launch failed. */
int32_t bsa_probe_mfma(int64_t iters, int32_t workgroups, float* out, void* stream);

/* FLOPs of one bsa_probe_mfma call with these arguments. */
double bsa_probe_mfma_flops(int64_t iters, int32_t workgroups);

#ifdef __cplusplus
}
#endif

#endif /* BSATTN_PROBE_H */
