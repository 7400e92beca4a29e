// Launch queues of the tile kernels (forward, dQ, dK/dV).
//
// The XCDs of one chip run the same work a few percent apart, and a launch
// ends with its slowest XCD.  So the last rows of every XCD's run of launch
// slots (slot s runs on XCD s % 8) are left to queue workgroups, launched
// after the slots that run one workgroup each: each claims the next slot of
// its own XCD's queue, or when that is empty, of the queue with the most
// slots left, so an XCD that runs ahead takes over the end of a slower one.
// Queue x holds slots static_slots + 8 t + x for t < tail_len[x].  Which
// workgroup runs a slot does not change what it computes.
//
// The counters live in plan memory, one set per call; every access is a
// system-scope atomic, which bypasses the XCDs' own L2 caches, so all XCDs
// see one counter.  Each queue workgroup also counts itself done; the last
// one clears the set for the call that next uses it (every claim of its call
// is made by then), so no extra kernel or memset is needed.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.h"

namespace bsa {

struct LaunchQueue {
  int32_t static_slots;      // workgroups below run their own slot
  int32_t dyn_total;         // queue workgroups launched after them
  const int32_t* tail_len;   // device [8]: slots in each XCD's queue
  int32_t* cnt;              // device [9]: this call's queue counters, then its done counter
};

// Wave 0 of a queue workgroup: the slot it claims, or -1 when every queue is
// empty.  The claim on its own queue is one atomic add; after that, lanes
// 0..7 read the 8 counters and lane 0 claims on the fullest queue.  A claim
// that comes too late leaves that queue seen empty, so at most 8 fail before
// a slot is claimed or every queue is seen empty.  Wave-uniform result.
__device__ inline int queue_claim(const LaunchQueue& lq) {
  const int lane = threadIdx.x & 63;
  const int x = blockIdx.x & 7;
  int t0 = 0;
  if (lane == 0) t0 = __hip_atomic_fetch_add(lq.cnt + x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  t0 = __shfl(t0, 0);
  if (t0 < lq.tail_len[x]) return lq.static_slots + 8 * t0 + x;
  for (int tries = 0; tries <= 8; ++tries) {
    int rem = -1, who = lane;
    if (lane < 8) {
      const int q = (x + lane) & 7;
      rem = lq.tail_len[q] - __hip_atomic_load(lq.cnt + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    // The fullest queue (lowest lane on ties); lanes 0..7 reduce among themselves.
#pragma unroll
    for (int off = 4; off >= 1; off >>= 1) {
      const int orem = __shfl_xor(rem, off), owho = __shfl_xor(who, off);
      if (orem > rem || (orem == rem && owho < who)) {
        rem = orem;
        who = owho;
      }
    }
    if (__shfl(rem, 0) <= 0) return -1;
    const int q = (x + __shfl(who, 0)) & 7;
    int t = 0;
    if (lane == 0) t = __hip_atomic_fetch_add(lq.cnt + q, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    t = __shfl(t, 0);
    if (t < lq.tail_len[q]) return lq.static_slots + 8 * t + q;
  }
  return -1;
}

// The whole workgroup: the slot it runs (its own below static_slots, else a
// claimed one; -1 for none), the same in every lane.  s_slot is a __shared__
// int of the kernel; done receives thread 0's done ticket (queue workgroups).
// Every thread of the workgroup must call this once, at the start.
__device__ inline int queue_slot(const LaunchQueue& lq, int* s_slot, int& done) {
  done = 0;
  if (int(blockIdx.x) < lq.static_slots) return int(blockIdx.x);
  if (threadIdx.x < 64) {
    const int s = queue_claim(lq);
    if (threadIdx.x == 0) {
      *s_slot = s;
      done = __hip_atomic_fetch_add(lq.cnt + 8, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*s_slot);
}

// At the end of a queue workgroup (any thread may call it; thread 0 acts):
// the last one to count itself done clears the call's counters.
__device__ inline void queue_release(const LaunchQueue& lq, int done) {
  if (int(blockIdx.x) >= lq.static_slots && threadIdx.x == 0 && done == lq.dyn_total - 1)
    for (int x = 0; x < 9; ++x) __hip_atomic_store(lq.cnt + x, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Host: the queue of one launch of kind k (0: forward or dQ over `work`,
// 1: dK/dV over the descriptors), with the next counter set in turn; a
// launch without a queue runs every slot as its own workgroup.
inline LaunchQueue launch_queue(Plan& P, int k) {
  LaunchQueue lq;
  lq.static_slots = int32_t(P.queue_static[k]);
  lq.dyn_total = int32_t(8 * P.queue_dyn_per_xcd[k]);
  lq.tail_len = P.d_queue + 8 * k;
  lq.cnt = nullptr;
  if (lq.dyn_total > 0) {
    const uint32_t set = P.queue_launches.fetch_add(1, std::memory_order_relaxed) % kQueueCounterSets;
    lq.cnt = P.d_queue + 16 + 16 * set;
  }
  return lq;
}

}  // namespace bsa
