// Device pieces shared by the bf16 and the FP8 attention kernels: the persistent work queues
// and the constants of the raw buffer loads and counter waits.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.h"

namespace wa {
namespace {

// s_waitcnt with vmcnt = 0 (lgkmcnt = 0) and the other counters left at their maximum.
constexpr int kVmcnt0 = 0x0F70;
constexpr int kLgkmcnt0 = 0xC07F;

// Word 3 of a raw buffer resource on gfx9 parts: 32-bit data format, no swizzle, so each
// access of a lane is range checked against num_records (word 2) and reads 0 past it.
constexpr int32_t kBufferWord3 = 0x00020000;

// Next work unit for a block on XCD `xcd`, run by one whole wave: its own XCD's queue first
// (the queue rows of the launch order: window units, then global-leg units, then -1
// padding), then the other XCDs' queues (work stealing at the end of the launch).  -1 when
// every queue is empty.  A queue counter that has passed the queue's last unit marks it
// empty; lanes 0..7 probe all eight queues at once, so a block that runs out costs two
// round trips to memory, not eight.
__device__ __forceinline__ int fetch_unit(const int32_t* __restrict__ work, int32_t* __restrict__ counters,
                                          int per_xcd, int xcd, int lane) {
  int u = -1;
  if (lane == 0) {
    const int i = atomicAdd(counters + xcd, 1);
    if (i < per_xcd) u = work[xcd * per_xcd + i];
  }
  u = __builtin_amdgcn_readfirstlane(u);
  while (u < 0) {
    const int y = lane & (kXcdCount - 1);
    const int x = xcd + y < kXcdCount ? xcd + y : xcd + y - kXcdCount;
    bool open = false;
    if (lane < kXcdCount) {
      const int c = __hip_atomic_load(counters + x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      open = c < per_xcd && work[x * per_xcd + c] >= 0;
    }
    const uint64_t m = __builtin_amdgcn_ballot_w64(open);
    if (m == 0) break;  // every queue is empty
    const int x0 = (xcd + __builtin_ctzll(m)) % kXcdCount;
    if (lane == 0) {
      const int i = atomicAdd(counters + x0, 1);
      if (i < per_xcd) u = work[x0 * per_xcd + i];
    }
    u = __builtin_amdgcn_readfirstlane(u);
  }
  return u;
}

// The last block of a persistent launch to finish resets the queue counters (kXcdCount
// queues, then the count of finished blocks) for the next launch; every block has made its
// last fetch when it counts itself finished.  Called by one thread per block.
__device__ __forceinline__ void finish_persistent(int32_t* __restrict__ counters) {
  __threadfence();
  if (atomicAdd(counters + kXcdCount, 1) == int(gridDim.x) - 1) {
    for (int x = 0; x <= kXcdCount; ++x) atomicExch(counters + x, 0);
  }
}

}  // namespace
}  // namespace wa
