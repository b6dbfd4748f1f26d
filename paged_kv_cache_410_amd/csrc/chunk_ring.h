// Constants and helpers of the chunk kernel's LDS ring of block pairs (which
// the waves of a workgroup fill with LDS-direct loads), and the online
// softmax's start value.
#pragma once

#include "pa_device.h"

// LDS ring slots (3 or 4 pairs of blocks).
#ifndef PA_CHUNK_RING
#define PA_CHUNK_RING 3
#endif

namespace pa {

namespace {

constexpr int kD = 128;
constexpr int kRowBytes = kD * 2;
constexpr int kTileBytes = kBlock * kRowBytes;      // one K or V tile of one block
constexpr int kSlotBytes = 4 * kTileBytes;          // a pair of blocks: K A, K B, V A, V B
constexpr int kPieceBytes = kWave * 16;             // one load instruction
constexpr int kPieces = kSlotBytes / kPieceBytes;   // per pair

// The reference max of a column before any finite logit: the lowest finite
// float rather than -inf, so that the exponents x - m need no guard against
// -inf - -inf (a column whose logits so far are all -inf gets exp2(-inf) = 0).
constexpr float kNoRef = -__FLT_MAX__;

// s_waitcnt bounding only the vector memory count (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier with no memory fence: a fence would wait for every load
// in flight, the ring's prefetches included. The empty asm statements keep
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace

}  // namespace pa
