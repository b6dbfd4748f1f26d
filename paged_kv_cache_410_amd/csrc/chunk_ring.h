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

// Geometry of the ring for bf16 rows of D elements (D = 64 or 128).
template <int D>
struct Ring {
  static_assert(D == 64 || D == 128, "head_dim");
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = kRowBytes / 16;                  // 16-byte chunks per row
  static constexpr int kTileBytes = kBlock * kRowBytes;           // one K or V tile of one block
  static constexpr int kSlotBytes = 4 * kTileBytes;               // a pair: K A, K B, V A, V B
  static constexpr int kPieceBytes = kWave * 16;                  // one load instruction
  static constexpr int kPieces = kSlotBytes / kPieceBytes;        // per pair
  static constexpr int kPiecesPerTile = kTileBytes / kPieceBytes;
  static constexpr int kRowsPerPiece = kPieceBytes / kRowBytes;

  // LDS position (in 16-byte units within its row) of chunk c of row r of a
  // K tile, and of a V tile. Swapping position and chunk gives the same map,
  // so the loads use it to pick the chunk that each lane's position holds.
  // 256-byte rows (the LDS's 64 banks span one row): K chunk c of row r at
  //   c ^ r, so the 16 rows of an operand read fall on 16 positions; V chunk
  //   c at c ^ (2 r mod 16), so any 8 consecutive rows put the chunk pairs of
  //   a transposed read on 8 different pairs of positions.
  // 128-byte rows (two rows span the banks, even rows on the lower half): K
  //   chunk c at c ^ (r / 2 mod 8), so the 8 even and the 8 odd rows of an
  //   operand read each fall on 8 positions; V chunk c at c ^ (2 (r / 2 mod
  //   4)), so the 4 even and the 4 odd rows of any 8 consecutive ones put
  //   their chunk pairs on 4 different pairs of positions.
  __device__ static __forceinline__ int k_pos(int r, int c) {
    return kChunks == 16 ? (c ^ r) & 15 : (c ^ (r >> 1)) & 7;
  }
  __device__ static __forceinline__ int v_pos(int r, int c) {
    return kChunks == 16 ? (c ^ (2 * r)) & 15 : (c ^ (2 * ((r >> 1) & 3))) & 7;
  }
};

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
