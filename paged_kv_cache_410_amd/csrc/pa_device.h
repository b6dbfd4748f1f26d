// Device-side building blocks shared by the decode kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kWave = 64;
constexpr int kBlock = 16;  // tokens per KV block
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- bf16 bits
// bf16 -> fp32 is exact: the 16 stored bits are the high half of a binary32.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16 pair (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// 16-bit halves of two words: (x.lo, y.lo) and (x.hi, y.hi).
__device__ __forceinline__ uint32_t pack_lo16(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi16(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x07060302u);
}
__device__ __forceinline__ uint32_t word(const uint4& u, int k) {
  return k == 0 ? u.x : k == 1 ? u.y : k == 2 ? u.z : u.w;
}
__device__ __forceinline__ uint32_t word(const uint2& u, int k) { return k == 0 ? u.x : u.y; }

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ---------------------------------------------------------------- cross-lane
// DPP lane permutations inside a row of 16 lanes.
enum : int {
  kDppXor1 = 0xB1,        // quad_perm [1,0,3,2]
  kDppXor2 = 0x4E,        // quad_perm [2,3,0,1]
  kDppHalfMirror = 0x141, // lane i <-> 7-i within each half-row of 8
  kDppMirror = 0x140,     // lane i <-> 15-i within each row of 16
};

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xf, 0xf, false));
}

// The gfx950 permlane swaps exchange rows (16 lanes) between two registers.
// Fed the same value twice they return, in some order, a lane's own value and
// that of its partner lane l ^ 16 (permlane16) or l ^ 32 (permlane32). Every
// use below combines the two symmetrically (sum, max, softmax merge), so which
// of the pair is "own" never matters.
struct LanePair {
  float a, b;
};
__device__ __forceinline__ LanePair pair16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ LanePair pair32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// Sum over aligned groups of N consecutive lanes (N in 4, 8, 16, 32, 64); every lane gets it.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group size");
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  if constexpr (N >= 8) x += dpp<kDppHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kDppMirror>(x);
  if constexpr (N >= 32) {
    LanePair p = pair16(x);
    x = p.a + p.b;
  }
  if constexpr (N >= 64) {
    LanePair p = pair32(x);
    x = p.a + p.b;
  }
  return x;
}

// Max over aligned groups of N consecutive lanes (N = 8 or 16), as group_sum.
template <int N>
__device__ __forceinline__ float group_max(float x) {
  static_assert(N == 8 || N == 16, "group size");
  x = fmaxf(x, dpp<kDppXor1>(x));
  x = fmaxf(x, dpp<kDppXor2>(x));
  x = fmaxf(x, dpp<kDppHalfMirror>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp<kDppMirror>(x));
  return x;
}

// Max over the 4 rows of the wave (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float rows_max(float x) {
  LanePair p = pair16(x);
  x = fmaxf(p.a, p.b);
  p = pair32(x);
  return fmaxf(p.a, p.b);
}
// NaN-propagating maximum: v_maximum3_f32, with no quieting of the inputs
// first (fmaxf spends one v_max_f32 per operand on that).
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float rows_vmax(float x) {
  LanePair p = pair16(x);
  x = vmax(p.a, p.b);
  p = pair32(x);
  return vmax(p.a, p.b);
}
// rows_vmax of two values at once, in three lane swaps instead of four. This
// one depends on the order of the swaps' results, as measured on gfx950 with
// rows (16-lane groups) a0..a3 of the first operand and b0..b3 of the second:
// permlane16_swap returns [a0 b0 a2 b2] and [a1 b1 a3 b3], permlane32_swap
// [a0 a1 b0 b1] and [a2 a3 b2 b3]. So the maximum of the first swap's
// results is [a01 b01 a23 b23], folding it over the halves gives
// [A B A B], and a last swap of that with itself returns A and B on all
// four rows, in that order.
__device__ __forceinline__ void rows_vmax2(float a, float b, float& ma, float& mb) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  const float c = vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const LanePair p = pair32(c);
  const float d = vmax(p.a, p.b);
  const LanePair q = pair16(d);
  ma = q.a;
  mb = q.b;
}
__device__ __forceinline__ float rows_sum(float x) {
  LanePair p = pair16(x);
  x = p.a + p.b;
  p = pair32(x);
  return p.a + p.b;
}

// fast 2^x (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Online-softmax merge of two partial states over disjoint token sets, in the
// log2 domain: (m, l, o) with o unnormalised. Empty states carry m = -inf.
struct SoftmaxScales {
  float a, b, m;
};
__device__ __forceinline__ SoftmaxScales merge_scales(float m_a, float m_b) {
  const float m = fmaxf(m_a, m_b);
  const float m_use = (m == -INFINITY) ? 0.0f : m;
  return {exp2_fast(m_a - m_use), exp2_fast(m_b - m_use), m};
}

// Non-temporal-free plain 16-byte global load/store helpers.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// The index of this thread's wave in its workgroup, as a wave-uniform value
// (so branches on it stay scalar and the compiler can count loads in flight
// exactly instead of draining them at every join).
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
}

// ------------------------------------------------------- workgroup mapping
// Workgroups of one dispatch go round-robin to the 8 XCDs (workgroup L runs on
// XCD L % 8), and each XCD has its own L2. With kSwizzle the grid's
// coordinates are taken from a remapped linear id so that each XCD runs one
// contiguous range of work items instead of every eighth one: workgroups that
// read the same K/V (neighbours in grid order) then share one L2. Decode
// workgroups share nothing and keep the plain order (PA_XCD_SWIZZLE=1 remaps
// them too, for measurement).
#ifndef PA_XCD_SWIZZLE
#define PA_XCD_SWIZZLE 0
#endif
constexpr int kXcds = 8;
struct GridPos {
  int x, y, z;
};
template <bool kSwizzle = (PA_XCD_SWIZZLE != 0)>
__device__ __forceinline__ GridPos grid_pos() {
  if constexpr (!kSwizzle) {
    return {(int)blockIdx.x, (int)blockIdx.y, (int)blockIdx.z};
  } else {
    const uint32_t X = gridDim.x, Y = gridDim.y;
    const uint32_t n = X * Y * gridDim.z;
    const uint32_t L = blockIdx.x + X * (blockIdx.y + Y * blockIdx.z);
    const uint32_t xcd = L % kXcds, j = L / kXcds, q = n / kXcds, r = n % kXcds;
    const uint32_t w = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + j;
    return {(int)(w % X), (int)((w / X) % Y), (int)(w / (X * Y))};
  }
}

// Groups of S consecutive work items (in grid order) that read the same data
// run on one XCD, and successive groups go round-robin over the XCDs: the
// j-th workgroup dispatched to XCD k takes member j % S of group
// k + 8 * (j / S). Items past the last whole round of 8 groups keep their
// place. A bijection on [0, n); S must divide gridDim.x.
__device__ __forceinline__ GridPos grid_pos_grouped(uint32_t S) {
  const uint32_t X = gridDim.x, Y = gridDim.y;
  const uint32_t n = X * Y * gridDim.z;
  const uint32_t L = blockIdx.x + X * (blockIdx.y + Y * blockIdx.z);
  const uint32_t round = kXcds * S;
  uint32_t w = L;
  if (L < n / round * round) {
    const uint32_t k = L % kXcds, j = L / kXcds;
    w = (k + kXcds * (j / S)) * S + j % S;
  }
  return {(int)(w % X), (int)((w / X) % Y), (int)(w / (X * Y))};
}

// ---------------------------------------------------------------- tile loads
// A buffer resource over `bytes` bytes at `base` (raw buffer, no stride; the
// word-3 value is the gfx9-family one for untyped dword loads). A load whose
// offset falls outside [0, bytes) is dropped by the hardware range check and
// returns zeros without touching memory, so a resource of 0 bytes turns a
// tile load into a no-op that still counts as one issued load.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
// Cache policy of the K/V tile loads. Streaming (the non-temporal bit): K/V
// read once per step pass the caches by, which sustains a higher HBM rate.
// Shared (default caching): when several sequences read the same physical
// blocks (forks, beams, a prefix cache), the caches serve the repeats.
// Measured on the 13B-shape batch: streaming 256 us vs cached 288 us; on the
// copy-on-write batch: cached 183 us vs streaming 273 us.
enum class TilePolicy { kStream, kShared };
template <TilePolicy kPolicy>
__device__ __forceinline__ uint4 ld16(rsrc_t r, int off) {
  constexpr int kAux = kPolicy == TilePolicy::kStream ? 2 : 0;  // nt bit
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAux));
}
// A piece of a K/V row per lane: 16 bytes (head_dim 128: a 16-lane group
// covers a 256-byte row) or 8 bytes (head_dim 64, 128-byte rows).
template <int kBytes>
struct TilePiece;
template <>
struct TilePiece<16> {
  using type = uint4;
};
template <>
struct TilePiece<8> {
  using type = uint2;
};
template <TilePolicy kPolicy, int kBytes>
__device__ __forceinline__ typename TilePiece<kBytes>::type ld_piece(rsrc_t r, int off) {
  if constexpr (kBytes == 16) {
    return ld16<kPolicy>(r, off);
  } else {
    constexpr int kAux = kPolicy == TilePolicy::kStream ? 2 : 0;  // nt bit
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kAux));
  }
}

// The same load written by the hardware straight into LDS
// (buffer_load_dwordx4 ... lds): lane i's 16 bytes land at lds + 16 i, with
// `lds` wave-uniform; lanes outside the resource's range write zeros. Its
// completion is counted like a register load's (vmcnt).
template <TilePolicy kPolicy>
__device__ __forceinline__ void ld16_lds(rsrc_t r, void* lds, int off) {
  constexpr int kAux = kPolicy == TilePolicy::kStream ? 2 : 0;  // nt bit
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off,
                                           0, 0, kAux);
}

// Software pipeline over the blocks one wave reads: logical blocks
// first + k * stride of one block-table row, for k = k0 .. k1 - 1.
//   load(slot, b, k, exists) issue the K/V tile loads of physical block b,
//                           the wave's k-th block, into ring slot `slot`;
//                           exists == false asks for an empty load (past the
//                           wave's last block; k is then meaningless)
//   consume(slot, k)        use ring slot `slot` for the wave's k-th block
// Every step refills one slot unconditionally and only the compute is
// branched on, so the compiler sees the same loads in flight on every path
// and waits for exactly the slot it consumes (loads complete in order).
// Block ids are read from the table 64 at a time (lane j of chunk c holds the
// id of block first + (64 c + j) * stride, broadcast with readlane): no table
// read sits between two tile prefetches, where it would drain the ring.
// Tiles are prefetched DEPTH - 1 blocks ahead; the ring drains once per chunk.
//
// ids0 is chunk 0, loaded by the caller (first_chunk_ids) before it waits on
// anything else, so the table read overlaps the kernel's other start-up
// loads. A wave that starts further on (k0 > 0: the shared-prefix tail pass,
// which learns k0 only from a load of its own) still takes its ids from ids0
// when k0 < 64.
__device__ __forceinline__ int first_chunk_ids(const int32_t* row, int first, int stride, int lim,
                                               int lane) {
  const int i = first + lane * stride;
  return i < lim ? row[i] : -1;
}

template <int DEPTH, typename Load, typename Consume>
__device__ __forceinline__ void block_pipeline(const int32_t* row, int first, int stride, int k0,
                                               int k1, int lane, int ids0, Load&& load,
                                               Consume&& consume) {
  for (int c0 = k0 / kWave * kWave; c0 < k1; c0 += kWave) {
    const int ids = c0 == 0 ? ids0 : (c0 + lane < k1 ? row[first + (c0 + lane) * stride] : -1);
    const int lo = max(k0, c0) - c0;        // this chunk's first lane
    const int cn = min(kWave, k1 - c0) - lo;  // and its block count
#pragma unroll
    for (int d = 0; d < DEPTH - 1; ++d)
      load(d, __builtin_amdgcn_readlane(ids, min(lo + d, kWave - 1)), c0 + lo + d, d < cn);
    for (int j0 = 0; j0 < cn; j0 += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        const int j = j0 + d;
        const int jl = j + DEPTH - 1;
        load((d + DEPTH - 1) % DEPTH, __builtin_amdgcn_readlane(ids, min(lo + jl, kWave - 1)),
             c0 + lo + jl, jl < cn);
        if (j < cn) consume(d, c0 + lo + j);
      }
    }
  }
}

// The same pipeline over a wave's items k = 0 .. k1 - 1 of any list: item k's
// block id and a tag (what the caller needs to place it) come from
// fetch(c0, id, tag), lane j giving item c0 + j, 64 items at a time; the
// first 64 (ids0, tags0) are fetched by the caller, early. load(slot, id,
// tag, exists) and consume(slot, tag) as in block_pipeline.
template <int DEPTH, typename Fetch, typename Load, typename Consume>
__device__ __forceinline__ void list_pipeline(int k1, int lane, int ids0, int tags0, Fetch&& fetch,
                                              Load&& load, Consume&& consume) {
  for (int c0 = 0; c0 < k1; c0 += kWave) {
    int ids = ids0, tags = tags0;
    if (c0 > 0) fetch(c0, ids, tags);
    const int cn = min(kWave, k1 - c0);
#pragma unroll
    for (int d = 0; d < DEPTH - 1; ++d) {
      const int jl = min(d, kWave - 1);
      load(d, __builtin_amdgcn_readlane(ids, jl), __builtin_amdgcn_readlane(tags, jl), d < cn);
    }
    for (int j0 = 0; j0 < cn; j0 += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        const int j = j0 + d;
        const int jl = min(j + DEPTH - 1, kWave - 1);
        load((d + DEPTH - 1) % DEPTH, __builtin_amdgcn_readlane(ids, jl),
             __builtin_amdgcn_readlane(tags, jl), j + DEPTH - 1 < cn);
        if (j < cn) consume(d, __builtin_amdgcn_readlane(tags, j));
      }
    }
  }
}

}  // namespace pa
