// Block-table bookkeeping kernels: slot mapping, the cache write of new K/V
// rows, and copy-on-write block copies. All three move integers or raw bits.
//
// Method: "Why OS Virtual Memory Paging Saved LLM Inference" (a8q9.cn),
// section 2 (block table from logical positions to physical blocks; blocks
// filled as tokens are generated) and section 3 (a branch writing into a
// shared block first receives a private copy of it).
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

// Largest block id whose slots all fit an int32 slot number.
constexpr int32_t kMaxSlotBlock = (INT32_MAX - (kBlock - 1)) / kBlock;

// slot = table[seq][p / 16] * 16 + p % 16, or -1 when there is no valid slot
// (a negative table entry, or one whose slots would not fit an int32).
__device__ __forceinline__ int32_t slot_of(const int32_t* __restrict__ bt,
                                           const int32_t* __restrict__ seq_ids,
                                           const int32_t* __restrict__ pos, int32_t i, int32_t B,
                                           int32_t MB) {
  const int32_t s = seq_ids ? seq_ids[i] : i;
  const int32_t p = pos[i];
  int32_t slot = -1;
  if (s >= 0 && s < B && p >= 0 && p / kBlock < MB) {
    const int32_t b = bt[(size_t)s * MB + p / kBlock];
    if (b >= 0 && b <= kMaxSlotBlock) slot = b * kBlock + p % kBlock;
  }
  return slot;
}

__global__ void slot_mapping_kernel(int32_t* __restrict__ out, const int32_t* __restrict__ bt,
                                    const int32_t* __restrict__ seq_ids,
                                    const int32_t* __restrict__ pos, int32_t T, int32_t B,
                                    int32_t MB) {
  const int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T) return;
  out[i] = slot_of(bt, seq_ids, pos, i, B, MB);
}

// Cache write stores. A write of at least PA_WRITE_NT_MIN_BYTES (K and V rows
// together) uses non-temporal stores: with default stores the rows stay dirty
// in the caches and their write-back to HBM overlaps whatever runs next, the
// step's attention. On the copy-on-write batch (285 MB of rows per step) the
// attention took 106 us after the write against 92 us without it; with
// non-temporal stores 96 us, and the whole step 200 us against 207. A smaller
// write stays cached (about half of the 256 MB last-level cache or less),
// where the attention that follows reads it back: on the 64/8-head
// copy-on-write batch (71 MB) its tail pass took 21.3 us after default stores
// and 24.6 us after non-temporal ones.
#ifndef PA_WRITE_NT_MIN_BYTES
#define PA_WRITE_NT_MIN_BYTES (128ll << 20)
#endif
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
template <bool kNT>
__device__ __forceinline__ void store_row_chunk(uint4* p, const uint4& v) {
  if constexpr (kNT)
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, v), reinterpret_cast<u32x4_t*>(p));
  else
    *p = v;
}

// Pool index of 16-byte chunk c of head g's row in slot `slot`.
__device__ __forceinline__ int64_t pool_chunk(int32_t slot, int32_t g, int32_t c, int32_t Hkv,
                                              int32_t chunks_per_row) {
  return (((int64_t)(slot / kBlock) * Hkv + g) * kBlock + slot % kBlock) * chunks_per_row + c;
}

// One thread per 16-byte chunk of a (token, kv head) row; K and V together.
// Source row (t, g) -> pool row (slot / 16, g, slot % 16). The source chunks
// are read before the slot is known, so both loads are in flight together.
template <bool kNT>
__global__ void write_kv_kernel(const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
                                uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
                                const int32_t* __restrict__ slots, int32_t T, int32_t Hkv,
                                int32_t chunks_per_row, int64_t n_slots) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)T * Hkv * chunks_per_row;
  if (i >= total) return;
  const uint4 kx = k_new[i];
  const uint4 vx = v_new[i];
  const int32_t c = (int32_t)(i % chunks_per_row);
  const int64_t row = i / chunks_per_row;
  const int32_t g = (int32_t)(row % Hkv);
  const int32_t t = (int32_t)(row / Hkv);
  const int32_t slot = slots[t];
  if (slot < 0 || slot >= n_slots) return;
  const int64_t dst = pool_chunk(slot, g, c, Hkv, chunks_per_row);
  store_row_chunk<kNT>(k_cache + dst, kx);
  store_row_chunk<kNT>(v_cache + dst, vx);
}

// Slot mapping and cache write in one pass: each thread derives its token's
// slot from the block table itself, then stores its chunk; the thread of
// chunk 0, head 0 also records the slot when `slots_out` is given. The result
// equals slot_mapping_kernel followed by write_kv_kernel.
template <bool kNT>
__global__ void append_kv_kernel(const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
                                 uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
                                 int32_t* __restrict__ slots_out, const int32_t* __restrict__ bt,
                                 const int32_t* __restrict__ seq_ids,
                                 const int32_t* __restrict__ pos, int32_t T, int32_t B, int32_t MB,
                                 int32_t Hkv, int32_t chunks_per_row, int64_t n_slots) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)T * Hkv * chunks_per_row;
  if (i >= total) return;
  const uint4 kx = k_new[i];
  const uint4 vx = v_new[i];
  const int32_t c = (int32_t)(i % chunks_per_row);
  const int64_t row = i / chunks_per_row;
  const int32_t g = (int32_t)(row % Hkv);
  const int32_t t = (int32_t)(row / Hkv);
  const int32_t slot = slot_of(bt, seq_ids, pos, t, B, MB);
  if (slots_out && g == 0 && c == 0) slots_out[t] = slot;
  if (slot < 0 || slot >= n_slots) return;
  const int64_t dst = pool_chunk(slot, g, c, Hkv, chunks_per_row);
  store_row_chunk<kNT>(k_cache + dst, kx);
  store_row_chunk<kNT>(v_cache + dst, vx);
}

// Copy-on-write copies: grid.y = pair, grid.z = 0 (K) / 1 (V); workgroup x
// of a pair takes U consecutive 4 KiB pieces of the block (256 threads x 16 B
// each) and issues all its loads before its first store, so the whole copy is
// in flight at once and each workgroup makes one round trip.
#ifndef PA_COPY_UNROLL
#define PA_COPY_UNROLL 4
#endif
#ifndef PA_COPY_NT
#define PA_COPY_NT 0
#endif
constexpr int kCopyThreads = 256;
template <int U, bool kNT>
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    u32x4_t* __restrict__ k_cache, u32x4_t* __restrict__ v_cache, const int32_t* __restrict__ pairs,
    int32_t NB, int64_t chunks_per_block) {
  const int32_t src = pairs[2 * blockIdx.y];
  const int32_t dst = pairs[2 * blockIdx.y + 1];
  if (src < 0 || src >= NB || dst < 0 || dst >= NB) return;
  u32x4_t* base = blockIdx.z ? v_cache : k_cache;
  const u32x4_t* from = base + (int64_t)src * chunks_per_block;
  u32x4_t* to = base + (int64_t)dst * chunks_per_block;
  const int64_t i0 = (int64_t)blockIdx.x * (U * kCopyThreads) + threadIdx.x;
  u32x4_t v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = i0 + u * kCopyThreads;
    if (i < chunks_per_block) v[u] = kNT ? __builtin_nontemporal_load(from + i) : from[i];
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = i0 + u * kCopyThreads;
    if (i < chunks_per_block) {
      if (kNT)
        __builtin_nontemporal_store(v[u], to + i);
      else
        to[i] = v[u];
    }
  }
}

hipError_t launch_slot_mapping(int32_t* out, const int32_t* bt, const int32_t* seq_ids,
                               const int32_t* pos, int32_t T, int32_t B, int32_t MB,
                               hipStream_t stream) {
  const int threads = 256;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3((T + threads - 1) / threads), dim3(threads), 0,
                     stream, out, bt, seq_ids, pos, T, B, MB);
  return hipGetLastError();
}

hipError_t launch_write_kv(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                           const int32_t* slots, int32_t T, int32_t NB, int32_t Hkv,
                           int32_t row_bytes, hipStream_t stream) {
  const int32_t chunks = row_bytes / 16;
  const int64_t total = (int64_t)T * Hkv * chunks;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  const bool nt = 2 * total * 16 >= PA_WRITE_NT_MIN_BYTES;
  hipLaunchKernelGGL(nt ? write_kv_kernel<true> : write_kv_kernel<false>, dim3((unsigned)blocks),
                     dim3(threads), 0, stream, (const uint4*)k_new, (const uint4*)v_new,
                     (uint4*)k_cache, (uint4*)v_cache, slots, T, Hkv, chunks,
                     (int64_t)NB * kBlock);
  return hipGetLastError();
}

hipError_t launch_append_kv(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                            int32_t* slots_out, const int32_t* bt, const int32_t* seq_ids,
                            const int32_t* pos, int32_t T, int32_t B, int32_t MB, int32_t NB,
                            int32_t Hkv, int32_t row_bytes, hipStream_t stream) {
  const int32_t chunks = row_bytes / 16;
  const int64_t total = (int64_t)T * Hkv * chunks;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  const bool nt = 2 * total * 16 >= PA_WRITE_NT_MIN_BYTES;
  hipLaunchKernelGGL(nt ? append_kv_kernel<true> : append_kv_kernel<false>, dim3((unsigned)blocks),
                     dim3(threads), 0, stream, (const uint4*)k_new, (const uint4*)v_new,
                     (uint4*)k_cache, (uint4*)v_cache, slots_out, bt, seq_ids, pos, T, B, MB, Hkv,
                     chunks, (int64_t)NB * kBlock);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t n,
                              int32_t NB, size_t block_bytes, hipStream_t stream) {
  constexpr int U = PA_COPY_UNROLL;
  const int64_t chunks = (int64_t)(block_bytes / 16);
  const int64_t gx = (chunks + U * kCopyThreads - 1) / (U * kCopyThreads);
  hipLaunchKernelGGL((copy_blocks_kernel<U, PA_COPY_NT != 0>), dim3((unsigned)gx, (unsigned)n, 2),
                     dim3(kCopyThreads), 0, stream, (u32x4_t*)k_cache, (u32x4_t*)v_cache, pairs,
                     NB, chunks);
  return hipGetLastError();
}

}  // namespace pa
