// Host-side launch interface between the C ABI (pa_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pa_device.h"

namespace pa {

// Everything a decode kernel reads. Lengths are in elements unless noted.
struct DecodeParams {
  void* out;                    // [B][Hq][D] I/O dtype
  const void* q;                // [B][Hq][D]
  const void* k_cache;          // [NB][Hkv][16][D]
  const void* v_cache;
  const int32_t* block_tables;  // [B][MB]
  const int32_t* context_lens;  // [B]
  const int32_t* query_start;   // [B + 1] query rows per sequence, or null: one row per sequence
  float* ws_ml;                 // split only: [rows][n_parts][Hq][2] = (m, l), log2 domain
  void* ws_o;                   // split only: [rows][n_parts][Hq][D]: fp32 rows (unnormalised)
                                // when part_f32, else scaled fp16 rows (PartScale)
  int32_t B, Hq, Hkv, G, NB, MB;
  int32_t D;                    // head_dim
  int32_t ctx_limit;            // min(max_ctx, MB * 16): larger contexts are rejected
  int32_t partition;            // tokens per partition; 0 = one partition per sequence
  int32_t n_parts;              // grid extent over partitions
  int32_t max_q;                // grid bound on query rows per sequence (1 for decode)
  int32_t rows;                 // query rows in q / out (B for decode)
  int32_t n_tiles;              // MFMA: 16-column tiles per kv head (rows x heads per group)
  float qscale;                 // scale * log2(e): logits are kept in the log2 domain
  int32_t shared_kv;            // K/V tiles read through the caches (blocks shared by sequences)
  // Shared-prefix decode (pa_decode_shared), else null / 0:
  //  group pass: grid z runs over groups of consecutive sequences
  //    (group_start[j] .. group_start[j+1]-1) that share their first
  //    seq_shared[group_start[j]] tokens; every member row attends over
  //    exactly those tokens, read once for the whole group;
  //  tail pass: sequence s attends over its tokens seq_shared[s] .. ctx - 1,
  //    merges the group pass's partials of its row and writes the final row.
  //  The group pass writes partials: partition p goes to slot part_base + p.
  const int32_t* group_start;   // [n_groups + 1] (group pass)
  const int32_t* seq_shared;    // [B] shared tokens per sequence, a multiple of 16
  int32_t tail_pass;            // 1: attend from seq_shared[s] on
  int32_t fold_tails;           // group pass only: after the shared blocks, each member's own
                                // blocks too (its columns alone), and the final rows: no tail
                                // pass, no partials
  int32_t tail_shared_kv;       // fold_tails: the members' own blocks read through the caches
  int32_t n_cus;                // compute units of the device (launch shapes)
  int32_t part_base;            // first partial slot this pass writes
  int32_t always_partial;       // write partials even for a single partition
  int32_t shared_partition;     // tail pass: partition length of the group pass (0 = one)
  int32_t few_items;            // vector kernel: an unsplit grid with at most 8 items per CU
  int32_t pass_parts;           // grid y of this pass (partitions)
  int32_t pass_items;           // grid z of this pass (sequences, or groups)
  int32_t part_f32;             // partial rows are fp32 (fp32 I/O), else scaled fp16 (bf16 I/O)
};

// Slot of partial j of query row `row`, query head h (x2 floats in ws_ml, xD in
// ws_o). Partition-major within a row: the heads of one kv group, which one
// workgroup finishes together, write one contiguous range instead of a
// scattered piece per head (scattered partial stores cost several times
// their bytes in the decode kernels' time).
__device__ __forceinline__ size_t part_slot(const DecodeParams& P, size_t row, int h, int j) {
  return (row * P.n_parts + j) * P.Hq + h;
}

// Cache policy of the partial-row stores (buffer-instruction aux bits) for
// rows of 256 bytes (head_dim 128 in fp16, 64 in fp32): 16 = sc1, device
// scope. On the GQA workload (about 9 MB of fp16 rows per call, stored while
// the kernel streams 1.16 GB) the default policy costs 16 us against a timing
// probe that stores no rows (202.3 vs 186.9 us); with sc1 the call takes
// 198.1-199.5 us (nt: 199.0-199.8, sc0: 201.9). Rows of other sizes keep the
// default: 128 bytes (head_dim 64 in fp16; on the same batch at head_dim 64
// sc1 gave 121.5 us and nt 121.8 against 118.3) and 512 bytes (head_dim 128
// in fp32; on the fp32 GQA batch sc1 gave 131.3 us, nt 132.5, sc1 + nt 140.2,
// against 128.2).
#ifndef PA_PART_STORE_AUX
#define PA_PART_STORE_AUX 16
#endif
typedef unsigned int u32x4_part_t __attribute__((ext_vector_type(4)));

// Store 16 bytes at byte `off` of the partial row of (row, head h, partition
// slot j); rows are D elements of `eb` bytes. The buffer resource spans the
// Hq rows of (row, j), which are contiguous (part_slot), so offsets stay
// small whatever the workspace's size.
__device__ __forceinline__ void store_part16(const DecodeParams& P, size_t row, int h, int j,
                                             int eb, int off, const uint4& v) {
  const int64_t row_bytes = (int64_t)P.D * eb;
  char* base = static_cast<char*>(P.ws_o) + part_slot(P, row, 0, j) * row_bytes;
  if ((int64_t)P.Hq * row_bytes <= INT32_MAX) {
    const rsrc_t r = make_rsrc(base, (int)(P.Hq * row_bytes));
    const u32x4_part_t d = __builtin_bit_cast(u32x4_part_t, v);
    const int o = (int)(h * row_bytes) + off;
    if (row_bytes == 256)
      __builtin_amdgcn_raw_buffer_store_b128(d, r, o, 0, PA_PART_STORE_AUX);
    else
      __builtin_amdgcn_raw_buffer_store_b128(d, r, o, 0, 0);
  } else {
    st16(base + h * row_bytes + off, v);
  }
}

// The same for 8 bytes (the chunk kernel's fp16 rows: a lane holds 4
// consecutive dims of each 16-dim output tile).
__device__ __forceinline__ void store_part8(const DecodeParams& P, size_t row, int h, int j,
                                            int eb, int off, const uint2& v) {
  const int64_t row_bytes = (int64_t)P.D * eb;
  char* base = static_cast<char*>(P.ws_o) + part_slot(P, row, 0, j) * row_bytes;
  if ((int64_t)P.Hq * row_bytes <= INT32_MAX) {
    const rsrc_t r = make_rsrc(base, (int)(P.Hq * row_bytes));
    typedef unsigned int u32x2_part_t __attribute__((ext_vector_type(2)));
    const u32x2_part_t d = __builtin_bit_cast(u32x2_part_t, v);
    const int o = (int)(h * row_bytes) + off;
    if (row_bytes == 256)
      __builtin_amdgcn_raw_buffer_store_b64(d, r, o, 0, PA_PART_STORE_AUX);
    else
      __builtin_amdgcn_raw_buffer_store_b64(d, r, o, 0, 0);
  } else {
    *reinterpret_cast<uint2*>(base + h * row_bytes + off) = v;
  }
}

// Element type of the partial rows for I/O dtype T (float, or bf16 bits).
template <typename T>
struct PartElem {
  using type = float;
};
template <>
struct PartElem<uint16_t> {
  using type = _Float16;
};
__device__ __forceinline__ float elem_f32(float x) { return x; }
__device__ __forceinline__ float elem_f32(_Float16 x) { return (float)x; }

// A partial of bf16 attention (max m, sum l, unnormalised row o, all in the
// log2-domain state of the online softmax) is stored in fp16 as
//   z = o / c,  (m', l') = (m + log2 c, l / c),  c = l * 2^k,
// an equivalent state: raising a state's max by log2 c multiplies its weight
// 2^(m - M) in every later merge by c, which the division of o and l by c
// undoes, so the merge kernel and the tail pass take it like any other partial. o / l is a
// convex combination of V rows; with y = max |o / l| and k = floor(log2 y) - 14
// the row's largest |z| lies in [2^14, 2^15), inside fp16's normal range
// (largest finite 65504, smallest normal 2^-14) whatever the scale of V, so
// every element keeps fp16's 11-bit significand relative to the row's largest
// and the final bf16 rounding stays the dominant error. k is clamped to
// [-100, 113]: 2^-k stays a normal fp32, and l' = 2^-k <= 2^100 leaves the
// merges' fp32 sums of up to 65535 partials far from overflow (only rows
// whose every |o / l| is below 2^-114 then keep z below fp16's normal range).
// amax is the row's max |o|.
struct PartScale {
  float mul, m, l;  // store o * mul, and (m, l)
};
__device__ __forceinline__ PartScale part_scale_f16(float m, float l, float amax) {
  if (!(l > 0.0f)) return {0.0f, m, l};  // no token: zero row, weight 0
  const float y = amax / l;
  int k = (int)((__float_as_uint(y) >> 23) & 0xffu) - 127 - 14;  // floor(log2 y) - 14
  k = k < -100 ? -100 : (k > 113 ? 113 : k);
  const float inv_pow = __uint_as_float((uint32_t)(127 - k) << 23);  // 2^-k
  return {inv_pow / l, m + __builtin_amdgcn_logf(l) + (float)k, inv_pow};
}
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  const f16x2_t v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Online-softmax merge of the group pass's partials of one row into a tail
// pass's state (M, L, o: log2-domain max, sum, unnormalised dims), for the n
// dims this lane holds, starting at dim `dim0` of (row, head h). The group pass
// wrote ceil(shared / shared_partition) partials (one when not split) at
// slots 0.. of the row's n_parts.
template <typename T, int N>
__device__ __forceinline__ void merge_shared_partials(const DecodeParams& P, int shared_tokens,
                                                      size_t row, int h, int dim0, int D, float& M,
                                                      float& L, float (&o)[N]) {
  if (shared_tokens <= 0) return;
  const int bpp = P.shared_partition / 16;
  const int nps = bpp > 0 ? (shared_tokens / 16 + bpp - 1) / bpp : 1;
  for (int j = 0; j < nps && j < P.n_parts; ++j) {
    const size_t part = part_slot(P, row, h, j);
    const float mj = P.ws_ml[2 * part], lj = P.ws_ml[2 * part + 1];
    const SoftmaxScales sc = merge_scales(M, mj);
    L = L * sc.a + lj * sc.b;
    if (P.part_f32) {
      const float* oj = static_cast<const float*>(P.ws_o) + part * D + dim0;
#pragma unroll
      for (int e = 0; e < N; ++e) o[e] = o[e] * sc.a + oj[e] * sc.b;
    } else {
      const auto* oj = static_cast<const typename PartElem<T>::type*>(P.ws_o) + part * D + dim0;
#pragma unroll
      for (int e = 0; e < N; ++e) o[e] = o[e] * sc.a + elem_f32(oj[e]) * sc.b;
    }
    M = sc.m;
  }
}

// Table row and first logical block of work item s (grid z): a sequence, or,
// in the group pass, a group (whose shared blocks are read through its first
// member's table). The tail pass starts at the sequence's shared tokens. An
// out-of-range group start or shared length marks the item bad.
struct ItemStart {
  int trow, start_blk;
  bool bad;
};
__device__ __forceinline__ ItemStart item_start(const DecodeParams& P, int s) {
  ItemStart r{s, 0, false};
  if (P.group_start) {
    const int f = P.group_start[s];
    r.bad = f < 0 || f >= P.rows;
    r.trow = r.bad ? 0 : f;
  } else if (P.tail_pass) {
    const int sh = P.seq_shared[s];
    r.bad = sh < 0 || sh % 16 != 0 || sh / 16 > P.MB;
    r.start_blk = r.bad ? 0 : sh / 16;
  }
  return r;
}

// The query rows of sequence s and the context each row attends over.
// Without query_start (decode) sequence s has one row, row s. With it, the
// sequence's n rows are query_start[s] .. query_start[s+1]-1, the last n
// tokens of its context: row i sits at position ctx - n + i and attends to
// positions 0 .. ctx - n + i, so its context length is ctx - n + i + 1.
// `bad` marks a sequence whose length, row count or row bound is invalid.
// A decode row's context length is ctx itself (ctx - 1 + 0 + 1).
struct SeqRows {
  int first, n, ctx;
  bool bad;
  int n_causal;  // 1: row i attends ctx - n + i + 1 tokens; 0: every row attends ctx
  __device__ __forceinline__ int row_ctx(int i) const {
    return bad ? 0 : n_causal ? ctx - n + i + 1 : ctx;
  }
};
__device__ __forceinline__ SeqRows seq_rows(const DecodeParams& P, int s) {
  SeqRows r;
  if (P.group_start) {
    // group pass: group s; every row attends over the group's shared tokens
    // (no causal offset: n is set so that row_ctx(i) = ctx for the last row,
    // and the group kernel gives every column the same context)
    r.first = P.group_start[s];
    r.n = P.group_start[s + 1] - r.first;
    const bool rows_ok = r.n >= 1 && r.n <= P.max_q && r.first >= 0 && r.first + r.n <= P.rows;
    r.ctx = rows_ok ? P.seq_shared[r.first] : 0;
    r.bad = !rows_ok || r.ctx < 0 || r.ctx > P.ctx_limit || r.ctx % 16 != 0;
    if (!rows_ok) r.n = 0;
    r.n_causal = 0;
    return r;
  }
  r.n_causal = 1;
  r.first = s;
  r.n = 1;
  if (P.query_start) {
    r.first = P.query_start[s];
    r.n = P.query_start[s + 1] - r.first;
  }
  r.ctx = P.context_lens[s];
  // (a decode row attends over the whole context, which may be empty: zeros;
  // new tokens of a chunk must already be in the cache: n <= ctx)
  r.bad = r.ctx < 0 || r.ctx > P.ctx_limit || r.n < 0 || (P.query_start && r.n > r.ctx) ||
          r.n > P.max_q || r.first < 0 || r.first + r.n > P.rows;
  if (r.bad && (r.n < 0 || r.first < 0 || r.first + r.n > P.rows)) r.n = 0;  // no row to write
  return r;
}

hipError_t launch_slot_mapping(int32_t* out, const int32_t* bt, const int32_t* seq_ids,
                               const int32_t* pos, int32_t T, int32_t B, int32_t MB,
                               hipStream_t stream);
hipError_t launch_write_kv(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                           const int32_t* slots, int32_t T, int32_t NB, int32_t Hkv,
                           int32_t row_bytes, hipStream_t stream);
hipError_t launch_append_kv(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                            int32_t* slots_out, const int32_t* bt, const int32_t* seq_ids,
                            const int32_t* pos, int32_t T, int32_t B, int32_t MB, int32_t NB,
                            int32_t Hkv, int32_t row_bytes, hipStream_t stream);
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t n,
                              int32_t NB, size_t block_bytes, hipStream_t stream);

// dtype: 0 = fp32, 1 = bf16 (pa_dtype values)
hipError_t launch_decode_valu(const DecodeParams& p, int dtype, int D, hipStream_t stream);
hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t stream);
hipError_t launch_chunk_mfma(const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_mfma_f32(const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_reduce(const DecodeParams& p, int dtype, int D, hipStream_t stream);

// Precondition checks: count[0] = number of violating entries (two launches).
hipError_t launch_check_slots(const int32_t* slots, int32_t T, int32_t* count, hipStream_t stream);
hipError_t launch_check_pairs(const int32_t* pairs, int32_t n, int32_t NB, int32_t* count,
                              hipStream_t stream);
hipError_t launch_check_groups(const int32_t* group_start, const int32_t* seq_shared,
                               const int32_t* bt, const int32_t* ctx_lens, int32_t B,
                               int32_t n_groups, int32_t max_group, int32_t MB, int32_t* count,
                               hipStream_t stream);
hipError_t launch_check_tables(const int32_t* bt, const int32_t* ctx_lens, int32_t B, int32_t MB,
                               int32_t NB, int32_t ctx_limit, int32_t* count, hipStream_t stream);

// Query-head groups of up to 16 handled by one MFMA workgroup.
__host__ __device__ inline int mfma_q_groups(int G) { return (G + 15) / 16; }

}  // namespace pa
