// Host-side launch interface between the C ABI (pa_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

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
  float* ws_ml;                 // split only: [B][Hq][n_parts][2] = (m, l), log2 domain
  float* ws_o;                  // split only: [B][Hq][n_parts][D], unnormalised
  int32_t B, Hq, Hkv, G, NB, MB;
  int32_t ctx_limit;            // min(max_ctx, MB * 16): larger contexts are rejected
  int32_t partition;            // tokens per partition; 0 = one partition per sequence
  int32_t n_parts;              // grid extent over partitions
  int32_t max_q;                // grid bound on query rows per sequence (1 for decode)
  int32_t rows;                 // query rows in q / out (B for decode)
  int32_t n_tiles;              // MFMA: 16-column tiles per kv head (rows x heads per group)
  float qscale;                 // scale * log2(e): logits are kept in the log2 domain
  int32_t shared_kv;            // K/V tiles read through the caches (blocks shared by sequences)
};

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
  __device__ __forceinline__ int row_ctx(int i) const { return bad ? 0 : ctx - n + i + 1; }
};
__device__ __forceinline__ SeqRows seq_rows(const DecodeParams& P, int s) {
  SeqRows r;
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
hipError_t launch_decode_reduce(const DecodeParams& p, int dtype, int D, hipStream_t stream);

// Precondition checks: count[0] = number of violating entries (two launches).
hipError_t launch_check_slots(const int32_t* slots, int32_t T, int32_t* count, hipStream_t stream);
hipError_t launch_check_pairs(const int32_t* pairs, int32_t n, int32_t NB, int32_t* count,
                              hipStream_t stream);
hipError_t launch_check_tables(const int32_t* bt, const int32_t* ctx_lens, int32_t B, int32_t MB,
                               int32_t NB, int32_t ctx_limit, int32_t* count, hipStream_t stream);

// Query-head groups of up to 16 handled by one MFMA workgroup.
__host__ __device__ inline int mfma_q_groups(int G) { return (G + 15) / 16; }

}  // namespace pa
