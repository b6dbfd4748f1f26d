/*
 * Paged decode attention oracle: plain, slow, fp64 CPU code.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the correctness reference for the
 * GPU library. Only the test suite, the smoke check and the CPU-baseline leg
 * of the benchmark load it. It shares no code, header, table or helper with
 * the GPU path, and the GPU path never calls it.
 *
 * What it computes (and where that is defined):
 *
 *   "Why OS Virtual Memory Paging Saved LLM Inference" (a8q9.cn), section
 *   "2. The PagedAttention Architecture": the KV cache is cut into fixed-size
 *   physical blocks (e.g. 16 tokens); a block table maps each sequence's
 *   logical token positions to physical blocks; when attention is computed
 *   for a new token, the kernel looks up each block's physical address in the
 *   table and fetches the key/value vectors from wherever they sit.
 *
 *   "Can OS paging techniques reduce LLM serving memory waste?"
 *   (inquiringlines.com), mechanism paragraph: attention runs block by
 *   block, so the blocks may be non-contiguous; the result is unchanged.
 *
 *   "vLLM & PagedAttention" (completesystemdesign.dev), section "01. The
 *   Problem": to produce the next token the model looks back at the keys and
 *   values of every earlier token.
 *
 * Paging changes only WHERE a token's K/V row lives, so the decode result is
 * plain single-query softmax attention over the sequence's first ctx tokens
 * (the pages never write the formula; the textbook definition is used):
 *
 *   x_t   = scale * sum_d q[d] * K_t[d]              t = 0 .. ctx-1
 *   m     = max_t x_t
 *   w_t   = exp(x_t - m)
 *   out_d = (sum_t w_t * V_t[d]) / (sum_t w_t)
 *
 * with K_t, V_t read through the block table:
 *   b = block_tables[s][t / bs], o = t % bs,
 *   K_t = k_cache[b][g][o][:],   g = h / (Hq / Hkv)   (query-head groups are
 *   contiguous; the pages are silent on grouped heads, this is the reading).
 *
 * The pool layout is [num_blocks][num_kv_heads][bs][head_dim], row-major, for
 * both K and V (the pages fix no layout; this is the reading taken).
 *
 * Several new tokens per sequence (oracle_multi_query): each new token is a
 * query of its own, at its logical position, and attends to every position up
 * to and including its own (the same look-back rule the decode step applies
 * to its single new token, applied token by token), as when a prompt is
 * processed in chunks or several drafted tokens are checked in one pass.
 *
 * Everything is accumulated in double. bf16 inputs are widened exactly
 * (the 16 stored bits are the top half of an IEEE binary32). The softmax is
 * the two-pass textbook form (all logits first, then the max, then the
 * weights), not an online/streaming one.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

/* Read element idx of a dtype-tagged array and widen it to double exactly. */
static double widen(const void* base, size_t idx, int dtype) {
  if (dtype == ORACLE_F32) {
    return (double)((const float*)base)[idx];
  }
  uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Attention of one query row over the first L logical tokens of table row s,
 * kv head g: the row q[q_off .. q_off + D - 1] against K/V rows t = 0 .. L-1,
 * written to out[0 .. D-1]. Returns 0 on success, -1 if a block id read from
 * the table is out of range (the oracle checks what the GPU library takes as
 * a precondition), -2 if out of memory. */
static int attend(double* out, const void* q, size_t q_off, int32_t L,
                  const void* k_cache, const void* v_cache,
                  const int32_t* block_tables, int32_t s, int32_t g,
                  int32_t Hkv, int32_t D, int32_t bs, int32_t NB, int32_t MB,
                  double scale, int dtype) {
  for (int32_t d = 0; d < D; ++d) out[d] = 0.0;
  if (L <= 0) return 0; /* empty context: output defined as zeros */

  double* x = (double*)malloc(sizeof(double) * (size_t)L);
  if (!x) return -2;

  /* pass 1: every logit */
  for (int32_t t = 0; t < L; ++t) {
    const int32_t b = block_tables[(size_t)s * MB + t / bs];
    if (b < 0 || b >= NB) {
      free(x);
      return -1;
    }
    const int32_t o = t % bs;
    const size_t row = (((size_t)b * Hkv + g) * bs + o) * D;
    double dot = 0.0;
    for (int32_t d = 0; d < D; ++d)
      dot += widen(q, q_off + d, dtype) * widen(k_cache, row + d, dtype);
    x[t] = scale * dot;
  }

  /* pass 2: max, weights, normaliser */
  double m = x[0];
  for (int32_t t = 1; t < L; ++t)
    if (x[t] > m) m = x[t];
  double Z = 0.0;
  for (int32_t t = 0; t < L; ++t) {
    x[t] = exp(x[t] - m);
    Z += x[t];
  }

  /* pass 3: weighted sum of values */
  for (int32_t t = 0; t < L; ++t) {
    const int32_t b = block_tables[(size_t)s * MB + t / bs];
    const int32_t o = t % bs;
    const size_t row = (((size_t)b * Hkv + g) * bs + o) * D;
    for (int32_t d = 0; d < D; ++d) out[d] += x[t] * widen(v_cache, row + d, dtype);
  }
  for (int32_t d = 0; d < D; ++d) out[d] /= Z;
  free(x);
  return 0;
}

/* One (sequence s, query head h) decode row: the sequence's single query
 * attends over all context_lens[s] cached tokens. */
static int decode_one(double* out, const void* q, const void* k_cache,
                      const void* v_cache, const int32_t* block_tables,
                      const int32_t* context_lens, int32_t s, int32_t h,
                      int32_t Hq, int32_t Hkv, int32_t D, int32_t bs,
                      int32_t NB, int32_t MB, double scale, int dtype) {
  const int32_t G = Hq / Hkv;
  return attend(out, q, ((size_t)s * Hq + h) * D, context_lens[s], k_cache,
                v_cache, block_tables, s, h / G, Hkv, D, bs, NB, MB, scale,
                dtype);
}

/*
 * oracle_decode
 *   out          double; [B][Hq][D] when pairs == NULL, else [n_pairs][D]
 *   q            [B][Hq][D]            dtype-tagged
 *   k_cache      [NB][Hkv][bs][D]      dtype-tagged
 *   v_cache      [NB][Hkv][bs][D]      dtype-tagged
 *   block_tables int32 [B][MB]
 *   context_lens int32 [B]
 *   scale        the fp32 scale the GPU gets, widened to double
 *   pairs        optional int32 [n_pairs][2] = (s, h) rows to compute
 *   n_threads    OpenMP threads (<= 0: library default)
 * Returns 0, or -1 on a bad argument / out-of-range block id, -2 on OOM.
 */
int oracle_decode(double* out, const void* q, const void* k_cache,
                  const void* v_cache, const int32_t* block_tables,
                  const int32_t* context_lens, int32_t B, int32_t Hq,
                  int32_t Hkv, int32_t D, int32_t bs, int32_t NB, int32_t MB,
                  float scale, int32_t dtype, const int32_t* pairs,
                  int64_t n_pairs, int32_t n_threads) {
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return -1;
  if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || bs <= 0 || MB < 0 || NB < 0)
    return -1;
  if (Hq % Hkv != 0) return -1;
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;

  const int64_t n = pairs ? n_pairs : (int64_t)B * Hq;
  int err = 0;
#ifdef _OPENMP
  if (n_threads <= 0) n_threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads) reduction(min : err)
#endif
  for (int64_t i = 0; i < n; ++i) {
    int32_t s, h;
    if (pairs) {
      s = pairs[2 * i];
      h = pairs[2 * i + 1];
    } else {
      s = (int32_t)(i / Hq);
      h = (int32_t)(i % Hq);
    }
    if (s < 0 || s >= B || h < 0 || h >= Hq) {
      err = -1;
      continue;
    }
    int r = decode_one(out + (size_t)i * D, q, k_cache, v_cache, block_tables,
                       context_lens, s, h, Hq, Hkv, D, bs, NB, MB,
                       (double)scale, dtype);
    if (r < err) err = r;
  }
  (void)n_threads;
  return err;
}

/*
 * oracle_multi_query — several new query tokens per sequence, causal.
 *
 * Sequence s owns query rows query_start[s] .. query_start[s+1]-1 (n_s rows);
 * they are the last n_s tokens of its context, so row i (0-based) sits at
 * logical position ctx_s - n_s + i and attends to positions 0 .. ctx_s - n_s
 * + i, its own included: the decode rule applied to each new token in turn
 * (chunked prefill, or checking several drafted tokens at once). With
 * n_s = 1 for every s this is oracle_decode.
 *
 *   out          double; [Tq][Hq][D] when pairs == NULL, else [n_pairs][D]
 *   q            [Tq][Hq][D]            dtype-tagged
 *   query_start  int32 [B+1], non-decreasing, query_start[0] = 0,
 *                query_start[B] = Tq
 *   pairs        optional int32 [n_pairs][2] = (row, head) outputs to compute
 * A sequence with n_s > ctx_s is an error (-1).
 */
int oracle_multi_query(double* out, const void* q, const void* k_cache,
                       const void* v_cache, const int32_t* block_tables,
                       const int32_t* context_lens, const int32_t* query_start,
                       int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv,
                       int32_t D, int32_t bs, int32_t NB, int32_t MB,
                       float scale, int32_t dtype, const int32_t* pairs,
                       int64_t n_pairs, int32_t n_threads) {
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens ||
      !query_start)
    return -1;
  if (B < 0 || Tq < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || bs <= 0 || MB < 0 ||
      NB < 0)
    return -1;
  if (Hq % Hkv != 0) return -1;
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
  if (query_start[0] != 0 || query_start[B] != Tq) return -1;
  for (int32_t s = 0; s < B; ++s) {
    const int32_t n = query_start[s + 1] - query_start[s];
    if (n < 0 || n > context_lens[s]) return -1;
  }
  const int32_t G = Hq / Hkv;
  const int64_t n_rows = pairs ? n_pairs : (int64_t)Tq * Hq;
  int err = 0;
#ifdef _OPENMP
  if (n_threads <= 0) n_threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads) reduction(min : err)
#endif
  for (int64_t r = 0; r < n_rows; ++r) {
    const int32_t j = pairs ? pairs[2 * r] : (int32_t)(r / Hq);
    const int32_t h = pairs ? pairs[2 * r + 1] : (int32_t)(r % Hq);
    if (j < 0 || j >= Tq || h < 0 || h >= Hq) {
      err = -1;
      continue;
    }
    int32_t s = 0;
    while (query_start[s + 1] <= j) ++s; /* the sequence owning row j */
    const int32_t n = query_start[s + 1] - query_start[s];
    const int32_t i = j - query_start[s];
    const int32_t L = context_lens[s] - n + i + 1;
    int rc = attend(out + (size_t)r * D, q, ((size_t)j * Hq + h) * D, L,
                    k_cache, v_cache, block_tables, s, h / G, Hkv, D, bs, NB,
                    MB, (double)scale, dtype);
    if (rc < err) err = rc;
  }
  (void)n_threads;
  return err;
}

/* Number of OpenMP threads a parallel region gets by default. */
int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
