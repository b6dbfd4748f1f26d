/*
 * pa.h — paged KV-cache decode attention for AMD Instinct MI355X (gfx950).
 *
 * A KV cache split into fixed-size physical blocks, a per-sequence block
 * table from logical token positions to physical blocks, single-query decode
 * attention that gathers K/V through that table, the write of each step's new
 * K/V into its slot, and the copy of shared blocks before a write
 * (copy-on-write). Sources of the method:
 *
 *   [P1] "Why OS Virtual Memory Paging Saved LLM Inference: The vLLM
 *        Breakthrough" (a8q9.cn): section 2 "The PagedAttention Architecture"
 *        (fixed-size blocks, block table, on-demand allocation, attention
 *        kernel reading blocks through the table); section 3 "Copy-on-Write
 *        for Prompt Sharing".
 *   [P2] "vLLM & PagedAttention: Operating Systems Ideas for LLM Serving"
 *        (completesystemdesign.dev): section 01 "The Problem" (decode reads
 *        every earlier token's K and V each step and is memory-bound).
 *   [P3] "Can OS paging techniques reduce LLM serving memory waste?"
 *        (inquiringlines.com): mechanism paragraph (attention block by block,
 *        non-contiguous blocks, per-request block tables, block sharing).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every tensor argument is a DEVICE pointer owned by the caller; the
 *    library never allocates or frees device memory and keeps no state
 *    between calls, with one exception: the scratch area of
 *    pa_decode_noalloc, reserved with the library's code on each GPU (the
 *    block manager at the end is host-only and owns only host memory).
 *    Tensors are dense and row-major in the shapes given.
 *  - Cache pools: k_cache and v_cache are [NB][Hkv][bs][D] each: one
 *    (block, kv head) tile is bs contiguous token rows of D elements.
 *  - Element type `dt` (PA_F32 or PA_BF16) applies to q, out, the new K/V
 *    rows and both pools alike.
 *  - Supported: bs == 16; D in {64, 128}; Hq % Hkv == 0. Query head h reads
 *    kv head h / (Hq / Hkv).
 *  - Calls enqueue their kernels on `stream` (NULL = the null stream) and
 *    return once launched; nothing synchronises. A launch failure returns
 *    PA_EHIP. Host-side validation runs before any launch; on any error
 *    nothing is launched and no memory is touched.
 *  - Device-side contents are read defensively: an out-of-range block id,
 *    slot or context length never causes an out-of-bounds access. What each
 *    call does with such entries is stated with the call.
 *  - Thread-safe and reentrant: no global mutable state, apart from
 *    pa_decode_noalloc's per-GPU scratch area (see there).
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_EINVAL = -1,        /* null pointer, bad size, inconsistent arguments   */
  PA_EUNSUPPORTED = -2,  /* valid request outside the compiled kernels       */
  PA_EWORKSPACE = -3,    /* workspace missing or smaller than required       */
  PA_EHIP = -4,          /* the HIP runtime rejected a launch                */
  PA_ENOBLOCKS = -5      /* block manager: not enough free blocks            */
} pa_status;

typedef enum { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

/*
 * Flags of pa_decode / pa_multi_query.
 *   PA_KV_SHARED  some physical block is referenced by more than one sequence
 *                 of the call (forks, beams, a prefix cache: [P1] section 3,
 *                 [P3] mechanism paragraph). K/V tiles are then read through
 *                 the caches so that repeated reads of a shared block are
 *                 served there; without it they are streamed past the caches
 *                 (read once per step), which sustains a higher HBM rate.
 *                 Results are the same either way; only speed differs.
 */
#define PA_KV_SHARED 1u
/*
 *   PA_KV_SHARED_GROUPS  pa_decode_shared only: the shared blocks of different
 *                 groups overlap (one prefix split over several groups); the
 *                 group pass then reads through the caches. PA_KV_SHARED there
 *                 applies to each sequence's own blocks (the tail pass).
 */
#define PA_KV_SHARED_GROUPS 2u

/* Static, human-readable text for a status code. Never NULL. */
const char* pa_status_str(pa_status s);

/*
 * pa_slot_mapping — physical slot of logical token positions.
 *
 * [P1] section 2: the block table maps a sequence's logical token positions
 * to physical blocks, as a page table maps pages. Position p lies in
 * logical block p / bs at offset p % bs, so for token i of sequence
 * s = seq_ids[i] at position p = positions[i]:
 *     slot_mapping[i] = block_tables[s][p / bs] * bs + p % bs.
 *
 *   slot_mapping  out, int32 [T]
 *   block_tables  int32 [B][MB]; entries may be -1 (unused)
 *   seq_ids       int32 [T], or NULL for seq_ids[i] = i (then T must be <= B)
 *   positions     int32 [T]
 * A negative position, a position at or past MB * bs, a sequence index
 * outside [0, B), a negative table entry or one above (INT32_MAX - 15) / 16
 * (whose slots do not fit an int32) gives slot -1 (the "no write" marker
 * pa_write_kv skips). T == 0 is a no-op.
 */
pa_status pa_slot_mapping(int32_t* slot_mapping, const int32_t* block_tables,
                          const int32_t* seq_ids, const int32_t* positions,
                          int32_t T, int32_t B, int32_t MB, int32_t bs,
                          hipStream_t stream);

/*
 * pa_write_kv — write each new token's K and V rows into its slot
 * (the reshape-and-cache step).
 *
 * [P1] section 2: blocks fill as tokens are generated. Row i of k_new/v_new
 * (all Hkv heads) goes to slot s = slot_mapping[i]:
 *     k_cache[s / bs][g][s % bs][:] = k_new[i][g][:]   for every kv head g,
 * and likewise for V. The copy is of raw bits (NaN payloads and denormals
 * are preserved).
 *
 *   k_new, v_new   [T][Hkv][D]
 *   k_cache, v_cache [NB][Hkv][bs][D], modified in place
 *   slot_mapping   int32 [T]; slot < 0 or slot >= NB * bs is skipped
 * Slots must be distinct within one call (else which row lands is
 * unspecified). T == 0 is a no-op.
 */
pa_status pa_write_kv(const void* k_new, const void* v_new, void* k_cache,
                      void* v_cache, const int32_t* slot_mapping, int32_t T,
                      int32_t NB, int32_t Hkv, int32_t D, int32_t bs,
                      pa_dtype dt, hipStream_t stream);

/*
 * pa_append_kv — pa_slot_mapping and pa_write_kv in one launch.
 *
 * [P1] section 2: each new token's slot comes from its sequence's block table
 * (block_tables[s][p / bs] * bs + p % bs, as in pa_slot_mapping), and its K
 * and V rows are written there (as in pa_write_kv). The effect on the pools,
 * and on slot_mapping when it is given, is exactly that of the two calls in a
 * row; one kernel replaces two dependent launches on the decode step.
 *
 *   k_new, v_new     [T][Hkv][D]
 *   k_cache, v_cache [NB][Hkv][bs][D], modified in place
 *   slot_mapping     out, int32 [T], or NULL when the caller does not need it
 *   block_tables     int32 [B][MB]; entries may be -1 (unused)
 *   seq_ids          int32 [T], or NULL for seq_ids[i] = i (then T must be <= B)
 *   positions        int32 [T]
 * Tokens whose slot is -1 (see pa_slot_mapping) or at or past NB * bs are not
 * written. Slots must be distinct within one call. T == 0 is a no-op.
 */
pa_status pa_append_kv(const void* k_new, const void* v_new, void* k_cache,
                       void* v_cache, int32_t* slot_mapping,
                       const int32_t* block_tables, const int32_t* seq_ids,
                       const int32_t* positions, int32_t T, int32_t B, int32_t MB,
                       int32_t NB, int32_t Hkv, int32_t D, int32_t bs, pa_dtype dt,
                       hipStream_t stream);

/*
 * pa_copy_blocks — copy-on-write block copies.
 *
 * [P1] section 3: branches of one request share the physical prompt blocks;
 * a branch about to write into a shared block first gets a private copy.
 * For each pair i: K[dst] = K[src] and V[dst] = V[src], whole blocks (all kv
 * heads, slots and dims), raw bits.
 *
 *   pairs  int32 [n][2] = (src, dst), device memory
 * Pairs with an id outside [0, NB) are skipped. Destinations must be
 * distinct and no destination may also be a source within one call (then
 * the parallel copy equals the in-order one). n == 0 is a no-op.
 */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs,
                         int32_t n, int32_t NB, int32_t Hkv, int32_t D,
                         int32_t bs, pa_dtype dt, hipStream_t stream);

/*
 * Precondition checks, for debugging a caller. The write, copy and attention
 * calls take these on trust (their own checks cover the rest); each check
 * counts the violating entries of its input on the device and writes the
 * number to count[0] (device memory, int32; 0 = none). Two launches on
 * `stream`, no allocation; read count[0] after the stream is synchronised.
 *
 * pa_check_slots — [P1] section 2: the cache write fills the slots the block
 * table maps new tokens to, so two tokens of one pa_write_kv / pa_append_kv
 * call must not share a slot. Counts tokens whose slot is >= 0 and equal to
 * an earlier token's. Cost O(T^2 / 64) loads.
 */
pa_status pa_check_slots(const int32_t* slot_mapping, int32_t T, int32_t* count,
                         hipStream_t stream);

/*
 * pa_check_pairs — [P1] section 3: copy-on-write copies of one pa_copy_blocks
 * call run in parallel, so among pairs with both ids in [0, NB) (the others
 * are skipped), no destination may repeat and no destination may also be a
 * source. Counts the pairs whose destination repeats an earlier pair's or is
 * some pair's source. Cost O(n^2).
 */
pa_status pa_check_pairs(const int32_t* pairs, int32_t n, int32_t NB, int32_t* count,
                         hipStream_t stream);

/*
 * pa_check_tables — [P1] section 2: attention reads a sequence's first
 * ceil(L / bs) table entries. Counts the sequences whose context length L is
 * negative or above min(max_ctx, MB * bs), or one of whose entries below
 * ceil(L / bs) lies outside [0, NB). (pa_decode returns NaN rows for such
 * sequences.)
 */
pa_status pa_check_tables(const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                          int32_t MB, int32_t NB, int32_t max_ctx, int32_t bs, int32_t* count,
                          hipStream_t stream);

/*
 * pa_check_groups — [P1] section 3: pa_decode_shared reads a group's shared
 * blocks once, through its first member's table. Counts the groups whose
 * bounds are malformed (not in order from 0 to B, empty, or larger than
 * max_group) and the members of well-formed groups whose shared length
 * differs from the first member's, is not a multiple of bs, exceeds the
 * member's context or table, or whose first S / bs table entries differ from
 * the first member's. Cost O(B * MB).
 */
pa_status pa_check_groups(const int32_t* group_start, const int32_t* seq_shared,
                          const int32_t* block_tables, const int32_t* context_lens,
                          int32_t B, int32_t n_groups, int32_t max_group, int32_t MB,
                          int32_t bs, int32_t* count, hipStream_t stream);

/*
 * pa_decode_default_partition — split-context partition size (tokens) the
 * library would pick for this shape on the current device: 0 (no split) when
 * the unsplit workgroups already fill the GPU (at least 4 per compute
 * unit, one per sequence and kv head or query head), when max_ctx is at most
 * 512, or, with grouped query heads (Hq / Hkv >= 2), at most 2048; else a
 * multiple of bs. Never fails; returns 0 for invalid shapes.
 */
int32_t pa_decode_default_partition(int32_t B, int32_t Hq, int32_t Hkv,
                                    int32_t D, int32_t max_ctx);

/*
 * pa_decode_workspace_bytes — device workspace pa_decode (rows = B) or
 * pa_multi_query (rows = Tq) needs for this split: 0 when partition == 0 or
 * max_ctx <= partition, otherwise room for one partial result per (query
 * row, query head, partition): an fp32 (max, sum) pair of the partition's
 * online-softmax state, and a row of D elements. The row is the state's
 * unnormalised output in fp32 for fp32 I/O; for bf16 I/O, an fp16 row of an
 * equivalent rescaled state (the row divided by its sum times a power of
 * two, the pair adjusted to match). Sized as (8 + 4 D) bytes per partial,
 * plus alignment, for both dtypes. The contents are scratch: nothing is kept
 * between calls.
 */
size_t pa_decode_workspace_bytes(int32_t rows, int32_t Hq, int32_t D,
                                 int32_t max_ctx, int32_t partition);

/*
 * pa_decode — single-query decode attention over the paged cache.
 *
 * [P1] section 2 / [P3] mechanism paragraph: for the new token, look up each
 * logical block's physical block in the table and read K/V from it; the
 * result equals attention over the contiguous history. [P2] section 01: the
 * query attends over every cached token of its sequence. For sequence s,
 * query head h, kv head g = h / (Hq / Hkv), L = context_lens[s]:
 *     x_t   = scale * dot(q[s][h], K_t),   t = 0 .. L-1
 *     out   = sum_t softmax(x)_t * V_t
 * where K_t = k_cache[block_tables[s][t / bs]][g][t % bs]. L counts the
 * tokens in the cache including the step's own token (write it with
 * pa_write_kv first). Accumulation is fp32; bf16 output is rounded to
 * nearest even.
 *
 *   out            [B][Hq][D], must not alias any input
 *   q              [B][Hq][D]
 *   k_cache, v_cache [NB][Hkv][bs][D]
 *   block_tables   int32 [B][MB]; only entries t / bs < ceil(L / bs) are read
 *   context_lens   int32 [B], device memory
 *   max_ctx        host-side upper bound on every context_lens[s] (sizes the
 *                  grid without a device-to-host read)
 *   scale          fp32 logit scale (usually 1 / sqrt(D)); any finite value,
 *                  negative and zero included (NaN or infinity: PA_EINVAL)
 *   partition      tokens per split-context partition: 0 = no split, else a
 *                  positive multiple of bs. With a split, every partition is
 *                  attended independently and a second kernel merges the
 *                  partitions of each (sequence, head) with log-sum-exp
 *                  weights.
 *   workspace      device buffer of at least
 *                  pa_decode_workspace_bytes(B, Hq, D, max_ctx, partition)
 *                  bytes, 256-byte aligned (may be NULL when that is 0)
 *   flags          0 or PA_KV_SHARED; other bits give PA_EINVAL
 * L == 0 gives an all-zero row. A sequence whose L is negative or exceeds
 * min(max_ctx, MB * bs), or whose table holds an id outside [0, NB) at a
 * position it reads, gets an all-NaN output row and its K/V are not read.
 */
pa_status pa_decode(void* out, const void* q, const void* k_cache,
                    const void* v_cache, const int32_t* block_tables,
                    const int32_t* context_lens, int32_t B, int32_t Hq,
                    int32_t Hkv, int32_t D, int32_t bs, int32_t NB, int32_t MB,
                    int32_t max_ctx, float scale, int32_t partition,
                    void* workspace, size_t workspace_bytes, uint32_t flags,
                    pa_dtype dt, hipStream_t stream);

/*
 * pa_decode_noalloc — pa_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, hosts that
 * forbid hipMalloc. It takes no workspace: split-context partials go to a
 * scratch area of PA_NOALLOC_SCRATCH_BYTES (64 MiB) that the library holds
 * on each GPU it runs on, from the loading of its code there until the
 * process ends. The first call on a device looks up that device's copy
 * (hipGetSymbolAddress); no call allocates or frees device memory.
 *
 * Arguments, results and error rows are pa_decode's, without workspace and
 * workspace_bytes; the kernels, and so the output bits, are the same as
 * pa_decode's with a workspace. A split whose pa_decode_workspace_bytes(B,
 * Hq, D, max_ctx, partition) exceeds PA_NOALLOC_SCRATCH_BYTES returns
 * PA_EWORKSPACE and launches nothing.
 *
 * Every call on one GPU shares that GPU's scratch area, which keeps the last
 * call's contents. Nothing in it needs to start at zero (each call writes
 * every partial it reads back), but calls that overlap in time on one GPU
 * (other streams, other host threads) race on it: order them, e.g. on one
 * stream. Unlike the other entry points, this one keeps state: the scratch
 * area and the per-device address looked up on first use (thread-safe).
 */
#define PA_NOALLOC_SCRATCH_BYTES (64u << 20)
pa_status pa_decode_noalloc(void* out, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* block_tables,
                            const int32_t* context_lens, int32_t B, int32_t Hq,
                            int32_t Hkv, int32_t D, int32_t bs, int32_t NB,
                            int32_t MB, int32_t max_ctx, float scale,
                            int32_t partition, uint32_t flags, pa_dtype dt,
                            hipStream_t stream);

/*
 * pa_decode_shared — pa_decode for a batch whose sequences share leading
 * blocks (parallel samples of one prompt, beams, a common prefix), reading
 * each shared block once per group of sharers instead of once per sequence.
 *
 * [P1] section 3 / [P3] mechanism paragraph: sequences forked from one
 * prompt, or requests with a common prefix, point their tables at the same
 * physical blocks. The result is pa_decode's, up to the order of summation:
 * attention over 0 .. L-1 splits into the shared tokens 0 .. S_s-1 and the
 * sequence's own S_s .. L-1, and the two online-softmax partials are merged
 * by log-sum-exp weights as between split-context partitions.
 *
 *   group_start  int32 [n_groups + 1], device: group j is the sequences
 *                group_start[j] .. group_start[j+1]-1 (consecutive, at least
 *                one, at most max_group); the groups cover 0 .. B-1 in order
 *   seq_shared   int32 [B], device: S_s, the leading tokens sequence s shares
 *                with its group: a multiple of bs, the same for every member,
 *                at most context_lens[s]; the members' block_tables agree on
 *                the first S_s / bs entries (0 for a sequence that shares
 *                nothing)
 *   max_group    host bound on the group sizes (in bf16, groups of more than
 *                16 / (Hq / Hkv) members run on the chunk kernel, whose waves
 *                share each block through LDS; in fp32, one workgroup per 16
 *                (member, query head) columns)
 *   max_shared   host bound on every S_s (a multiple of bs, <= max_ctx)
 *   partition    tokens per partition of the shared part (0 = one partition;
 *                else a positive multiple of bs); each sequence's own tokens
 *                are one partition
 *   workspace    at least pa_decode_shared_workspace_bytes(B, Hq, D,
 *                max_shared, partition) bytes, 256-byte aligned (may be NULL
 *                when that is 0)
 *   flags        PA_KV_SHARED (blocks past the shared part read by several
 *                sequences) and/or PA_KV_SHARED_GROUPS (shared parts of
 *                different groups overlap); other bits give PA_EINVAL
 * Other arguments and error rows as pa_decode. In bf16, when the shared part
 * is one partition and a group's columns fit one 16-column tile, one launch:
 * each group's workgroup reads its shared blocks, then every member's own
 * blocks (the workspace goes unused). Otherwise two launches: the shared part
 * of every group (one read of its blocks for all members' query heads, on
 * the matrix cores, into the workspace), then every sequence's own tokens,
 * merged with its shared part into the final row (in bf16 with more than 16
 * query heads per kv head, one query head per workgroup). bf16 and fp32.
 * A shared length that is
 * negative, not a multiple of bs or beyond the table gives that sequence an
 * all-NaN row (the group pass takes the first member's, so a bad one there gives the
 * whole group NaN rows). Member tables that disagree on the shared entries
 * are not detected (the group's first member's blocks are used for all);
 * members whose shared lengths differ get undefined rows (no read leaves the
 * workspace). B == 0 is a no-op.
 */
size_t pa_decode_shared_workspace_bytes(int32_t B, int32_t Hq, int32_t D,
                                        int32_t max_shared, int32_t partition);
/* A partition length for the shared part: 0 (one partition) when the group
 * pass has at least one workgroup per compute unit of the current device,
 * else about half of max_shared (a multiple of bs), so that the pass fills
 * the device. 0 for arguments that give nothing to split. */
int32_t pa_decode_shared_default_partition(int32_t n_groups, int32_t Hq,
                                           int32_t Hkv, int32_t max_group,
                                           int32_t max_shared);
pa_status pa_decode_shared(void* out, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* block_tables,
                           const int32_t* context_lens,
                           const int32_t* group_start, const int32_t* seq_shared,
                           int32_t B, int32_t n_groups, int32_t max_group,
                           int32_t max_shared, int32_t Hq, int32_t Hkv,
                           int32_t D, int32_t bs, int32_t NB, int32_t MB,
                           int32_t max_ctx, float scale, int32_t partition,
                           void* workspace, size_t workspace_bytes,
                           uint32_t flags, pa_dtype dt, hipStream_t stream);

/*
 * pa_shared_groups — the groups and shared lengths pa_decode_shared takes,
 * from the block tables (HOST memory; the block manager's view).
 *
 * [P1] section 3: sharers of a block point their tables at the same physical
 * block. Scans the sequences in order and starts a group at sequence s; the
 * next sequence joins while the group has fewer than max_group members and
 * its table agrees with the group's first member's on at least one leading
 * block that lies whole inside both contexts. The group's shared length is
 * bs times the number of leading whole blocks on which every member agrees;
 * a group of one shares nothing (0). Writes group_start [B + 1 at most, the
 * first *n_groups + 1 entries used] and seq_shared [B]. Table entries past a
 * sequence's context are not read.
 */
pa_status pa_shared_groups(const int32_t* block_tables, const int32_t* context_lens,
                           int32_t B, int32_t MB, int32_t bs, int32_t max_group,
                           int32_t* group_start, int32_t* seq_shared,
                           int32_t* n_groups);

/*
 * pa_multi_query — causal attention of several new tokens per sequence over
 * the paged cache (a prompt processed in chunks, or several drafted tokens
 * checked in one pass).
 *
 * "vLLM & PagedAttention" (completesystemdesign.dev), section 01: a new
 * token attends over the keys and values of every earlier token; here each
 * new token of a chunk does so in turn, its own and the chunk's earlier
 * tokens included. [P1] section 2: K/V are read through the block table.
 * Sequence s owns query rows query_start[s] .. query_start[s+1]-1 (n_s rows),
 * the last n_s tokens of its context (write their K/V with pa_write_kv
 * first). Row i (0-based) sits at position ctx_s - n_s + i and, for query head
 * h and kv head g = h / (Hq / Hkv):
 *     out[row][h] = sum_t softmax(x)_t V_t,  x_t = scale * dot(q[row][h], K_t),
 *     t = 0 .. ctx_s - n_s + i.
 * With every n_s = 1 this is pa_decode. Accumulation is fp32; bf16 output is
 * rounded to nearest even.
 *
 *   out, q         [Tq][Hq][D]; out must not alias any input
 *   query_start    int32 [B + 1], device memory, non-decreasing, with
 *                  query_start[0] = 0 and query_start[B] = Tq
 *   max_q          host-side upper bound on every n_s (sizes the grid)
 *   workspace      at least pa_decode_workspace_bytes(Tq, Hq, D, max_ctx,
 *                  partition) bytes, 256-byte aligned
 * Other arguments as pa_decode. A sequence whose n_s exceeds its context
 * length or max_q, or whose context length is invalid, gets all-NaN rows
 * (those among its first max_q); a sequence whose rows fall outside
 * [0, Tq) gets none written. B == 0 or Tq == 0 is a no-op.
 */
pa_status pa_multi_query(void* out, const void* q, const void* k_cache,
                         const void* v_cache, const int32_t* block_tables,
                         const int32_t* context_lens,
                         const int32_t* query_start, int32_t B, int32_t Tq,
                         int32_t max_q, int32_t Hq, int32_t Hkv, int32_t D,
                         int32_t bs, int32_t NB, int32_t MB, int32_t max_ctx,
                         float scale, int32_t partition, void* workspace,
                         size_t workspace_bytes, uint32_t flags, pa_dtype dt,
                         hipStream_t stream);

/*
 * Block manager — host-side bookkeeping of the physical block pool.
 *
 * [P1] section 2: blocks are handed out one at a time, only when a token
 * needs a new one; each sequence has a table from logical to physical
 * blocks. [P1] section 3 / [P3] mechanism paragraph: sequences may share
 * blocks; a sequence about to write into a shared block gets a private copy
 * first. Sharing is tracked with per-block reference counts. The free list
 * hands out blocks from its front and takes freed blocks back at its front.
 * All pointers below are HOST memory. One manager must not be used from two
 * threads at once; distinct managers are independent.
 */
typedef struct pa_block_manager pa_block_manager;

/* free_order: host int32 [num_blocks], a permutation of 0..num_blocks-1 giving
 * the initial free-list order, or NULL for 0, 1, 2, ... */
pa_status pa_bm_create(pa_block_manager** bm, int32_t num_blocks,
                       int32_t block_size, const int32_t* free_order);
void pa_bm_destroy(pa_block_manager* bm);

/* A new, empty sequence; its id is written to *seq. */
pa_status pa_bm_add_seq(pa_block_manager* bm, int32_t* seq);

/* A new sequence sharing every block of `parent` (their counts go up). */
pa_status pa_bm_fork(pa_block_manager* bm, int32_t parent, int32_t* child);

/*
 * Append n tokens to `seq`. slots: host int32 [n] receives the physical slot
 * of each new token. At most one copy-on-write pair arises per call (only the
 * partly filled last block can be shared); it is written to pair[0..1] as
 * (src, dst) and *n_pairs is set to 0 or 1; the caller copies that block
 * (pa_copy_blocks) before writing the tokens (pa_write_kv). If the free list
 * cannot supply every block the call needs, PA_ENOBLOCKS is returned and
 * nothing changes.
 */
pa_status pa_bm_append(pa_block_manager* bm, int32_t seq, int32_t n,
                       int32_t* slots, int32_t* pair, int32_t* n_pairs);

/*
 * As pa_bm_append, for tokens whose ids are known: tokens host int32 [n].
 * Every block these tokens fill becomes shareable with later requests (see
 * pa_bm_add_seq_cached). Appending tokens of unknown content (pa_bm_append)
 * ends that for the rest of the sequence.
 */
pa_status pa_bm_append_tokens(pa_block_manager* bm, int32_t seq,
                              const int32_t* tokens, int32_t n, int32_t* slots,
                              int32_t* pair, int32_t* n_pairs);

/*
 * Prefix sharing across requests ([P3] mechanism paragraph: requests share
 * KV blocks within and across a batch; [P2] introduction: prefix caching).
 * A new sequence for a request whose prompt is tokens host int32 [n]: its
 * first blocks are the longest run of the prompt's full blocks that some
 * earlier pa_bm_append_tokens registered, with exactly this prefix, at most
 * (n - 1) / block_size of them (at least one prompt token is left to
 * process). *n_cached receives the number of prompt tokens already in the
 * cache; continue with pa_bm_append_tokens(seq, tokens + *n_cached, ...).
 * Blocks are matched on their exact token ids and on the exact preceding
 * chain, never on a hash alone.
 * A registered block that its last holder releases is kept, evictable: it
 * counts as free, allocation uses the free list first and then evicts kept
 * blocks in the order they were released (oldest first), dropping their
 * registration.
 */
pa_status pa_bm_add_seq_cached(pa_block_manager* bm, const int32_t* tokens,
                               int32_t n, int32_t* seq, int32_t* n_cached);

/*
 * Beam search ([P1] section 3: beams share prompt blocks): sequence dst drops
 * its blocks and shares every block of src instead, as a pruned beam replaced
 * by a surviving one. dst == src is a no-op.
 */
pa_status pa_bm_fork_into(pa_block_manager* bm, int32_t dst, int32_t src);

/* Drop `seq`; blocks no other sequence holds become free (or kept, when
 * registered for sharing). */
pa_status pa_bm_free_seq(pa_block_manager* bm, int32_t seq);

pa_status pa_bm_seq_len(const pa_block_manager* bm, int32_t seq, int32_t* len);
/* Blocks an append may take: free ones plus kept (evictable) ones. */
pa_status pa_bm_num_free(const pa_block_manager* bm, int32_t* n);
/* Kept blocks: registered for sharing, held by no sequence. */
pa_status pa_bm_num_cached(const pa_block_manager* bm, int32_t* n);
pa_status pa_bm_refcount(const pa_block_manager* bm, int32_t block, int32_t* ref);

/* The table of `seq`: up to cap ids to out (host int32), count to *n. */
pa_status pa_bm_block_table(const pa_block_manager* bm, int32_t seq,
                            int32_t* out, int32_t cap, int32_t* n);

/*
 * Dense tables for a batch: tables host int32 [n_seqs][MB] (unused = -1) and
 * lens host int32 [n_seqs]. PA_EINVAL if a table is longer than MB.
 */
pa_status pa_bm_fill_tables(const pa_block_manager* bm, const int32_t* seqs,
                            int32_t n_seqs, int32_t MB, int32_t* tables,
                            int32_t* lens);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
