// Paged attention on the matrix cores (bf16, head_dim 128 or 64): grouped
// query heads, and several new query tokens per sequence.
//
// Method: as the vector path ("Why OS Virtual Memory Paging Saved LLM
// Inference" (a8q9.cn), section 2: K/V gathered block by block through the
// block table; online softmax over blocks). A kv head serves the G query
// heads of its group and, with several new tokens per sequence, every new
// token's row: each 16-token K tile meets up to 16 such (row, head) columns,
// a small real contraction done on the MFMA units, so that every K/V byte is
// read once per 16 columns instead of once per column.
//
// Columns: the n x G (query row, head of the group) pairs of a sequence and
// kv head, row-major, in tiles of 16; one workgroup per (kv head, tile,
// partition, sequence). A kv head with more than one tile goes to the chunk
// kernel (chunk_mfma.hip, same layouts), whose waves share each block. Column (i, q) attends over its row's causal prefix
// (ctx - n + i + 1 tokens): a per-column limit masks the logits. The decode
// step is n = 1: the columns are the G heads.
//
// Layouts (wave64; lane = 16 * rg + col, rg = lane / 16, col = lane % 16):
//   S^T = K Q^T with v_mfma_f32_16x16x32_bf16, 4 steps over D (kk = 0..3):
//     A (16 tokens x 32 dims): lane holds K[t = col][32 kk + 8 rg + 0..7].
//     K is loaded like V (4 whole rows per load instruction, which streams
//     faster than 16 row segments) and transposed into this layout through
//     a per-wave LDS stage.
//     B (32 dims x 16 cols):   lane holds Q[q = col][32 kk + 8 rg + 0..7]
//     result: lane holds S^T[t = 4 rg + i][q = col], i = 0..3
//   So every lane owns one column (col) and 4 tokens: the softmax max is an
//   in-lane max plus a max over the 4 row groups.
//   O^T = V^T P^T with v_mfma_f32_16x16x16_bf16 (K dimension = 16 tokens):
//     V is loaded row-wise: lane holds V[t = 4 rg + j][8 col + 0..7], j = 0..3
//     (each load instruction reads 4 whole 256-byte rows).
//     For output tile e (e = 0..7) the A operand (16 "dims" x 16 tokens) is
//     {V[4 rg + j][8 col + e]}_j, i.e. row m = col stands for dim 8 m + e;
//     it is assembled from the loaded registers with byte permutes.
//     B (16 tokens x 16 cols): lane holds P^T[t = 4 rg + j][q = col] = the
//     lane's own 4 probabilities, rounded to bf16.
//     result tile e: lane holds O^T[d = 8 (4 rg + i) + e][q = col].
//   Every accumulator a lane holds belongs to its own column, so the
//   online-softmax rescale is a per-lane multiply.
// Columns past the last real one are zero-padded and never written.
#include "pa_device.h"
#include "pa_launch.h"

// Waves per workgroup (split contexts, and unsplit ones) and K/V tiles in
// flight per wave.
#ifndef PA_MFMA_WAVES
#define PA_MFMA_WAVES 4
#endif
#ifndef PA_MFMA_WAVES_UNSPLIT
#define PA_MFMA_WAVES_UNSPLIT 8
#endif
// Waves per workgroup of the shared-prefix group pass (a group's shared
// blocks, usually few work items: smaller workgroups all fit at once).
#ifndef PA_MFMA_GROUP_WAVES
#define PA_MFMA_GROUP_WAVES 4
#endif
#ifndef PA_MFMA_DEPTH
#define PA_MFMA_DEPTH 2
#endif
// Waves per workgroup of the group pass with the members' own blocks folded
// in: PA_MFMA_FOLD_WAVES_FEW when the pass has at most one workgroup per
// compute unit (the prefix batch, 256 workgroups: 105 vs 110 us with 4),
// else PA_MFMA_FOLD_WAVES (the copy-on-write batch, 512: 4 waves 113 vs 114
// with 8).
#ifndef PA_MFMA_FOLD_WAVES
#define PA_MFMA_FOLD_WAVES 4
#endif
#ifndef PA_MFMA_FOLD_WAVES_FEW
#define PA_MFMA_FOLD_WAVES_FEW 8
#endif
// Waves per workgroup of the shared-prefix tail pass (each sequence's own
// blocks past its group's shared ones: few per sequence). The 64/8-head
// copy-on-write batch (tails of 1-256 tokens): 4 waves 37.4 us for the call,
// 2 waves 37.0, 8 waves 41.5.
#ifndef PA_MFMA_TAIL_WAVES
#define PA_MFMA_TAIL_WAVES 4
#endif
// Column tiles per kv head from which a call goes to the chunk kernel; with
// fewer, one workgroup per tile here (the tiles of a kv head on one XCD). On
// the GQA batch with 3, 4 or 8 new tokens per sequence (2 or 4 tiles per kv
// head, 512-token partitions): 4.4-4.6 TB/s on the chunk kernel, 3.3-3.4
// with 2 tiles and 2.1 with 4 here.
#ifndef PA_CHUNK_MIN_TILES
#define PA_CHUNK_MIN_TILES 2
#endif
// Minimum waves per SIMD the register allocation must allow.
#ifndef PA_MFMA_MIN_WAVES
#define PA_MFMA_MIN_WAVES 3
#endif

namespace pa {

// The waves of a workgroup interleave the blocks of one column tile (wave w
// takes blocks w, w + NW, ...) and merge their states through LDS. A kv head
// with more than one tile (several query rows per sequence) goes to the
// chunk kernel instead, whose waves share each block.
//
// kFold (the shared-prefix group pass, one partition, one tile): after the
// group's shared blocks (every column), each member's own blocks, read
// through its own table row, with only that member's columns unmasked; the
// workgroup then writes the members' final rows. Member j's own blocks
// S_j / 16 + w, + w + NW, ... go to wave w, so the order of a member's
// arithmetic does not depend on the other members: their blocks reach its
// columns as masked logits, which leave its state bit for bit as it was
// (probabilities 0, rescale by exactly 1). kTailPolicy is the cache policy of
// the members' own blocks.
template <int D, int NW, int DEPTH, TilePolicy kPolicy, bool kFold = false,
          TilePolicy kTailPolicy = kPolicy>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(PA_MFMA_MIN_WAVES)))
void decode_mfma_kernel(DecodeParams P) {
  static_assert(D == 128 || D == 64, "head_dim");
  constexpr int kRowBytes = D * 2;
  constexpr int kQK = D / 32;         // 16x16x32 steps of S^T over D
  constexpr int kPiece = D / 8;       // bytes of a row per lane of a 16-lane group
  constexpr int kTiles = D / 16;      // 16-dim output tiles of O^T
  using Piece = typename TilePiece<kPiece>::type;
  constexpr int kPad = 4;  // LDS row padding (floats) against bank conflicts
  constexpr int kStageRow = kRowBytes + 16;  // LDS stride of a staged K row
  static_assert(kBlock * kStageRow <= 16 * (D + kPad) * 4, "K stage must fit a merge region");

  const int lane = threadIdx.x & (kWave - 1);
  const int w = wave_id();
  const int col = lane & 15;
  const int rg = lane >> 4;

  // A kv head with several tiles goes to the chunk kernel unless
  // PA_CHUNK_MIN_TILES is raised; then its tiles run here, one workgroup
  // each, kept on one XCD (they read the same K/V).
  const GridPos gp = P.n_tiles > 1 ? grid_pos_grouped(P.n_tiles) : grid_pos();
  const int p = gp.y;
  const int g = gp.x / P.n_tiles;    // kv head
  const int tile = gp.x % P.n_tiles;  // 16-column tile of this kv head's (row, head) pairs
  const int s = gp.z;

  const ItemStart is = item_start(P, s);
  const int32_t* bt_row = P.block_tables + (size_t)is.trow * P.MB;
  const int bpp = P.partition / kBlock;  // blocks per partition (0: no split)
  // (the tail pass is unsplit and walks the same blocks as an unsplit call,
  // from its first block past the shared ones: see k0 below)
  const int blk_begin = p * bpp;
  // this wave's blocks: first, first + kStride, ...
  constexpr int kStride = NW;
  const int first = blk_begin + w;

  // Start-up loads, issued before anything waits on them: the wave's first 64
  // block ids (bounded by the partition's table range, as the context length
  // is not known yet), the sequence's rows and context length, the queries.
  const int ids0 = first_chunk_ids(bt_row, first, kStride,
                                   bpp > 0 ? min(P.MB, blk_begin + bpp) : P.MB, lane);
  const SeqRows sr = seq_rows(P, s);
  // Columns of this tile: global column gc = 16 tile + col of the n x G grid
  // of (query row, head of the group), row-major; gc >= n G is padding.
  const int ncols = min(sr.n, P.max_q) * P.G;
  const int c_begin = 16 * tile;
  if (c_begin >= ncols) return;  // no real column
  const int c_end = min(ncols, c_begin + 16);
  const int gc = c_begin + col;
  const bool col_ok = gc < c_end;
  const int gcl = col_ok ? gc : c_end - 1;  // padded lanes shadow a real column
  const int qi = gcl / P.G;                 // this lane's query row
  const int qh = g * P.G + gcl % P.G;       // and query head
  const int qrow = sr.first + qi;

  // B operand of S^T: Q[column col][32 kk + 8 rg ..], zero for padded columns.
  bf16x8_t qop[kQK];
  // LDS, one region per wave: while the wave streams its blocks, the first
  // kStageBytes hold the K tile it is transposing (below); at the end the
  // region holds the wave's merge rows (16 columns x D floats, padded). The
  // wave overwrites its stage only after its last read of it, and a wave's
  // LDS accesses complete in order, so no barrier guards either use.
  __shared__ float sm_o[NW][16][D + kPad];
  char* const stage = reinterpret_cast<char*>(&sm_o[w][0][0]);
  {
    const char* qp = reinterpret_cast<const char*>(P.q) + ((size_t)qrow * P.Hq + qh) * kRowBytes;
#pragma unroll
    for (int kk = 0; kk < kQK; ++kk) {
      uint4 u = ld16(qp + (32 * kk + 8 * rg) * 2);
      if (!col_ok) u = make_uint4(0, 0, 0, 0);
      qop[kk] = __builtin_bit_cast(bf16x8_t, u);
    }
  }

  // Context of each column (its row's causal prefix) and of the whole tile.
  const int ctx_col = sr.row_ctx(qi);                       // this lane's column
  const int ctx_min = sr.row_ctx(c_begin / P.G);            // first column's row
  const int ctx = sr.row_ctx((c_end - 1) / P.G);            // last column's row: the longest
  const bool bad_ctx = sr.bad || is.bad || is.start_blk * kBlock > ctx;
  const int nblk = (ctx + kBlock - 1) / kBlock;
  const int blk_end = bpp > 0 ? min(nblk, blk_begin + bpp) : nblk;
  const int span = nblk - is.start_blk;  // blocks this pass reads (tail pass: past the shared ones)
  const int nparts_s = bpp > 0 ? (span + bpp - 1) / bpp : (span > 0 ? 1 : 0);
  if (p >= max(nparts_s, 1)) return;  // partition past the tile's longest context

  float m = -INFINITY, lsum = 0.0f;
  f32x4_t acc[kTiles];
#pragma unroll
  for (int e = 0; e < kTiles; ++e) acc[e] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  bool bad = bad_ctx;   // the whole tile (wave-uniform)
  bool bad_me = false;  // this lane's column only (kFold: its member's own blocks)

  // kFold: lane j < members holds member j's context, its first own block and
  // how many of its own blocks this wave reads (blocks w, w + NW, ... of its
  // run), with the exclusive prefix sum of those counts; ttot = this wave's
  // own-block items, all members together.
  int m_ctx = 0, m_b0 = 0, m_cum = 0, ttot = 0;
  if constexpr (kFold) {
    const int nm = min(sr.n, P.max_q);  // 0 when the group's bounds are malformed
    int m_cnt = 0;
    bool m_bad = false;
    if (lane < nm) {
      m_ctx = P.context_lens[sr.first + lane];
      const int sh = P.seq_shared[sr.first + lane];
      m_bad = m_ctx < 0 || m_ctx > P.ctx_limit || sh < 0 || sh % kBlock != 0 || sh > m_ctx;
      m_b0 = m_bad ? 0 : sh / kBlock;
      const int own = m_bad ? 0 : (m_ctx + kBlock - 1) / kBlock - m_b0;
      m_cnt = own > w ? (own - w + NW - 1) / NW : 0;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int cj = __builtin_amdgcn_readlane(m_cnt, j);
      m_cum += j < lane ? cj : 0;
      ttot += cj;
    }
    bad_me = __shfl(m_bad ? 1 : 0, qi) != 0;
  }
  // kFold: block id and tag (member j << 27 | logical block) of this wave's
  // own-block item c0 + lane. Member j's items start at its prefix sum.
  auto own_item = [&](int c0, int& id, int& tag) {
    const int r = c0 + lane;
    int j = 0;  // the member whose items hold r (members with none are passed over)
#pragma unroll
    for (int mm = 1; mm < 16; ++mm) j += r >= __builtin_amdgcn_readlane(m_cum, mm) ? 1 : 0;
    const int b0 = __shfl(m_b0, j), cum = __shfl(m_cum, j);  // every lane takes part
    id = -1;
    tag = 0;
    if (r < ttot) {
      const int blk = b0 + w + NW * (r - cum);
      id = P.block_tables[(size_t)(sr.first + j) * P.MB + blk];
      tag = (j << 27) | blk;
    }
  };
  int oids0 = -1, otags0 = 0;
  if constexpr (kFold) own_item(0, oids0, otags0);  // in flight during the shared blocks

  const char* kbase = reinterpret_cast<const char*>(P.k_cache);
  const char* vbase = reinterpret_cast<const char*>(P.v_cache);
  const size_t head_off = (size_t)g * kBlock * kRowBytes;
  const size_t block_stride = (size_t)P.Hkv * kBlock * kRowBytes;
  // K and V tiles are loaded alike, four whole rows per load: lane holds
  // piece col (dims (kPiece / 2) col .. + kPiece / 2 - 1) of row 4 rg + j in
  // register j.
  const int row_lane = (4 * rg) * kRowBytes + col * kPiece;  // + 1 row per j

  // Issue the loads of physical block b's tile (logical block blk) into
  // (kb, vb). An id outside the pool marks the group bad and loads nothing;
  // so does a block that does not exist (an empty ring refill).
  auto load = [&](Piece (&kb)[4], Piece (&vb)[4], int b, int blk, bool exists) {
    const bool valid = b >= 0 && b < P.NB;
    bad |= exists && !valid;
    const size_t off = (size_t)(valid ? b : 0) * block_stride + head_off;
    // only the block's rows inside the context are fetched (the rest read as 0)
    const int rows = min(kBlock, ctx - blk * kBlock);
    const int bytes = exists && valid ? rows * kRowBytes : 0;
    const rsrc_t rk = make_rsrc(kbase + off, bytes);
    const rsrc_t rv = make_rsrc(vbase + off, bytes);
#pragma unroll
    for (int j = 0; j < 4; ++j) kb[j] = ld_piece<kPolicy, kPiece>(rk, row_lane + j * kRowBytes);
#pragma unroll
    for (int j = 0; j < 4; ++j) vb[j] = ld_piece<kPolicy, kPiece>(rv, row_lane + j * kRowBytes);
  };
  // kFold: member j's own block (tag): its rows inside the member's context;
  // an id outside the pool spoils only that member's columns.
  auto load_own = [&](Piece (&kb)[4], Piece (&vb)[4], int b, int tag, bool exists) {
    const int j = tag >> 27, blk = tag & ((1 << 27) - 1);
    const bool valid = b >= 0 && b < P.NB;
    bad_me |= exists && !valid && qi == j;
    const size_t off = (size_t)(valid ? b : 0) * block_stride + head_off;
    const int rows = min(kBlock, __builtin_amdgcn_readlane(m_ctx, j) - blk * kBlock);
    const int bytes = exists && valid ? rows * kRowBytes : 0;
    const rsrc_t rk = make_rsrc(kbase + off, bytes);
    const rsrc_t rv = make_rsrc(vbase + off, bytes);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      kb[jj] = ld_piece<kTailPolicy, kPiece>(rk, row_lane + jj * kRowBytes);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      vb[jj] = ld_piece<kTailPolicy, kPiece>(rv, row_lane + jj * kRowBytes);
  };

  // One tile: S^T, the online-softmax update and O^T += V^T P^T. When
  // `partial`, this lane's tokens 4 rg + i at or past `lim` (tile-local) are
  // masked.
  auto consume = [&](const Piece (&kb)[4], const Piece (&vbin)[4], bool partial, int lim) {
    // Transpose K through the wave's LDS stage into the A operand layout:
    // step kk needs, in lane (rg, col), dims 32 kk + 8 rg .. + 7 (16-byte
    // chunk 4 kk + rg) of row t = col. Rows are kStageRow apart (the row plus
    // 16 B of padding), so both the row writes and the strided reads are
    // free of bank conflicts.
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<Piece*>(stage + (4 * rg + j) * kStageRow + col * kPiece) = kb[j];
    f32x4_t st = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < kQK; ++kk) {
      const uint4 ka = *reinterpret_cast<const uint4*>(stage + col * kStageRow + (4 * kk + rg) * 16);
      st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka), qop[kk], st,
                                                  0, 0, 0);
    }
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = st[i] * P.qscale;
      if (partial && 4 * rg + i >= lim) x[i] = -INFINITY;
    }
    // Rows at or past the tile's longest context were not fetched (the tile's
    // buffer range ends there) and read as zeros, never as stale or NaN data.
    const Piece (&vb)[4] = vbin;
    const float mx = rows_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = exp2_fast(m - m_use);
    // The accumulators need rescaling only when some column's max rose; for
    // the others alpha is exactly 2^0 = 1, so skipping is bit-identical.
    const bool rescale = __builtin_amdgcn_ballot_w64(m_new > m) != 0;
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = exp2_fast(x[i] - m_use);
    lsum = lsum * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
    m = m_new;
    if (rescale) {
#pragma unroll
      for (int e = 0; e < kTiles; ++e) acc[e] *= alpha;
    }
    const uint32_t p01 = pack_bf16x2(pr[0], pr[1]);
    const uint32_t p23 = pack_bf16x2(pr[2], pr[3]);
    const s16x4_t pop = __builtin_bit_cast(s16x4_t, make_uint2(p01, p23));
#pragma unroll
    for (int k = 0; k < kPiece / 4; ++k) {  // 32-bit word k of each V piece: dims 2k, 2k+1
      const uint32_t w0 = word(vb[0], k), w1 = word(vb[1], k);
      const uint32_t w2 = word(vb[2], k), w3 = word(vb[3], k);
      const s16x4_t a_lo = __builtin_bit_cast(s16x4_t, make_uint2(pack_lo16(w0, w1), pack_lo16(w2, w3)));
      const s16x4_t a_hi = __builtin_bit_cast(s16x4_t, make_uint2(pack_hi16(w0, w1), pack_hi16(w2, w3)));
      acc[2 * k] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_lo, pop, acc[2 * k], 0, 0, 0);
      acc[2 * k + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_hi, pop, acc[2 * k + 1], 0, 0, 0);
    }
  };

  // This wave's blocks: first + k * kStride, k < nk, through a ring of DEPTH tiles.
  {
    const int nk = first < blk_end ? (blk_end - first + kStride - 1) / kStride : 0;
    // tail pass: skip this wave's blocks inside the shared part
    const int k0 = is.start_blk > first ? (is.start_blk - first + kStride - 1) / kStride : 0;
    Piece kb[DEPTH][4], vb[DEPTH][4];
    block_pipeline<DEPTH>(
        bt_row, first, kStride, k0, nk, lane, ids0,
        [&](int d, int b, int k, bool exists) {
          load(kb[d], vb[d], b, first + k * kStride, exists);
        },
        [&](int d, int k) {
          const int blk = first + k * kStride;
          // some column masks some row of this block (wave-uniform)
          consume(kb[d], vb[d], blk * kBlock + kBlock > ctx_min, ctx_col - blk * kBlock);
        });
    if constexpr (kFold) {
      list_pipeline<DEPTH>(
          ttot, lane, oids0, otags0, own_item,
          [&](int d, int b, int tag, bool exists) { load_own(kb[d], vb[d], b, tag, exists); },
          [&](int d, int tag) {
            const int j = tag >> 27, blk = tag & ((1 << 27) - 1);
            const int lim = qi == j ? __builtin_amdgcn_readlane(m_ctx, j) - blk * kBlock : 0;
            consume(kb[d], vb[d], true, lim);
          });
    }
  }

  lsum = rows_sum(lsum);  // per column: sum over the 4 row groups

  // Waves -> LDS -> one merged state per (head, dim).
  __shared__ float sm_m[NW][16], sm_l[NW][16];
  __shared__ int sm_bad[NW];
  __shared__ int sm_badc[kFold ? NW : 1][16];  // kFold: per column
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float* dst = &sm_o[w][col][kTiles * (4 * rg + i)];
    // tile e holds dim kTiles (4 rg + i) + e
#pragma unroll
    for (int e4 = 0; e4 < kTiles; e4 += 4)
      *reinterpret_cast<float4*>(dst + e4) =
          make_float4(acc[e4][i], acc[e4 + 1][i], acc[e4 + 2][i], acc[e4 + 3][i]);
  }
  if (rg == 0) {
    sm_m[w][col] = m;
    sm_l[w][col] = lsum;
    if constexpr (kFold) sm_badc[w][col] = bad_me ? 1 : 0;
  }
  if (lane == 0) sm_bad[w] = bad ? 1 : 0;
  __syncthreads();

  bool any_bad = false;
#pragma unroll
  for (int v = 0; v < NW; ++v) any_bad |= sm_bad[v] != 0;
  // thread -> (column qq, 8-dim chunk ch): a column's D / 8 threads are
  // consecutive lanes
  constexpr int kChunks = D / 8;
  for (int t = threadIdx.x; t < 16 * kChunks; t += NW * kWave) {
    const int qq = t / kChunks, ch = t % kChunks;
    const int c = c_begin + qq;
    if (c >= c_end) continue;
    const int i = c / P.G;
    const int h = g * P.G + c % P.G;
    // Partitions of this column's own context: with one, partition 0 writes
    // the final row; with several, each writes its partial.
    const int cblk = (sr.row_ctx(i) + kBlock - 1) / kBlock - is.start_blk;
    const int np = bpp > 0 ? (cblk + bpp - 1) / bpp : 1;
    if (np <= 1 ? p != 0 : p >= np) continue;
    bool col_bad = any_bad;
    if constexpr (kFold) {
#pragma unroll
      for (int v = 0; v < NW; ++v) col_bad |= sm_badc[v][qq] != 0;
    }
    float M = sm_m[0][qq];
#pragma unroll
    for (int v = 1; v < NW; ++v) M = fmaxf(M, sm_m[v][qq]);
    const float m_use = (M == -INFINITY) ? 0.0f : M;
    float L = 0.0f, ov[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ov[e] = 0.0f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const float sc = exp2_fast(sm_m[v][qq] - m_use);
      L += sm_l[v][qq] * sc;
#pragma unroll
      for (int e = 0; e < 8; ++e) ov[e] += sm_o[v][qq][8 * ch + e] * sc;
    }
    const size_t row = (size_t)(sr.first + i);
    // Several partitions of this column's context, or the group pass of a
    // shared prefix: write this partition's partial and its (m, l); else the
    // final row (the tail pass first folds in the group pass's partials of
    // the row).
    if (np > 1 || P.always_partial) {
      // fp16 partial (see PartScale); a column's lanes lie in one DPP row
      float amax = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(ov[e]));
      const PartScale ps = part_scale_f16(M, L, group_max<kChunks>(amax));
      uint4 u;
      u.x = pack_f16x2(ov[0] * ps.mul, ov[1] * ps.mul);
      u.y = pack_f16x2(ov[2] * ps.mul, ov[3] * ps.mul);
      u.z = pack_f16x2(ov[4] * ps.mul, ov[5] * ps.mul);
      u.w = pack_f16x2(ov[6] * ps.mul, ov[7] * ps.mul);
      if (any_bad) u = make_uint4(0x7e007e00u, 0x7e007e00u, 0x7e007e00u, 0x7e007e00u);  // NaN
      const size_t part = part_slot(P, row, h, P.part_base + p);
      store_part16(P, row, h, P.part_base + p, 2, 8 * ch * 2, u);
      if (ch == 0) {
        P.ws_ml[2 * part] = any_bad ? 0.0f : ps.m;
        P.ws_ml[2 * part + 1] = any_bad ? __builtin_nanf("") : ps.l;
      }
    } else {
      if (P.tail_pass)
        merge_shared_partials<uint16_t, 8>(P, is.bad ? 0 : is.start_blk * kBlock, row, h, 8 * ch,
                                           D, M, L, ov);
      const float inv = L > 0.0f ? 1.0f / L : 0.0f;
      float res[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) res[e] = col_bad ? __builtin_nanf("") : ov[e] * inv;
      uint4 u;
      u.x = pack_bf16x2(res[0], res[1]);
      u.y = pack_bf16x2(res[2], res[3]);
      u.z = pack_bf16x2(res[4], res[5]);
      u.w = pack_bf16x2(res[6], res[7]);
      st16(reinterpret_cast<char*>(P.out) + ((row * P.Hq + h) * D + 8 * ch) * 2, u);
    }
  }
}

hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t stream) {
  // several column tiles per kv head: the chunk kernel, whose waves share
  // each block
  if (p.n_tiles >= PA_CHUNK_MIN_TILES) return launch_chunk_mfma(p, stream);
  constexpr int DEPTH = PA_MFMA_DEPTH;
  if (p.fold_tails) {
    // group pass with the members' own blocks folded in: the shared blocks'
    // policy from shared_kv, the own blocks' from tail_shared_kv
    auto fold = [&](auto d, auto nw) {
      constexpr int HD = decltype(d)::value;
      constexpr int NW = decltype(nw)::value;
      constexpr TilePolicy S = TilePolicy::kShared, T = TilePolicy::kStream;
      const dim3 grid(p.Hkv, 1, p.pass_items), block(NW * kWave);
      if (p.shared_kv && p.tail_shared_kv)
        hipLaunchKernelGGL((decode_mfma_kernel<HD, NW, DEPTH, S, true, S>), grid, block, 0,
                           stream, p);
      else if (p.shared_kv)
        hipLaunchKernelGGL((decode_mfma_kernel<HD, NW, DEPTH, S, true, T>), grid, block, 0,
                           stream, p);
      else if (p.tail_shared_kv)
        hipLaunchKernelGGL((decode_mfma_kernel<HD, NW, DEPTH, T, true, S>), grid, block, 0,
                           stream, p);
      else
        hipLaunchKernelGGL((decode_mfma_kernel<HD, NW, DEPTH, T, true, T>), grid, block, 0,
                           stream, p);
    };
    auto fold_waves = [&](auto d) {
      if ((int64_t)p.Hkv * p.pass_items <= p.n_cus)
        fold(d, std::integral_constant<int, PA_MFMA_FOLD_WAVES_FEW>{});
      else
        fold(d, std::integral_constant<int, PA_MFMA_FOLD_WAVES>{});
    };
    if (p.D == 128)
      fold_waves(std::integral_constant<int, 128>{});
    else if (p.D == 64)
      fold_waves(std::integral_constant<int, 64>{});
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  auto go = [&](auto d, auto nw) {
    constexpr int HD = decltype(d)::value;
    constexpr int NW = decltype(nw)::value;
    const dim3 grid(p.Hkv * p.n_tiles, p.pass_parts, p.pass_items), block(NW * kWave);
    if (p.shared_kv)
      hipLaunchKernelGGL((decode_mfma_kernel<HD, NW, DEPTH, TilePolicy::kShared>), grid, block, 0,
                         stream, p);
    else
      hipLaunchKernelGGL((decode_mfma_kernel<HD, NW, DEPTH, TilePolicy::kStream>), grid, block, 0,
                         stream, p);
  };
  auto by_waves = [&](auto d) {
    // A whole context per workgroup: more waves, each with a longer share of
    // its blocks. Split contexts (a partition's few blocks): fewer.
    if (p.group_start)
      go(d, std::integral_constant<int, PA_MFMA_GROUP_WAVES>{});
    else if (p.tail_pass)
      go(d, std::integral_constant<int, PA_MFMA_TAIL_WAVES>{});
    else if (p.pass_parts == 1)
      go(d, std::integral_constant<int, PA_MFMA_WAVES_UNSPLIT>{});
    else
      go(d, std::integral_constant<int, PA_MFMA_WAVES>{});
  };
  if (p.D == 128)
    by_waves(std::integral_constant<int, 128>{});
  else if (p.D == 64)
    by_waves(std::integral_constant<int, 64>{});
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
