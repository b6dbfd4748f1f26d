// Paged attention of many query columns per kv head on the matrix cores
// (bf16, head_dim 128 or 64): chunked prefill, or many drafted tokens per
// sequence.
//
// Method: as the decode kernels ("Why OS Virtual Memory Paging Saved LLM
// Inference" (a8q9.cn), section 2: K/V gathered block by block through the
// block table; online softmax over the blocks), with the causal limit of
// each new token ("vLLM & PagedAttention" (completesystemdesign.dev),
// section 01: a token attends to every earlier token and to itself).
//
// Columns: the n x G (query row, head of the group) pairs of a sequence and
// kv head, row-major, cut into tiles of 16, in the column layout of the
// decode MFMA kernel (S^T = K Q^T on v_mfma_f32_16x16x32_bf16; every
// accumulator a lane holds belongs to its own column). A workgroup of NW
// waves owns NW x TPW consecutive tiles, TPW per wave (one, or two for long
// chunks, which halves the LDS reads per flop), and each wave keeps its
// tiles' online-softmax states to the end.
//
// The waves stream the partition's K/V blocks, two at a time, through an LDS
// ring of R slots. A slot holds a pair of blocks A, B: K tiles (4 KiB each at
// head_dim 128, 2 KiB at 64) then V tiles, written by the loads themselves
// (buffer_load ... lds) in 1 KiB pieces (sixteen, or eight), one load
// instruction each, shared out over the waves: every byte crosses the vector memory path once per workgroup, not
// once per wave (the per-wave loads of a column tile kept that path busy
// most of the time). One barrier per pair publishes the slot and frees the
// previous one. Taking blocks in pairs makes O^T = V^T P^T one K = 32
// contraction (v_mfma_f32_16x16x32_bf16, the full-rate form) instead of two
// K = 16 ones, and halves the softmax's per-lane work per block. Output tile
// et of the PV product holds dims 16 et + 0..15 (row m: dim 16 et + m).
//
// LDS image of a tile (16 rows of 2 D bytes, in 16-byte chunks), row r at
// r * 2 D, each row's chunks permuted by the swizzle of Ring (chunk_ring.h):
//   K: the loads still read whole rows (a lane picks the chunk its position
//     holds), and the MFMA operand reads (chunk 4 kk + rg of row col, for
//     the 16 lanes of a row group) fall on 16 different bank groups, so
//     neither side conflicts;
//   V: the operand comes from transposing LDS reads (ds_read_b64_tr_b16),
//     each 16-lane group naming 32 bytes (chunks 2 et, 2 et + 1) of 4 rows;
//     the swizzle puts the chunk pairs of any 8 consecutive rows on
//     different bank groups (with K's swizzle, two rows 8 apart met).
// Lanes of a load past the block's rows inside the context write zeros.
#include "pa_device.h"
#include "pa_launch.h"
#include "chunk_ring.h"

// The register allocation's minimum waves per SIMD (8-wave, one-tile kernel).
#ifndef PA_CHUNK_MIN_WAVES
#define PA_CHUNK_MIN_WAVES 4
#endif
// Most waves per workgroup (2, 4 or 8).
#ifndef PA_CHUNK_MAX_WAVES
#define PA_CHUNK_MAX_WAVES 8
#endif
// Wave priority raised while a wave issues its S^T products (1), or never (0).
#ifndef PA_CHUNK_PRIO
#define PA_CHUNK_PRIO 0
#endif
// Column tiles (16 columns each) per wave for more than 8 tiles per kv
// head: 2 (on 4 waves) or 1 (on 8 waves).
#ifndef PA_CHUNK_TILES_PER_WAVE
#define PA_CHUNK_TILES_PER_WAVE 2
#endif

namespace pa {

template <int D, int NW, int R, int TPW, TilePolicy kPolicy>
__global__ __launch_bounds__(NW * kWave)
__attribute__((amdgpu_waves_per_eu(TPW > 1 ? 3 : NW >= 8 ? PA_CHUNK_MIN_WAVES : NW == 4 ? 3 : 2)))
void chunk_mfma_kernel(DecodeParams P) {
  using RG = Ring<D>;
  constexpr int kRowBytes = RG::kRowBytes;
  constexpr int kTileBytes = RG::kTileBytes;
  constexpr int kSlotBytes = RG::kSlotBytes;
  constexpr int kPieceBytes = RG::kPieceBytes;
  constexpr int kPieces = RG::kPieces;
  constexpr int kK = D / 32;  // contraction steps of S^T (32 dims each)
  constexpr int kE = D / 16;  // 16-dim output tiles of O^T
  static_assert(kPieces % NW == 0, "pieces must divide over the waves");
  static_assert(R >= 3 && R <= 4, "ring of 3 or 4 slots");
  static_assert(TPW == 1 || TPW == 2, "one or two column tiles per wave");
  constexpr int kPer = kPieces / NW;  // load instructions per wave per pair
  // One LDS object per slot, so that the compiler's load counting tells the
  // slots apart and waits only for the slot it reads.
  __shared__ __attribute__((aligned(16))) char ring0[kSlotBytes];
  __shared__ __attribute__((aligned(16))) char ring1[kSlotBytes];
  __shared__ __attribute__((aligned(16))) char ring2[R > 2 ? kSlotBytes : 16];
  __shared__ __attribute__((aligned(16))) char ring3[R > 3 ? kSlotBytes : 16];
  auto slot = [&](int d) -> char* {
    return d == 0 ? ring0 : d == 1 ? ring1 : d == 2 ? ring2 : ring3;
  };

  const int lane = threadIdx.x & (kWave - 1);
  const int w = wave_id();
  const int col = lane & 15;
  const int rg = lane >> 4;

  // Workgroups per (kv head, partition, sequence); those of one such triple
  // read the same K/V and are kept on one XCD.
  constexpr int kTilesPerWg = NW * TPW;
  const int groups = (P.n_tiles + kTilesPerWg - 1) / kTilesPerWg;
  const GridPos gp = grid_pos_grouped(groups);
  const int p = gp.y;
  const int s = gp.z;
  const int g = gp.x / groups;                     // kv head
  const int tile0 = (gp.x % groups) * kTilesPerWg;  // the workgroup's first tile

  // (the group pass of shared-prefix decode reads a group's shared blocks
  // through its first member's table; this kernel runs no tail pass)
  const ItemStart is = item_start(P, s);
  const int32_t* bt_row = P.block_tables + (size_t)is.trow * P.MB;
  const int bpp = P.partition / kBlock;  // blocks per partition (0: no split)
  const int blk_begin = p * bpp;
  const int ids0 =
      first_chunk_ids(bt_row, blk_begin, 1, bpp > 0 ? min(P.MB, blk_begin + bpp) : P.MB, lane);
  const SeqRows sr = seq_rows(P, s);

  // Columns: global column gc of the n x G grid, row-major; gc >= n G is
  // padding. Wave w owns tiles tile0 + TPW w + t, t < TPW.
  const int ncols = min(sr.n, P.max_q) * P.G;
  const int wg_begin = 16 * tile0;
  if (wg_begin >= ncols) return;  // the whole workgroup is padding
  const int wg_end = min(ncols, wg_begin + 16 * kTilesPerWg);
  const bool has_cols = 16 * (tile0 + TPW * w) < ncols;  // else the wave only loads (wave-uniform)

  // The logit scale (log2 domain) is applied in the exponent, after the max
  // is taken over the raw products, which needs it non-negative: a negative
  // scale flips the sign bits of Q instead (exact), and a zero scale becomes
  // a tiny positive one (every logit still rounds to 0).
  const bool q_neg = P.qscale < 0.0f;
  const float qs = fmaxf(fabsf(P.qscale), 1e-30f);

  // Per tile: this lane's column (padded lanes, and all lanes of a tile past
  // the last column, shadow a real column and carry a zero query), its
  // causal context, the tile's shortest context, and the B operand of S^T,
  // Q[column col][32 kk + 8 rg ..].
  int gc[TPW], ctx_col[TPW], ctx_min[TPW];
  bool col_ok[TPW];
  bf16x8_t qop[TPW][kK];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int cb = 16 * (tile0 + TPW * w + t);
    const bool tile_ok = cb < ncols;
    const int ce = tile_ok ? min(ncols, cb + 16) : wg_end;
    gc[t] = cb + col;
    col_ok[t] = tile_ok && gc[t] < ce;
    const int gcl = col_ok[t] ? gc[t] : ce - 1;
    const int qi = gcl / P.G;
    const int qh = g * P.G + gcl % P.G;
    ctx_col[t] = sr.row_ctx(qi);
    ctx_min[t] = sr.row_ctx((tile_ok ? cb : ce - 1) / P.G);
    if (has_cols) {
      const char* qp =
          reinterpret_cast<const char*>(P.q) + ((size_t)(sr.first + qi) * P.Hq + qh) * kRowBytes;
      const uint32_t flip = q_neg ? 0x80008000u : 0u;
#pragma unroll
      for (int kk = 0; kk < kK; ++kk) {
        uint4 u = ld16(qp + (32 * kk + 8 * rg) * 2);
        u = make_uint4(u.x ^ flip, u.y ^ flip, u.z ^ flip, u.w ^ flip);
        if (!col_ok[t]) u = make_uint4(0, 0, 0, 0);
        qop[t][kk] = __builtin_bit_cast(bf16x8_t, u);
      }
    }
  }

  // The workgroup's longest context: what the ring streams.
  const int ctx_wg = sr.row_ctx((wg_end - 1) / P.G);
  const int nblk = (ctx_wg + kBlock - 1) / kBlock;
  const int blk_end = bpp > 0 ? min(nblk, blk_begin + bpp) : nblk;
  const int nparts_wg = bpp > 0 ? (nblk + bpp - 1) / bpp : (nblk > 0 ? 1 : 0);
  if (p >= max(nparts_wg, 1)) return;  // partition past the workgroup's contexts

  // The reference m (what the probabilities are taken relative to) moves
  // only when a column's max passes it by more than kLazy: the
  // probabilities then stay below 2^kLazy, the result is the same up to
  // rounding, and the accumulators are rescaled a few times per column
  // instead of whenever its max creeps up. mlazy = m + kLazy, kept with m.
  constexpr float kLazy = 8.0f;
  float m[TPW], mlazy[TPW], lsum[TPW];
  f32x4_t acc[TPW][kE];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    m[t] = kNoRef;
    mlazy[t] = kNoRef + kLazy;
    lsum[t] = 0.0f;
#pragma unroll
    for (int e = 0; e < kE; ++e) acc[t][e] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }
  bool bad = sr.bad || is.bad;

  const char* kbase = reinterpret_cast<const char*>(P.k_cache);
  const char* vbase = reinterpret_cast<const char*>(P.v_cache);
  const size_t head_off = (size_t)g * kTileBytes;
  const size_t block_stride = (size_t)P.Hkv * kTileBytes;

  // This wave's pieces of every pair: piece q = kPer w + i of the slot (at q
  // KiB into it) holds kRowsPerPiece consecutive rows of tile
  // q / kPiecesPerTile (0: K of block A, 1: K of block B, 2: V of A, 3: V of
  // B); lane l writes position l % kChunks of row l / kChunks of the piece,
  // so it loads the chunk that the tile's swizzle (Ring::k_pos, v_pos) puts
  // there.
  constexpr int kPiecesPerTile = RG::kPiecesPerTile;
  int piece_off[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int q = kPer * w + i;
    const int r = RG::kRowsPerPiece * (q % kPiecesPerTile) + lane / RG::kChunks;
    const int pos = lane % RG::kChunks;
    const bool v_tile = q / kPiecesPerTile >= 2;
    piece_off[i] = r * kRowBytes + (v_tile ? RG::v_pos(r, pos) : RG::k_pos(r, pos)) * 16;
  }

  // Transposed V reads (ds_read_b64_tr_b16): in each group of 16 lanes, lane
  // t names 4 consecutive bf16 (row t of a 16 x 4 block) and lane i receives
  // element (row 4 e + i / 4, column i % 4) for e = 0..3. Lane (rg, col)
  // names row 4 rg + col / 4 of the V tile at dims 16 et + 4 (col % 4) ..
  // + 3, so it receives V[4 rg + e][16 et + col], e = 0..3: its operand of
  // output tile et, row m = col standing for dim 16 et + col. Offsets within
  // a (swizzled) V tile, per tile et:
  int vtr_off[kE];
#pragma unroll
  for (int et = 0; et < kE; ++et) {
    const int r = 4 * rg + col / 4;
    const int dim = 16 * et + 4 * (col % 4);
    vtr_off[et] = r * kRowBytes + RG::v_pos(r, dim / 8) * 16 + (dim % 8) * 2;
  }

  // Load the pair of blocks at lanes i, i + 1 of the current 64-block chunk
  // into slot d. Per lane of the chunk, off_lo/off_hi hold its tile's byte
  // offset in the pool and nbytes the bytes to fetch: the rows inside the
  // workgroup's context, or nothing for a bad id or a block past the chunk
  // (an empty refill past the last pair, kept so that every step issues the
  // same number of loads).
  auto issue = [&](int d, int i, int cn, uint32_t off_lo, uint32_t off_hi, int nbytes) {
    // The descriptor of tile t (0: K of A, 1: K of B, 2: V of A, 3: V of B),
    // built only for the tiles this wave's pieces belong to.
    auto rsrc_of = [&](int t) {
      const int li = i + (t & 1);
      const int lc = min(li, kWave - 1);
      const uint64_t off = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)off_hi, lc) << 32) |
                           (uint32_t)__builtin_amdgcn_readlane((int)off_lo, lc);
      const int bytes = li < cn ? __builtin_amdgcn_readlane(nbytes, lc) : 0;
      return make_rsrc((t >= 2 ? vbase : kbase) + off, bytes);
    };
    char* dst = slot(d);
    if constexpr (kPer <= kPiecesPerTile) {
      // all of the wave's pieces lie in one tile: one descriptor
      const rsrc_t r = rsrc_of((kPer * w) / kPiecesPerTile);
#pragma unroll
      for (int q = 0; q < kPer; ++q)
        ld16_lds<kPolicy>(r, dst + (kPer * w + q) * kPieceBytes, piece_off[q]);
    } else {
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int pc = kPer * w + q;
        ld16_lds<kPolicy>(rsrc_of(pc / kPiecesPerTile), dst + pc * kPieceBytes, piece_off[q]);
      }
    }
  };

  // Transposed V operand of output tile et from slot src: the A operand of
  // lane (rg, col) is V_A[4 rg + 0..3][16 et + col] then
  // V_B[4 rg + 0..3][16 et + col].
  typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
  auto v_operand = [&](const char* src, int et) {
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(__attribute__((address_space(3))) char*)(src + 2 * kTileBytes + vtr_off[et]));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(__attribute__((address_space(3))) char*)(src + 3 * kTileBytes + vtr_off[et]));
    const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
    return __builtin_bit_cast(bf16x8_t, make_uint4(l2.x, l2.y, h2.x, h2.y));
  };

  // Logits of tile t past the column's causal limit, and all of block B
  // when it lies past the partition, removed (lane (rg, col): tokens
  // 4 rg + 0..3 of each block).
  auto mask_logits = [&](int t, float (&x)[8], int blk, bool b_live) {
    const int tok0 = blk * kBlock + 4 * rg;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (tok0 + i >= ctx_col[t]) x[i] = -INFINITY;
      if (!b_live || tok0 + kBlock + i >= ctx_col[t]) x[4 + i] = -INFINITY;
    }
  };
  // The online softmax of tile t over one pair of blocks, from its raw
  // logits x (S^T of block A, then of block B), in two steps: move the
  // tile's reference where a column's max passed it (reference_from), then
  // take the probabilities against the reference (probs).
  //
  // A lane's largest logit of the pair, chained so that each two maxima
  // become one three-input maximum: 4 instructions for 8 values.
  auto lane_max = [](const float (&x)[8]) {
    const float a = vmax(vmax(x[0], x[1]), x[2]);
    const float b = vmax(vmax(x[3], x[4]), x[5]);
    return vmax(vmax(vmax(x[6], x[7]), a), b);
  };
  // Whether this lane's logits of tile t (lane max lm) pass the reference by
  // more than kLazy. Where no lane of the wave does, no column's reference
  // moves (a column's max is its lanes' largest, and rounding the product
  // with qs > 0 keeps the order): the reference step can be skipped, since
  // its alpha would be exactly 1.
  auto passes = [&](int t, float lm) { return lm * qs > mlazy[t]; };
  // col_max: the column's largest raw logit over the pair (all 4 row
  // groups). Moves the reference if that passes it by more than kLazy and
  // scales the tile's sum to the new reference; returns the factor alpha
  // that takes the accumulators there (sets up when it is not 1).
  auto reference_from = [&](int t, float col_max, bool& up) {
    const float mx = col_max * qs;  // -inf stays -inf (qs > 0)
    const float m_new = vmax(m[t], mx);
    up = m_new > mlazy[t];  // from kNoRef: any finite max
    const float ref = up ? m_new : m[t];
    // Exactly 1 where the reference stays; 0 (or 2^-inf) from kNoRef, where
    // the accumulators hold nothing yet.
    const float alpha = exp2_fast(m[t] - ref);
    m[t] = ref;
    mlazy[t] = ref + kLazy;
    lsum[t] *= alpha;
    return alpha;
  };
  // Probabilities of tile t against its reference, as the bf16 B operand of
  // the PV product, added to the tile's sum. The sum takes the
  // probabilities as rounded for the PV product (a dot product of each bf16
  // pair with (1, 1)): numerator and denominator see the same values, in 4
  // instructions instead of 8.
  auto probs = [&](int t, const float (&x)[8]) -> bf16x8_t {
    float pr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) pr[i] = exp2_fast(__builtin_fmaf(x[i], qs, -m[t]));
    const uint4 w4 = make_uint4(pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                                pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7]));
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
    float l = lsum[t];
    l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w4.x), ones, l, false);
    l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w4.y), ones, l, false);
    l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w4.z), ones, l, false);
    l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w4.w), ones, l, false);
    lsum[t] = l;
    return __builtin_bit_cast(bf16x8_t, w4);
  };
  // Raw logits of tile t (S^T of blocks A then B).
  auto logits = [&](const f32x4_t& sa, const f32x4_t& sb, float (&x)[8]) {
    const float v[8] = {sa[0], sa[1], sa[2], sa[3], sb[0], sb[1], sb[2], sb[3]};
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = v[i];
  };

  // One pair of blocks in slot d, for each of the wave's tiles: S^T of both
  // blocks (lane (rg, col) holds tokens 4 rg + 0..3 of each, column col),
  // the online softmax over their 32 tokens, then O^T += V^T P^T as one
  // K = 32 contraction: contraction slots 8 rg + 0..3 are block A's tokens
  // 4 rg + 0..3 and slots 8 rg + 4..7 block B's, so a lane's own
  // probabilities are its B operand as they stand. The K and V operands are
  // read once for all the wave's tiles. Pairs that reach a column's causal
  // limit, or whose block B is past the partition, are masked (a
  // wave-uniform branch, taken on few pairs).
  auto consume = [&](int d, int blk, bool b_live) {
    bool edge = !b_live;
#pragma unroll
    for (int t = 0; t < TPW; ++t) edge |= blk * kBlock + 2 * kBlock > ctx_min[t];
    const char* src = slot(d);
    f32x4_t sa[TPW], sb[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      sa[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      sb[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
    if constexpr (PA_CHUNK_PRIO != 0) __builtin_amdgcn_s_setprio(PA_CHUNK_PRIO);
#pragma unroll
    for (int kk = 0; kk < kK; ++kk) {
      const int o = col * kRowBytes + RG::k_pos(col, 4 * kk + rg) * 16;
      const bf16x8_t ka = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(src + o));
      const bf16x8_t kb =
          __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(src + kTileBytes + o));
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        sa[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qop[t][kk], sa[t], 0, 0, 0);
        sb[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qop[t][kk], sb[t], 0, 0, 0);
      }
    }
    if constexpr (PA_CHUNK_PRIO != 0) __builtin_amdgcn_s_setprio(0);
    if constexpr (TPW == 1) {
      // V operands read now, so that their latency passes under the softmax.
      bf16x8_t vop[kE];
#pragma unroll
      for (int et = 0; et < kE; ++et) vop[et] = v_operand(src, et);
      float x0[8];
      logits(sa[0], sb[0], x0);
      if (edge) mask_logits(0, x0, blk, b_live);
      const float lm0 = lane_max(x0);
      if (__builtin_amdgcn_ballot_w64(passes(0, lm0)) != 0) {
        bool up0;
        const float a0 = reference_from(0, rows_vmax(lm0), up0);
        if (__builtin_amdgcn_ballot_w64(up0) != 0) {
#pragma unroll
          for (int e = 0; e < kE; ++e) acc[0][e] *= a0;
        }
      }
      const bf16x8_t pop0 = probs(0, x0);
#pragma unroll
      for (int et = 0; et < kE; ++et)
        acc[0][et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[et], pop0, acc[0][et], 0, 0, 0);
    } else {
      // Both tiles' softmax together (one mask branch, and the two
      // dependency chains overlap). On most pairs one wave-wide test shows
      // that neither tile's reference moves; otherwise both tiles' column
      // maxima come from one lane exchange, and one branch rescales both
      // where either's reference moved (the other's alpha is then exactly 1).
      // Then the probabilities, and each V operand read just before its two
      // MFMAs (registers are short with two tiles).
      float x0[8], x1[8];
      logits(sa[0], sb[0], x0);
      logits(sa[1], sb[1], x1);
      if (edge) {
        mask_logits(0, x0, blk, b_live);
        mask_logits(1, x1, blk, b_live);
      }
      const float lm0 = lane_max(x0), lm1 = lane_max(x1);
      if (__builtin_amdgcn_ballot_w64(passes(0, lm0) || passes(1, lm1)) != 0) {
        float cm0, cm1;
        rows_vmax2(lm0, lm1, cm0, cm1);
        bool up0, up1;
        const float a0 = reference_from(0, cm0, up0);
        const float a1 = reference_from(1, cm1, up1);
        if (__builtin_amdgcn_ballot_w64(up0 || up1) != 0) {
#pragma unroll
          for (int e = 0; e < kE; ++e) {
            acc[0][e] *= a0;
            acc[1][e] *= a1;
          }
        }
      }
      const bf16x8_t pop0 = probs(0, x0), pop1 = probs(1, x1);
#pragma unroll
      for (int et = 0; et < kE; ++et) {
        const bf16x8_t v = v_operand(src, et);
        acc[0][et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, pop0, acc[0][et], 0, 0, 0);
        acc[1][et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, pop1, acc[1][et], 0, 0, 0);
      }
    }
  };

  // The ring: pair j (blocks 2 j, 2 j + 1 of the partition's range) sits in
  // slot j % R. Before pair j is read, each wave waits for its own pieces of
  // it (the R - 2 pairs issued after it may stay in flight), then a barrier
  // makes every wave's pieces visible and shows that every wave is done with
  // pair j - 1, whose slot takes pair j + R - 1. Block ids are read 64 at a
  // time: lane i holds the chunk's i-th block (its pool offset and byte
  // count, read per pair with readlane). The ring drains at each chunk's end.
  const int nk = max(0, blk_end - blk_begin);
  for (int c0 = 0; c0 < nk; c0 += kWave) {
    const int cn = min(kWave, nk - c0);  // blocks in this chunk
    const int pn = (cn + 1) / 2;         // pairs
    if (c0 > 0) ring_barrier();          // every wave is done with the previous chunk's slots
    const int ids = c0 == 0 ? ids0 : (lane < cn ? bt_row[blk_begin + c0 + lane] : -1);
    // Lane i: block c0 + i of the range. An id outside the pool marks the
    // columns bad and loads nothing; only rows inside the workgroup's context
    // are fetched (a block that exists starts inside it: at least one row).
    const bool ok_id = ids >= 0 && ids < P.NB;
    if (__builtin_amdgcn_ballot_w64(lane < cn && !ok_id) != 0) bad = true;
    const uint64_t off = (uint64_t)(uint32_t)(ok_id ? ids : 0) * block_stride + head_off;
    const int nbytes =
        lane < cn && ok_id ? min(kBlock, ctx_wg - (blk_begin + c0 + lane) * kBlock) * kRowBytes : 0;
    const uint32_t off_lo = (uint32_t)off, off_hi = (uint32_t)(off >> 32);
    auto issue_pair = [&](int d, int j) { issue(d, 2 * j, cn, off_lo, off_hi, nbytes); };
#pragma unroll
    for (int d = 0; d < R - 1; ++d) issue_pair(d, d);
    // Steps past the chunk's last pair still wait, meet and refill (with
    // empty loads): a refill under a branch costs the compiler its record of
    // which slot each load writes, and then it waits for every slot.
    for (int j0 = 0; j0 < pn; j0 += R) {
#pragma unroll
      for (int d = 0; d < R; ++d) {
        const int j = j0 + d;
        wait_vmcnt<(R - 2) * kPer>();
        ring_barrier();
        issue_pair((d + R - 1) % R, j + R - 1);
        if (has_cols && j < pn) consume(d, blk_begin + c0 + 2 * j, 2 * j + 1 < cn);
      }
    }
  }

  if (!has_cols) return;
  // Each tile's columns hold their whole state for this partition: lane
  // (rg, col) writes dims 16 et + 4 rg + 0..3 of its column, from acc[t][et].
  // A partial goes out as an fp16 row of an equivalent rescaled state
  // (part_scale_f16), as the decode kernels write theirs.
  const float nan = __builtin_nanf("");
  const bool split = bpp > 0 || P.always_partial;  // some column may write a partial
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const float l_col = rows_sum(lsum[t]);  // per column: sum over the 4 row groups
    float amax = 0.0f;                      // per column: the largest |o| (partials only)
    if (split) {
#pragma unroll
      for (int et = 0; et < kE; ++et)
        amax = vmax(amax, vmax(vmax(fabsf(acc[t][et][0]), fabsf(acc[t][et][1])),
                               vmax(fabsf(acc[t][et][2]), fabsf(acc[t][et][3]))));
      amax = rows_max(amax);
    }
    if (!col_ok[t]) continue;
    const int i = gc[t] / P.G;
    const int h = g * P.G + gc[t] % P.G;
    const int cblk = (sr.row_ctx(i) + kBlock - 1) / kBlock;
    const int np = bpp > 0 ? (cblk + bpp - 1) / bpp : 1;
    if (np <= 1 ? p != 0 : p >= np) continue;  // this column has no such partition
    const size_t orow = (size_t)(sr.first + i) * P.Hq + h;
    if (np > 1 || P.always_partial) {
      const size_t part = part_slot(P, sr.first + i, h, P.part_base + p);
      const PartScale ps = part_scale_f16(m[t] == kNoRef ? -INFINITY : m[t], l_col, amax);
#pragma unroll
      for (int et = 0; et < kE; ++et) {
        uint2 u = make_uint2(pack_f16x2(acc[t][et][0] * ps.mul, acc[t][et][1] * ps.mul),
                             pack_f16x2(acc[t][et][2] * ps.mul, acc[t][et][3] * ps.mul));
        if (bad) u = make_uint2(0x7e007e00u, 0x7e007e00u);  // NaN
        store_part8(P, sr.first + i, h, P.part_base + p, 2, (16 * et + 4 * rg) * 2, u);
      }
      if (rg == 0) {
        P.ws_ml[2 * part] = bad ? 0.0f : ps.m;
        P.ws_ml[2 * part + 1] = bad ? nan : ps.l;
      }
    } else {
      const float inv = l_col > 0.0f ? 1.0f / l_col : 0.0f;
#pragma unroll
      for (int et = 0; et < kE; ++et) {
        float res[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) res[e] = bad ? nan : acc[t][et][e] * inv;
        *reinterpret_cast<uint2*>(reinterpret_cast<char*>(P.out) +
                                  (orow * D + 16 * et + 4 * rg) * 2) =
            make_uint2(pack_bf16x2(res[0], res[1]), pack_bf16x2(res[2], res[3]));
      }
    }
  }
}

// Waves per workgroup and column tiles per wave. Up to 8 tiles per kv
// head: one tile per wave, on 4 waves up to 4 tiles, else on 8 (a wave
// without columns still brings its share of every block: the GQA batch with
// 3 new tokens per sequence, 2 tiles per kv head in 512-token partitions,
// took 4.63 TB/s with 4 waves, 4.55 with 2 and with 8). More: two tiles per
// wave on 4 waves, so that every K/V operand read from LDS serves 32 columns
// (with PA_CHUNK_TILES_PER_WAVE 1, one tile per wave on 8 waves).
hipError_t launch_chunk_mfma(const DecodeParams& p, hipStream_t stream) {
  constexpr int R = PA_CHUNK_RING;
  auto go = [&](auto d, auto nw, auto tpw) {
    constexpr int HD = decltype(d)::value;
    constexpr int NW = decltype(nw)::value;
    constexpr int TPW = decltype(tpw)::value;
    const dim3 grid(p.Hkv * ((p.n_tiles + NW * TPW - 1) / (NW * TPW)), p.pass_parts,
                    p.pass_items);
    hipLaunchKernelGGL((chunk_mfma_kernel<HD, NW, R, TPW, TilePolicy::kShared>), grid,
                       dim3(NW * kWave), 0, stream, p);
  };
  auto by_tiles = [&](auto d) {
    using I = std::integral_constant<int, 1>;
    if (PA_CHUNK_MAX_WAVES == 2)
      go(d, std::integral_constant<int, 2>{}, I{});
    else if (p.n_tiles <= 4 || PA_CHUNK_MAX_WAVES == 4)
      go(d, std::integral_constant<int, 4>{}, I{});
    else if (p.n_tiles <= 8 || PA_CHUNK_TILES_PER_WAVE == 1)
      go(d, std::integral_constant<int, 8>{}, I{});
    else
      go(d, std::integral_constant<int, 4>{}, std::integral_constant<int, 2>{});
  };
  if (p.D == 128)
    by_tiles(std::integral_constant<int, 128>{});
  else if (p.D == 64)
    by_tiles(std::integral_constant<int, 64>{});
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
