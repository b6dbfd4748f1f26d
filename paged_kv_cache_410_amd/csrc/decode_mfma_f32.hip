// Paged attention on the matrix cores in fp32 (v_mfma_f32_16x16x4_f32):
// grouped query heads, and several new query tokens per sequence, with fp32
// queries, K/V and outputs.
//
// Method: as the other decode kernels ("Why OS Virtual Memory Paging Saved
// LLM Inference" (a8q9.cn), section 2: K/V gathered block by block through
// the block table; online softmax over blocks), with the causal limit of
// each new token ("vLLM & PagedAttention" (completesystemdesign.dev),
// section 01). One workgroup per (kv head, 16-column tile, partition,
// sequence) serves a tile of the kv head's (query row, head) columns, so a
// kv head's K/V crosses the memory path once per 16 columns instead of once
// per column. The products are fp32 throughout (no operand is rounded).
// It also runs the two passes of shared-prefix decode in fp32 (a8q9.cn,
// section 3: sharers point at the same blocks): the group pass (work item =
// a group, columns = its members' query heads, the shared blocks read once
// through the first member's table) and the tail pass (each sequence's
// blocks past its shared ones, merged with the group pass's partials).
//
// Layouts (wave64; lane = 16 * rg + col, rg = lane / 16, col = lane % 16).
// v_mfma_f32_16x16x4_f32: A (16 x 4) lane holds A[col][rg], B (4 x 16) lane
// holds B[rg][col], result lane holds D[4 rg + i][col], i = 0..3.
//   Loads: K and V tiles alike, a 16-lane group reading 256 contiguous bytes
//     of one row: piece j (row 4 rg + j / H, bytes 256 (j % H) + 16 col of
//     the row), H = row bytes / 256. So lane (rg, col) holds
//     X[4 rg + jr][64 h + 4 col + c], c = 0..3, for jr < 4, h < H.
//   S^T = K Q^T, D / 4 steps; step kk contracts dims (D / 4) r + kk, r = 0..3
//     (row group r supplies the dims of its quarter):
//     A: lane holds K[t = col][(D / 4) rg + kk], read from a per-wave LDS
//        stage of the K tile (rows kRowBytes + 16 apart: the row writes and
//        the strided operand reads are free of bank conflicts);
//     B: lane holds Q[q = col][(D / 4) rg + kk] (registers, loaded once);
//     result: lane holds S^T[t = 4 rg + i][q = col].
//   O^T = V^T P^T, 4 steps over tokens; step kk contracts tokens 4 r + kk:
//     A of output tile et = 4 h + c: lane holds V[4 rg + kk][64 h + 4 col + c],
//       a loaded register as it stands (row m = col of tile et stands for
//       dim 64 h + 4 m + c);
//     B: lane holds P[4 rg + kk][q = col], its own probability kk;
//     result tile et: lane holds O[q = col][64 h + 16 rg + 4 i + c].
//   Every accumulator a lane holds belongs to its own column, so the
//   online-softmax rescale is a per-lane multiply.
#include "pa_device.h"
#include "pa_launch.h"

// Waves per workgroup (split contexts, and unsplit ones) and K/V tiles in
// flight per wave.
#ifndef PA_MFMA32_WAVES
#define PA_MFMA32_WAVES 4
#endif
#ifndef PA_MFMA32_WAVES_UNSPLIT
#define PA_MFMA32_WAVES_UNSPLIT 8
#endif
#ifndef PA_MFMA32_DEPTH
#define PA_MFMA32_DEPTH 2
#endif
// Minimum waves per SIMD the register allocation must allow (head_dim 128:
// two tiles of fp32 K and V in flight take 128 registers).
#ifndef PA_MFMA32_MIN_WAVES
#define PA_MFMA32_MIN_WAVES 2
#endif

namespace pa {

template <int D, int NW, int DEPTH, TilePolicy kPolicy>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(PA_MFMA32_MIN_WAVES)))
void decode_mfma_f32_kernel(DecodeParams P) {
  static_assert(D == 128 || D == 64, "head_dim");
  constexpr int kRowBytes = D * 4;
  constexpr int kH = kRowBytes / 256;  // 256-byte pieces per row
  constexpr int kPieces = 4 * kH;      // 16-byte loads per lane per tile
  constexpr int kQ = D / 16;           // 16-byte operand reads of a lane's quarter of the dims
  constexpr int kTiles = D / 16;       // 16-dim output tiles of O^T
  constexpr int kPad = 4;              // LDS row padding (floats) of the merge rows
  constexpr int kStageRow = kRowBytes + 16;
  static_assert(kBlock * kStageRow <= 16 * (D + kPad) * 4, "K stage must fit a merge region");

  const int lane = threadIdx.x & (kWave - 1);
  const int w = wave_id();
  const int col = lane & 15;
  const int rg = lane >> 4;

  // The tiles of one kv head read the same K/V: with several, they are kept
  // on one XCD (one L2).
  const GridPos gp = P.n_tiles > 1 ? grid_pos_grouped(P.n_tiles) : grid_pos();
  const int p = gp.y;
  const int g = gp.x / P.n_tiles;     // kv head
  const int tile = gp.x % P.n_tiles;  // 16-column tile of this kv head's (row, head) pairs
  const int s = gp.z;

  const ItemStart is = item_start(P, s);
  const int32_t* bt_row = P.block_tables + (size_t)is.trow * P.MB;
  const int bpp = P.partition / kBlock;  // blocks per partition (0: no split)
  const int blk_begin = p * bpp;
  constexpr int kStride = NW;  // wave w takes blocks first, first + NW, ...
  const int first = blk_begin + w;

  // Start-up loads, issued before anything waits on them: the wave's first 64
  // block ids, the sequence's rows and context length, the queries.
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

  // B operand of S^T: Q[column col][(D / 4) rg + kk], zero for padded columns.
  float qop[D / 4];
  {
    const char* qp = reinterpret_cast<const char*>(P.q) + ((size_t)qrow * P.Hq + qh) * kRowBytes +
                     D * rg;  // (D / 4) rg floats
#pragma unroll
    for (int i = 0; i < kQ; ++i) {
      uint4 u = ld16(qp + 16 * i);
      if (!col_ok) u = make_uint4(0, 0, 0, 0);
      qop[4 * i + 0] = __uint_as_float(u.x);
      qop[4 * i + 1] = __uint_as_float(u.y);
      qop[4 * i + 2] = __uint_as_float(u.z);
      qop[4 * i + 3] = __uint_as_float(u.w);
    }
  }
  // LDS, one region per wave: while the wave streams its blocks, the first
  // 16 kStageRow bytes hold the K tile it is transposing; at the end the
  // region holds the wave's merge rows (16 columns x D floats, padded). The
  // wave overwrites its stage only after its last read of it, and a wave's
  // LDS accesses complete in order, so no barrier guards either use.
  __shared__ float sm_o[NW][16][D + kPad];
  char* const stage = reinterpret_cast<char*>(&sm_o[w][0][0]);

  // Context of each column (its row's causal prefix) and of the whole tile.
  const int ctx_col = sr.row_ctx(qi);             // this lane's column
  const int ctx_min = sr.row_ctx(c_begin / P.G);  // first column's row
  const int ctx = sr.row_ctx((c_end - 1) / P.G);  // last column's row: the longest
  const int nblk = (ctx + kBlock - 1) / kBlock;
  const int blk_end = bpp > 0 ? min(nblk, blk_begin + bpp) : nblk;
  const int span = nblk - is.start_blk;  // blocks this pass reads (tail pass: past the shared ones)
  const int nparts_s = bpp > 0 ? (span + bpp - 1) / bpp : (span > 0 ? 1 : 0);
  if (p >= max(nparts_s, 1)) return;  // partition past the tile's longest context

  float m = -INFINITY, lsum = 0.0f;
  f32x4_t acc[kTiles];
#pragma unroll
  for (int e = 0; e < kTiles; ++e) acc[e] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  bool bad = sr.bad || is.bad || is.start_blk * kBlock > ctx;  // the whole tile (wave-uniform)

  const char* kbase = reinterpret_cast<const char*>(P.k_cache);
  const char* vbase = reinterpret_cast<const char*>(P.v_cache);
  const size_t head_off = (size_t)g * kBlock * kRowBytes;
  const size_t block_stride = (size_t)P.Hkv * kBlock * kRowBytes;
  // byte offset of piece j in a tile, and in the LDS stage
  auto piece_off = [&](int j) { return (4 * rg + j / kH) * kRowBytes + 256 * (j % kH) + 16 * col; };
  auto stage_off = [&](int j) { return (4 * rg + j / kH) * kStageRow + 256 * (j % kH) + 16 * col; };

  // Issue the loads of physical block b's tile (logical block blk) into
  // (kb, vb). An id outside the pool marks the tile bad and loads nothing;
  // so does a block that does not exist (an empty ring refill). Only the
  // block's rows inside the context are fetched; the rest read as zeros.
  auto load = [&](uint4 (&kb)[kPieces], uint4 (&vb)[kPieces], int b, int blk, bool exists) {
    const bool valid = b >= 0 && b < P.NB;
    bad |= exists && !valid;
    const size_t off = (size_t)(valid ? b : 0) * block_stride + head_off;
    const int rows = min(kBlock, ctx - blk * kBlock);
    const int bytes = exists && valid ? rows * kRowBytes : 0;
    const rsrc_t rk = make_rsrc(kbase + off, bytes);
    const rsrc_t rv = make_rsrc(vbase + off, bytes);
#pragma unroll
    for (int j = 0; j < kPieces; ++j) kb[j] = ld16<kPolicy>(rk, piece_off(j));
#pragma unroll
    for (int j = 0; j < kPieces; ++j) vb[j] = ld16<kPolicy>(rv, piece_off(j));
  };

  // One tile: S^T, the online-softmax update and O^T += V^T P^T. When
  // `partial`, this lane's tokens 4 rg + i at or past `lim` (tile-local) are
  // masked.
  auto consume = [&](const uint4 (&kb)[kPieces], const uint4 (&vb)[kPieces], bool partial,
                     int lim) {
#pragma unroll
    for (int j = 0; j < kPieces; ++j) *reinterpret_cast<uint4*>(stage + stage_off(j)) = kb[j];
    // two accumulators, so that consecutive products do not wait on each other
    f32x4_t s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < kQ; ++i) {
      const uint4 ka = *reinterpret_cast<const uint4*>(stage + col * kStageRow + D * rg + 16 * i);
      s0 = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(ka.x), qop[4 * i + 0], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(ka.y), qop[4 * i + 1], s1, 0, 0, 0);
      s0 = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(ka.z), qop[4 * i + 2], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(ka.w), qop[4 * i + 3], s1, 0, 0, 0);
    }
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = (s0[i] + s1[i]) * P.qscale;
      if (partial && 4 * rg + i >= lim) x[i] = -INFINITY;
    }
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
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int h = 0; h < kH; ++h) {
        const uint4 v = vb[kH * kk + h];
        acc[4 * h + 0] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.x), pr[kk],
                                                              acc[4 * h + 0], 0, 0, 0);
        acc[4 * h + 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.y), pr[kk],
                                                              acc[4 * h + 1], 0, 0, 0);
        acc[4 * h + 2] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.z), pr[kk],
                                                              acc[4 * h + 2], 0, 0, 0);
        acc[4 * h + 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.w), pr[kk],
                                                              acc[4 * h + 3], 0, 0, 0);
      }
    }
  };

  // This wave's blocks: first + k * kStride, k < nk, through a ring of DEPTH tiles.
  {
    const int nk = first < blk_end ? (blk_end - first + kStride - 1) / kStride : 0;
    // tail pass: skip this wave's blocks inside the shared part
    const int k0 = is.start_blk > first ? (is.start_blk - first + kStride - 1) / kStride : 0;
    uint4 kb[DEPTH][kPieces], vb[DEPTH][kPieces];
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
  }

  lsum = rows_sum(lsum);  // per column: sum over the 4 row groups

  // Waves -> LDS -> one merged state per (head, dim).
  __shared__ float sm_m[NW][16], sm_l[NW][16];
  __shared__ int sm_bad[NW];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int h = 0; h < kH; ++h)  // tile 4 h + c holds dim 64 h + 16 rg + 4 i + c
      *reinterpret_cast<float4*>(&sm_o[w][col][64 * h + 16 * rg + 4 * i]) =
          make_float4(acc[4 * h][i], acc[4 * h + 1][i], acc[4 * h + 2][i], acc[4 * h + 3][i]);
  }
  if (rg == 0) {
    sm_m[w][col] = m;
    sm_l[w][col] = lsum;
  }
  if (lane == 0) sm_bad[w] = bad ? 1 : 0;
  __syncthreads();

  bool any_bad = false;
#pragma unroll
  for (int v = 0; v < NW; ++v) any_bad |= sm_bad[v] != 0;
  // thread -> (column qq, 8-dim chunk ch)
  constexpr int kChunks = D / 8;
  const float nan = __builtin_nanf("");
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
    // One of several partitions, or the group pass of a shared prefix: the
    // unnormalised fp32 row and its (m, l). Else the final row (the tail pass
    // first folds in the group pass's partials of the row).
    const bool to_partial = np > 1 || P.always_partial;
    if (!to_partial && P.tail_pass)
      merge_shared_partials<float, 8>(P, is.bad ? 0 : is.start_blk * kBlock, row, h, 8 * ch, D, M,
                                      L, ov);
    const float mul = to_partial ? 1.0f : (L > 0.0f ? 1.0f / L : 0.0f);  // empty context: zeros
    float res[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) res[e] = any_bad ? nan : ov[e] * mul;
    const uint4 lo = make_uint4(__float_as_uint(res[0]), __float_as_uint(res[1]),
                                __float_as_uint(res[2]), __float_as_uint(res[3]));
    const uint4 hi = make_uint4(__float_as_uint(res[4]), __float_as_uint(res[5]),
                                __float_as_uint(res[6]), __float_as_uint(res[7]));
    if (to_partial) {
      const size_t part = part_slot(P, row, h, P.part_base + p);
      store_part16(P, row, h, P.part_base + p, 4, 32 * ch, lo);
      store_part16(P, row, h, P.part_base + p, 4, 32 * ch + 16, hi);
      if (ch == 0) {
        P.ws_ml[2 * part] = any_bad ? 0.0f : M;
        P.ws_ml[2 * part + 1] = any_bad ? nan : L;
      }
    } else {
      char* dst = reinterpret_cast<char*>(P.out) + ((row * P.Hq + h) * D + 8 * ch) * 4;
      st16(dst, lo);
      st16(dst + 16, hi);
    }
  }
}

// fp32 I/O with several columns per kv head (grouped heads, or several query
// rows): one workgroup per 16-column tile; decode, multi-query, and the group
// and tail passes of shared-prefix decode (not its one-pass form, which is
// bf16 only).
hipError_t launch_decode_mfma_f32(const DecodeParams& p, hipStream_t stream) {
  if (p.fold_tails) return hipErrorInvalidValue;
  constexpr int DEPTH = PA_MFMA32_DEPTH;
  auto go = [&](auto d, auto nw) {
    constexpr int HD = decltype(d)::value;
    constexpr int NW = decltype(nw)::value;
    const dim3 grid(p.Hkv * p.n_tiles, p.pass_parts, p.pass_items), block(NW * kWave);
    if (p.shared_kv)
      hipLaunchKernelGGL((decode_mfma_f32_kernel<HD, NW, DEPTH, TilePolicy::kShared>), grid, block,
                         0, stream, p);
    else
      hipLaunchKernelGGL((decode_mfma_f32_kernel<HD, NW, DEPTH, TilePolicy::kStream>), grid, block,
                         0, stream, p);
  };
  auto by_waves = [&](auto d) {
    // A whole context per workgroup: more waves, each with a longer share of
    // its blocks. Split contexts (a partition's few blocks) and the tail
    // pass (a sequence's own blocks): fewer.
    if (p.pass_parts == 1 && !p.tail_pass)
      go(d, std::integral_constant<int, PA_MFMA32_WAVES_UNSPLIT>{});
    else
      go(d, std::integral_constant<int, PA_MFMA32_WAVES>{});
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
