// Paged attention of many query columns per kv head on the matrix cores
// (bf16, head_dim 128): chunked prefill, or many drafted tokens per sequence.
//
// Method: as the decode kernels ("Why OS Virtual Memory Paging Saved LLM
// Inference" (a8q9.cn), section 2: K/V gathered block by block through the
// block table; online softmax over the blocks), with the causal limit of
// each new token ("vLLM & PagedAttention" (completesystemdesign.dev),
// section 01: a token attends to every earlier token and to itself).
//
// Columns: the n x G (query row, head of the group) pairs of a sequence and
// kv head, row-major, cut into tiles of 16, in the MFMA layouts of the decode
// MFMA kernel (S^T = K Q^T on v_mfma_f32_16x16x32_bf16, O^T = V^T P^T on
// v_mfma_f32_16x16x16_bf16; every accumulator a lane holds belongs to its own
// column). A workgroup of NW waves owns NW consecutive tiles, one per wave,
// and each wave keeps its tile's online-softmax state to the end.
//
// The waves stream the partition's K/V blocks together through an LDS ring
// of R slots. A slot holds one block's K tile (4 KiB) and V tile (4 KiB),
// written by the loads themselves (buffer_load ... lds) in eight 1 KiB
// pieces, one load instruction each, shared out over the waves: every byte
// crosses the vector memory path once per workgroup, not once per wave (the
// per-wave loads of a column tile kept that path busy most of the time). One
// barrier per block publishes the slot and frees the previous one.
//
// LDS image of a slot (rows of 256 bytes, 16 chunks of 16 bytes):
//   K row r at r * 256, its chunk c in position c ^ r: a 16-lane group loads
//     one whole row (chunk col ^ row), and the MFMA operand reads (chunk
//     4 kk + rg of row col) put the 16 lanes on 16 different positions of
//     the bank width, so neither side conflicts;
//   V row r at 4096 + r * 256, chunks in order: the operand reads (chunk col
//     of row 4 rg + j) take one row per 16-lane group.
// Lanes of a load past the block's rows inside the context write zeros.
#include "pa_device.h"
#include "pa_launch.h"

// LDS ring slots (3 or 4) and the register allocation's minimum waves per SIMD.
#ifndef PA_CHUNK_RING
#define PA_CHUNK_RING 4
#endif
#ifndef PA_CHUNK_MIN_WAVES
#define PA_CHUNK_MIN_WAVES 4
#endif
// Most waves per workgroup (2, 4 or 8).
#ifndef PA_CHUNK_MAX_WAVES
#define PA_CHUNK_MAX_WAVES 8
#endif

namespace pa {

namespace {

constexpr int kD = 128;
constexpr int kRowBytes = kD * 2;
constexpr int kTileBytes = kBlock * kRowBytes;      // one K or V tile
constexpr int kSlotBytes = 2 * kTileBytes;          // K, then V
constexpr int kPieceBytes = kWave * 16;             // one load instruction
constexpr int kPieces = kSlotBytes / kPieceBytes;   // per block

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

template <int NW, int R, TilePolicy kPolicy>
__global__ __launch_bounds__(NW * kWave)
__attribute__((amdgpu_waves_per_eu(NW >= 4 ? PA_CHUNK_MIN_WAVES : 3)))
void chunk_mfma_kernel(DecodeParams P) {
  static_assert(kPieces % NW == 0, "pieces must divide over the waves");
  static_assert(R >= 3 && R <= 4, "ring of 3 or 4 slots");
  constexpr int kPer = kPieces / NW;  // load instructions per wave per block
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
  const int groups = (P.n_tiles + NW - 1) / NW;
  const GridPos gp = grid_pos_grouped(groups);
  const int p = gp.y;
  const int s = gp.z;
  const int g = gp.x / groups;             // kv head
  const int tile0 = (gp.x % groups) * NW;  // the workgroup's first tile

  const int32_t* bt_row = P.block_tables + (size_t)s * P.MB;
  const int bpp = P.partition / kBlock;  // blocks per partition (0: no split)
  const int blk_begin = p * bpp;
  const int ids0 =
      first_chunk_ids(bt_row, blk_begin, 1, bpp > 0 ? min(P.MB, blk_begin + bpp) : P.MB, lane);
  const SeqRows sr = seq_rows(P, s);

  // Columns: global column gc of the n x G grid, row-major; gc >= n G is padding.
  const int ncols = min(sr.n, P.max_q) * P.G;
  const int wg_begin = 16 * tile0;
  if (wg_begin >= ncols) return;  // the whole workgroup is padding
  const int wg_end = min(ncols, wg_begin + 16 * NW);
  const int c_begin = 16 * (tile0 + w);
  const bool has_cols = c_begin < ncols;  // else the wave only loads (wave-uniform)
  const int c_end = has_cols ? min(ncols, c_begin + 16) : wg_end;
  const int gc = c_begin + col;
  const bool col_ok = has_cols && gc < c_end;
  const int gcl = col_ok ? gc : c_end - 1;  // padded lanes shadow a real column
  const int qi = gcl / P.G;
  const int qh = g * P.G + gcl % P.G;

  // The logit scale (log2 domain) is applied in the exponent, after the max
  // is taken over the raw products, which needs it non-negative: a negative
  // scale flips the sign bits of Q instead (exact), and a zero scale becomes
  // a tiny positive one (every logit still rounds to 0).
  const bool q_neg = P.qscale < 0.0f;
  const float qs = fmaxf(fabsf(P.qscale), 1e-30f);

  // B operand of S^T: Q[column col][32 kk + 8 rg ..], zero for padded columns.
  bf16x8_t qop[4];
  if (has_cols) {
    const char* qp =
        reinterpret_cast<const char*>(P.q) + ((size_t)(sr.first + qi) * P.Hq + qh) * kRowBytes;
    const uint32_t flip = q_neg ? 0x80008000u : 0u;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      uint4 u = ld16(qp + (32 * kk + 8 * rg) * 2);
      u = make_uint4(u.x ^ flip, u.y ^ flip, u.z ^ flip, u.w ^ flip);
      if (!col_ok) u = make_uint4(0, 0, 0, 0);
      qop[kk] = __builtin_bit_cast(bf16x8_t, u);
    }
  }

  // Contexts: each column's causal prefix; the wave's shortest and longest;
  // the workgroup's longest (what the ring streams).
  const int ctx_col = sr.row_ctx(qi);
  const int ctx_min = sr.row_ctx(c_begin / P.G);
  const int ctx_wg = sr.row_ctx((wg_end - 1) / P.G);
  const int nblk = (ctx_wg + kBlock - 1) / kBlock;
  const int blk_end = bpp > 0 ? min(nblk, blk_begin + bpp) : nblk;
  const int nparts_wg = bpp > 0 ? (nblk + bpp - 1) / bpp : (nblk > 0 ? 1 : 0);
  if (p >= max(nparts_wg, 1)) return;  // partition past the workgroup's contexts

  float m = -INFINITY, lsum = 0.0f;
  f32x4_t acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  bool bad = sr.bad;

  const char* kbase = reinterpret_cast<const char*>(P.k_cache);
  const char* vbase = reinterpret_cast<const char*>(P.v_cache);
  const size_t head_off = (size_t)g * kTileBytes;
  const size_t block_stride = (size_t)P.Hkv * kTileBytes;

  // This wave's pieces of every block: piece q = kPer w + i; pieces 0..3 are
  // K rows 4 q .. 4 q + 3, pieces 4..7 V rows 4 (q - 4) .. + 3.
  int piece_lds[kPer], piece_off[kPer];
  bool piece_v[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int q = kPer * w + i;
    piece_v[i] = q >= 4;
    const int r = 4 * (q & 3) + rg;
    piece_lds[i] = q * kPieceBytes;
    piece_off[i] = r * kRowBytes + (piece_v[i] ? col : ((col ^ r) & 15)) * 16;
  }

  // Load physical block b (logical block blk) into slot d. An id outside the
  // pool marks the columns bad and loads nothing; so does a block that does
  // not exist (an empty refill past the last block, kept so that every step
  // issues the same number of loads).
  auto issue = [&](int d, int b, int blk, bool exists) {
    const bool valid = b >= 0 && b < P.NB;
    bad |= exists && !valid;
    const size_t off = (size_t)(valid ? b : 0) * block_stride + head_off;
    const int rows = min(kBlock, ctx_wg - blk * kBlock);
    const int bytes = exists && valid ? rows * kRowBytes : 0;
    const rsrc_t rk = make_rsrc(kbase + off, bytes);
    const rsrc_t rv = make_rsrc(vbase + off, bytes);
    char* dst = slot(d);
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      ld16_lds<kPolicy>(piece_v[i] ? rv : rk, dst + piece_lds[i], piece_off[i]);
  };

  // S^T of the block in slot d: raw logits, lane (rg, col) holds tokens
  // 4 rg + 0..3 of column col.
  auto qk = [&](int d) -> f32x4_t {
    const char* src = slot(d);
    f32x4_t st = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const uint4 ka = *reinterpret_cast<const uint4*>(
          src + col * kRowBytes + (((4 * kk + rg) ^ col) & 15) * 16);
      st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka), qop[kk], st,
                                                  0, 0, 0);
    }
    return st;
  };

  // Online softmax over the block's logits st, then O^T += V^T P^T with the
  // block's V from slot d.
  auto softmax_pv = [&](int d, const f32x4_t st, int blk) {
    const char* src = slot(d);
    uint4 vb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      vb[j] = *reinterpret_cast<const uint4*>(src + kTileBytes + (4 * rg + j) * kRowBytes + col * 16);
    // Raw logits; those past a column's causal limit are removed (only a
    // block that reaches some column's limit needs the test: wave-uniform).
    float x[4] = {st[0], st[1], st[2], st[3]};
    if (blk * kBlock + kBlock > ctx_min) {
      const int tok0 = blk * kBlock + 4 * rg;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (tok0 + i >= ctx_col) x[i] = -INFINITY;
    }
    const float mx_raw = rows_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
    const float mx = mx_raw * qs;  // -inf stays -inf (qs > 0)
    // The reference m (what the probabilities are taken relative to) moves
    // only when a column's max passes it by more than kLazy: the
    // probabilities then stay below 2^kLazy, the result is the same up to
    // rounding, and the accumulators are rescaled a few times per column
    // instead of whenever its max creeps up.
    constexpr float kLazy = 8.0f;
    const float m_new = fmaxf(m, mx);
    const bool up = m_new > m + kLazy;  // from -inf: any finite max
    const float ref = up ? m_new : m;
    const float ref_use = (ref == -INFINITY) ? 0.0f : ref;
    const float alpha = exp2_fast(m - ref_use);  // exactly 1 where the reference stays
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = exp2_fast(__builtin_fmaf(x[i], qs, -ref_use));
    lsum = lsum * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
    m = ref;
    if (__builtin_amdgcn_ballot_w64(up) != 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= alpha;
    }
    const s16x4_t pop = __builtin_bit_cast(
        s16x4_t, make_uint2(pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3])));
#pragma unroll
    for (int k = 0; k < 4; ++k) {  // 32-bit word k of each V chunk: dims 2k, 2k+1
      const uint32_t w0 = word(vb[0], k), w1 = word(vb[1], k);
      const uint32_t w2 = word(vb[2], k), w3 = word(vb[3], k);
      const s16x4_t a_lo =
          __builtin_bit_cast(s16x4_t, make_uint2(pack_lo16(w0, w1), pack_lo16(w2, w3)));
      const s16x4_t a_hi =
          __builtin_bit_cast(s16x4_t, make_uint2(pack_hi16(w0, w1), pack_hi16(w2, w3)));
      acc[2 * k] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_lo, pop, acc[2 * k], 0, 0, 0);
      acc[2 * k + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_hi, pop, acc[2 * k + 1], 0, 0, 0);
    }
  };

  // The ring: block k sits in slot k % R. Step k of a wave takes S^T of
  // block k + 1 (independent of the softmax of block k, so the two overlap)
  // and the softmax and PV product of block k. Before it, each wave waits
  // for its own pieces of block k + 1 (the block issued after it may stay in
  // flight), then a barrier makes every wave's pieces visible and shows that
  // every wave is done with block k - 1 (its K was read at step k - 2, its V
  // at step k - 1), whose slot takes block k + R - 1. Block ids are read 64
  // at a time (lane j holds the chunk's j-th id, broadcast with readlane);
  // the ring drains at each chunk's end.
  const int nk = max(0, blk_end - blk_begin);
  for (int c0 = 0; c0 < nk; c0 += kWave) {
    const int cn = min(kWave, nk - c0);
    if (c0 > 0) ring_barrier();  // every wave is done with the previous chunk's slots
    const int ids = c0 == 0 ? ids0 : (lane < cn ? bt_row[blk_begin + c0 + lane] : -1);
#pragma unroll
    for (int d = 0; d < R - 1; ++d)
      issue(d, __builtin_amdgcn_readlane(ids, d), blk_begin + c0 + d, d < cn);
    wait_vmcnt<(R - 2) * kPer>();
    ring_barrier();
    f32x4_t s_next = {0.0f, 0.0f, 0.0f, 0.0f};
    if (has_cols) s_next = qk(0);
    // Steps past the chunk's last block still wait, meet and refill (with
    // empty loads): a refill under a branch costs the compiler its record of
    // which slot each load writes, and then it waits for every slot.
    for (int k0 = 0; k0 < cn; k0 += R) {
#pragma unroll
      for (int d = 0; d < R; ++d) {
        const int k = k0 + d;
        wait_vmcnt<(R - 3) * kPer>();
        ring_barrier();
        const int kl = k + R - 1;
        issue((d + R - 1) % R, __builtin_amdgcn_readlane(ids, min(kl, kWave - 1)),
              blk_begin + c0 + kl, kl < cn);
        const f32x4_t s_cur = s_next;
        if (has_cols && k + 1 < cn) s_next = qk((d + 1) % R);
        if (has_cols && k < cn) softmax_pv(d, s_cur, blk_begin + c0 + k);
      }
    }
  }

  if (!has_cols) return;
  lsum = rows_sum(lsum);  // per column: sum over the 4 row groups

  // The wave holds its columns' whole state for this partition: lane
  // (rg, col) writes dims 8 (4 rg + i) + 0..7 (i = 0..3) of column col, from
  // acc[0..7][i].
  if (!col_ok) return;
  const int i = gc / P.G;
  const int h = g * P.G + gc % P.G;
  const int cblk = (sr.row_ctx(i) + kBlock - 1) / kBlock;
  const int np = bpp > 0 ? (cblk + bpp - 1) / bpp : 1;
  if (np <= 1 ? p != 0 : p >= np) return;  // this column has no such partition
  const size_t orow = (size_t)(sr.first + i) * P.Hq + h;
  const float nan = __builtin_nanf("");
  if (np > 1) {
    const size_t part = orow * P.n_parts + p;
    float* dst = P.ws_o + part * kD;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      float* d8 = dst + 8 * (4 * rg + ii);
      *reinterpret_cast<float4*>(d8) =
          bad ? make_float4(nan, nan, nan, nan)
              : make_float4(acc[0][ii], acc[1][ii], acc[2][ii], acc[3][ii]);
      *reinterpret_cast<float4*>(d8 + 4) =
          bad ? make_float4(nan, nan, nan, nan)
              : make_float4(acc[4][ii], acc[5][ii], acc[6][ii], acc[7][ii]);
    }
    if (rg == 0) {
      P.ws_ml[2 * part] = bad ? 0.0f : m;
      P.ws_ml[2 * part + 1] = bad ? nan : lsum;
    }
  } else {
    const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      float res[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) res[e] = bad ? nan : acc[e][ii] * inv;
      uint4 u;
      u.x = pack_bf16x2(res[0], res[1]);
      u.y = pack_bf16x2(res[2], res[3]);
      u.z = pack_bf16x2(res[4], res[5]);
      u.w = pack_bf16x2(res[6], res[7]);
      st16(reinterpret_cast<char*>(P.out) + (orow * kD + 8 * (4 * rg + ii)) * 2, u);
    }
  }
}

// Waves per workgroup: as many as the kv head has tiles, up to 8 (a wave
// without columns still brings its share of every block).
hipError_t launch_chunk_mfma(const DecodeParams& p, hipStream_t stream) {
  constexpr int R = PA_CHUNK_RING;
  auto go = [&](auto nw) {
    constexpr int NW = decltype(nw)::value;
    const dim3 grid(p.Hkv * ((p.n_tiles + NW - 1) / NW), p.n_parts, p.B);
    hipLaunchKernelGGL((chunk_mfma_kernel<NW, R, TilePolicy::kShared>), grid, dim3(NW * kWave), 0,
                       stream, p);
  };
  if (p.n_tiles <= 2 || PA_CHUNK_MAX_WAVES == 2)
    go(std::integral_constant<int, 2>{});
  else if (p.n_tiles <= 4 || PA_CHUNK_MAX_WAVES == 4)
    go(std::integral_constant<int, 4>{});
  else
    go(std::integral_constant<int, 8>{});
  return hipGetLastError();
}

}  // namespace pa
