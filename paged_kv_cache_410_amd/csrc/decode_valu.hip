// Paged decode attention, vector-ALU path (one query row and head per workgroup).
//
// Method: "Why OS Virtual Memory Paging Saved LLM Inference" (a8q9.cn),
// section 2: the attention kernel reads each logical block's physical block
// id from the block table and fetches that block's K/V wherever it sits.
// "Can OS paging techniques reduce LLM serving memory waste?"
// (inquiringlines.com), mechanism paragraph: attention proceeds block by
// block. The softmax is accumulated online over blocks (running max, running
// sum, rescaled output), so every K/V byte is read exactly once.
//
// Work decomposition (gfx950, wave64):
//   grid   = (query head h + Hq * query row i, partition p, sequence s): the
//            heads of one sequence are dispatched together, so the tiles of
//            one physical block (all heads, contiguous in the pool) are read
//            close in time. A decode step has one query row per sequence;
//            with several new tokens per sequence (query_start) each row is
//            its own workgroup and attends over its causal prefix. (The
//            library sends every kv head with more than one such column,
//            grouped heads or several rows, to the matrix-core kernels: here
//            it serves one query head per kv head and one row per sequence.)
//   block  = NW waves; wave w takes blocks p0 + w, p0 + w + NW, ...
//   A (block, kv head) tile is 16 rows of D elements, contiguous in memory.
//   One 16-byte load per lane: LPT = D*e/16 lanes cover one token row, so a
//   wave-wide load covers TPI = 64/LPT rows, fully coalesced; NLD = 16/TPI
//   loads cover the tile. Lane (r = lane / LPT, c = lane % LPT) holds chunk c
//   of row j*TPI + r for load j.
//   QK: per-lane partial dot (v_dot2_f32_bf16 or fp32 FMA), then a DPP
//   all-reduce over the LPT lanes of the row. Every lane of a row then holds
//   the row's logit, so the V rows loaded in the same lane layout are
//   accumulated without any further data movement.
//   Each row group of lanes keeps its own online-softmax state; row groups
//   merge at the end through lane swaps, waves through LDS.
//   K/V tiles are prefetched DEPTH - 1 blocks ahead through a ring of
//   register buffers; the wave's block ids come from the table 64 at a time
//   (block_pipeline), so no table read sits between two tile prefetches.
#include "pa_device.h"
#include "pa_launch.h"

// Waves per workgroup and K/V tiles in flight per wave.
#ifndef PA_VALU_WAVES
#define PA_VALU_WAVES 8
#endif
// Waves per workgroup when an unsplit grid has few work items (at most 8 per
// compute unit): longer contexts per item, each shared by more waves.
#ifndef PA_VALU_WAVES_FEW
#define PA_VALU_WAVES_FEW 16
#endif
// Waves per workgroup of the shared-prefix tail pass (each sequence's own
// tokens past the shared ones: short runs of blocks).
#ifndef PA_VALU_TAIL_WAVES
#define PA_VALU_TAIL_WAVES 4
#endif
#ifndef PA_VALU_DEPTH
#define PA_VALU_DEPTH 3
#endif
// Ring depth of the tail pass: its runs of blocks are short (copy-on-write
// batch: 57.9 us at depth 2 against 60.5 at 3).
#ifndef PA_VALU_TAIL_DEPTH
#define PA_VALU_TAIL_DEPTH 2
#endif

namespace pa {

namespace {

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kPerChunk = 4;
  __device__ static void unpack(const uint4& u, float* f) {
    f[0] = __uint_as_float(u.x);
    f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z);
    f[3] = __uint_as_float(u.w);
  }
};
template <>
struct Elem<uint16_t> {  // bf16 bits
  static constexpr int kPerChunk = 8;
  __device__ static void unpack(const uint4& u, float* f) {
    f[0] = bf16lo(u.x);
    f[1] = bf16hi(u.x);
    f[2] = bf16lo(u.y);
    f[3] = bf16hi(u.y);
    f[4] = bf16lo(u.z);
    f[5] = bf16hi(u.z);
    f[6] = bf16lo(u.w);
    f[7] = bf16hi(u.w);
  }
};

// (own, partner) for lanes OFF apart inside the wave, OFF in {8, 16, 32}.
template <int OFF>
__device__ __forceinline__ LanePair lane_pair(float x) {
  if constexpr (OFF == 8) {
    // row_ror:8 inside a row of 16 lanes: lane i sees lane i ^ 8
    return {x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false))};
  } else if constexpr (OFF == 16) {
    return pair16(x);
  } else {
    static_assert(OFF == 32, "lane offset");
    return pair32(x);
  }
}

// Merge the online-softmax states of lanes OFF apart (different token rows,
// same D chunk) so both hold the state over the union of their tokens.
template <int OFF, int EPL>
__device__ __forceinline__ void merge_rows(float& m, float& l, float (&o)[EPL]) {
  const LanePair pm = lane_pair<OFF>(m);
  const LanePair pl = lane_pair<OFF>(l);
  const SoftmaxScales sc = merge_scales(pm.a, pm.b);
  l = pl.a * sc.a + pl.b * sc.b;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const LanePair po = lane_pair<OFF>(o[e]);
    o[e] = po.a * sc.a + po.b * sc.b;
  }
  m = sc.m;
}

template <int LPT, int EPL>
__device__ __forceinline__ void merge_all_rows(float& m, float& l, float (&o)[EPL]) {
  if constexpr (LPT <= 8) merge_rows<8, EPL>(m, l, o);
  if constexpr (LPT <= 16) merge_rows<16, EPL>(m, l, o);
  if constexpr (LPT <= 32) merge_rows<32, EPL>(m, l, o);
}

}  // namespace

// kTail: the shared-prefix tail pass (P.tail_pass), the only instantiations
// that merge group-pass partials.
template <typename T, int D, int NW, int DEPTH, TilePolicy kPolicy, bool kTail = false>
__global__ __launch_bounds__(NW * kWave) void decode_valu_kernel(DecodeParams P) {
  constexpr int EPL = Elem<T>::kPerChunk;  // elements per 16-byte lane chunk
  constexpr int LPT = D / EPL;             // lanes per token row
  constexpr int TPI = kWave / LPT;         // token rows per wave-wide load
  constexpr int NLD = kBlock / TPI;        // wave loads per (block, head) tile
  constexpr int kRowBytes = D * (int)sizeof(T);
  static_assert(LPT >= 8 && LPT <= 32 && NLD >= 1, "unsupported tile shape");

  const int lane = threadIdx.x & (kWave - 1);
  const int w = wave_id();
  const int r = lane / LPT;
  const int c = lane % LPT;

  const GridPos gp = grid_pos();
  const int h = gp.x % P.Hq;
  const int i = gp.x / P.Hq;  // query row of the sequence (0 for decode)
  const int p = gp.y;
  const int s = gp.z;
  const int g = h / P.G;

  const ItemStart is = item_start(P, s);
  const int32_t* bt_row = P.block_tables + (size_t)is.trow * P.MB;
  const int bpp = P.partition / kBlock;  // blocks per partition (0: no split)
  // (the tail pass is unsplit and walks the same blocks as an unsplit call,
  // from its first block past the shared ones: see k0 below)
  const int blk_begin = p * bpp;
  const int first = blk_begin + w;       // this wave's blocks: first, first + NW, ...

  // Start-up loads, issued before anything waits on them: the wave's first 64
  // block ids (bounded by the partition's table range, as the context length
  // is not known yet), the sequence's rows and context length, the query.
  const int ids0 = first_chunk_ids(bt_row, first, NW, bpp > 0 ? min(P.MB, blk_begin + bpp) : P.MB,
                                   lane);
  const SeqRows sr = seq_rows(P, s);
  if (i >= min(sr.n, P.max_q)) return;  // no such row
  const int row = sr.first + i;
  const size_t row_qo = ((size_t)row * P.Hq + h) * D;
  const uint4 qraw = ld16(reinterpret_cast<const char*>(P.q) + row_qo * sizeof(T) + c * 16);

  const int ctx = sr.row_ctx(i);         // tokens this row attends over
  const bool bad_ctx = sr.bad || is.bad || is.start_blk * kBlock > ctx;
  const int nblk = (ctx + kBlock - 1) / kBlock;
  const int blk_end = bpp > 0 ? min(nblk, blk_begin + bpp) : nblk;
  const int span = nblk - is.start_blk;  // blocks this pass reads (tail pass: past the shared ones)
  const int nparts_s = bpp > 0 ? (span + bpp - 1) / bpp : (span > 0 ? 1 : 0);
  if (p >= max(nparts_s, 1)) return;  // partition past this row's context

  float qf[EPL];
  Elem<T>::unpack(qraw, qf);

  float m = -INFINITY, l = 0.0f;
  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.0f;
  bool bad = bad_ctx;

  const char* kbase = reinterpret_cast<const char*>(P.k_cache);
  const char* vbase = reinterpret_cast<const char*>(P.v_cache);
  const int lane_off = r * kRowBytes + c * 16;
  const size_t head_off = (size_t)g * kBlock * kRowBytes;
  const size_t block_stride = (size_t)P.Hkv * kBlock * kRowBytes;

  // Issue the loads of physical block b's tile (logical block blk) into
  // (kb, vb). An id outside the pool marks the row bad and loads nothing;
  // so does a block that does not exist (an empty ring refill).
  auto load = [&](uint4 (&kb)[NLD], uint4 (&vb)[NLD], int b, int blk, bool exists) {
    const bool valid = b >= 0 && b < P.NB;
    bad |= exists && !valid;
    const size_t off = (size_t)(valid ? b : 0) * block_stride + head_off;
    // only the block's rows inside the context are fetched (the rest read as 0)
    const int rows = min(kBlock, ctx - blk * kBlock);
    const int bytes = exists && valid ? rows * kRowBytes : 0;
    const rsrc_t rk = make_rsrc(kbase + off, bytes);
    const rsrc_t rv = make_rsrc(vbase + off, bytes);
#pragma unroll
    for (int j = 0; j < NLD; ++j) kb[j] = ld16<kPolicy>(rk, lane_off + j * TPI * kRowBytes);
#pragma unroll
    for (int j = 0; j < NLD; ++j) vb[j] = ld16<kPolicy>(rv, lane_off + j * TPI * kRowBytes);
  };

  // Consume one tile: logits, online-softmax update, V accumulation.
  auto consume = [&](const uint4 (&kb)[NLD], const uint4 (&vb)[NLD], int blk) {
    float x[NLD];
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      float acc = 0.0f;
      if constexpr (sizeof(T) == 2) {
        acc = dot2_bf16(qraw.x, kb[j].x, acc);
        acc = dot2_bf16(qraw.y, kb[j].y, acc);
        acc = dot2_bf16(qraw.z, kb[j].z, acc);
        acc = dot2_bf16(qraw.w, kb[j].w, acc);
      } else {
        float kf[EPL];
        Elem<T>::unpack(kb[j], kf);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc = fmaf(qf[e], kf[e], acc);
      }
      x[j] = group_sum<LPT>(acc) * P.qscale;
    }
    const int tok0 = blk * kBlock;
    const bool partial = tok0 + kBlock > ctx;  // same for the whole wave
    if (partial) {
#pragma unroll
      for (int j = 0; j < NLD; ++j)
        if (tok0 + j * TPI + r >= ctx) x[j] = -INFINITY;
    }
    float mx = x[0];
#pragma unroll
    for (int j = 1; j < NLD; ++j) mx = fmaxf(mx, x[j]);
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = exp2_fast(m - m_use);
    float pj[NLD];
    float psum = 0.0f;
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      pj[j] = exp2_fast(x[j] - m_use);
      psum += pj[j];
    }
    l = l * alpha + psum;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] *= alpha;
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      float vf[EPL];
      Elem<T>::unpack(vb[j], vf);
      // rows past the context may hold anything (even NaN): select, not multiply
      const bool valid = !partial || (tok0 + j * TPI + r < ctx);
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = fmaf(pj[j], valid ? vf[e] : 0.0f, o[e]);
    }
    m = m_new;
  };

  // This wave's blocks: first + k * NW, k < nk, through a ring of DEPTH tiles.
  {
    const int nk = first < blk_end ? (blk_end - first + NW - 1) / NW : 0;
    // tail pass: skip this wave's blocks inside the shared part
    const int k0 = is.start_blk > first ? (is.start_blk - first + NW - 1) / NW : 0;
    uint4 kb[DEPTH][NLD], vb[DEPTH][NLD];
    block_pipeline<DEPTH>(
        bt_row, first, NW, k0, nk, lane, ids0,
        [&](int d, int b, int k, bool exists) { load(kb[d], vb[d], b, first + k * NW, exists); },
        [&](int d, int k) { consume(kb[d], vb[d], first + k * NW); });
  }


  // Row groups of this wave -> one state per D chunk (all rows agree).
  merge_all_rows<LPT, EPL>(m, l, o);

  float outv[EPL];
  float M = m, L = l;
  if constexpr (NW > 1) {
    __shared__ float sm_o[NW][D];
    __shared__ float sm_m[NW], sm_l[NW];
    __shared__ int sm_bad[NW];
    if (r == 0) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_o[w][c * EPL + e] = o[e];
      if (c == 0) {
        sm_m[w] = m;
        sm_l[w] = l;
        sm_bad[w] = bad ? 1 : 0;
      }
    }
    __syncthreads();
    if (w != 0 || r != 0) return;
    M = sm_m[0];
#pragma unroll
    for (int v = 1; v < NW; ++v) M = fmaxf(M, sm_m[v]);
    const float m_use = (M == -INFINITY) ? 0.0f : M;
    L = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) outv[e] = 0.0f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const float sc = exp2_fast(sm_m[v] - m_use);
      L += sm_l[v] * sc;
#pragma unroll
      for (int e = 0; e < EPL; ++e) outv[e] += sm_o[v][c * EPL + e] * sc;
      bad |= sm_bad[v] != 0;
    }
  } else {
    if (r != 0) return;
#pragma unroll
    for (int e = 0; e < EPL; ++e) outv[e] = o[e];
  }

  // Lanes 0 .. LPT-1 of wave 0 hold the result for chunk c. One partition of
  // several (or the group pass of a shared prefix): the partial and its
  // (m, l). Else the final row; the shared-prefix tail pass first folds in the
  // group pass's partials of the row.
  const bool to_partial = P.always_partial || (P.partition > 0 && nparts_s > 1);
  float mul;  // applied to every dim below
  if (to_partial) {
    mul = 1.0f;  // fp32 partials: the unnormalised state itself
    if constexpr (sizeof(T) == 2) {
      // fp16 partial (see PartScale); the row's LPT lanes are lanes 0 .. LPT-1
      float amax = 0.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(outv[e]));
      const PartScale ps = part_scale_f16(M, L, group_max<LPT>(amax));
      mul = ps.mul;
      M = ps.m;
      L = ps.l;
    }
  } else {
    if constexpr (kTail)
      merge_shared_partials<T, EPL>(P, is.bad ? 0 : is.start_blk * kBlock, row, h, c * EPL, D, M,
                                    L, outv);
    mul = L > 0.0f ? 1.0f / L : 0.0f;  // empty context -> zeros
  }
  float res[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) res[e] = bad ? __builtin_nanf("") : outv[e] * mul;
  if (to_partial) {
    const size_t part = part_slot(P, row, h, P.part_base + p);
    if (c == 0) {
      P.ws_ml[2 * part] = bad ? 0.0f : M;
      P.ws_ml[2 * part + 1] = bad ? __builtin_nanf("") : L;
    }
    if constexpr (sizeof(T) == 2) {
      store_part16(P, row, h, P.part_base + p, 2, c * 16,
                   make_uint4(pack_f16x2(res[0], res[1]), pack_f16x2(res[2], res[3]),
                              pack_f16x2(res[4], res[5]), pack_f16x2(res[6], res[7])));
    } else {
      store_part16(P, row, h, P.part_base + p, 4, c * 16,
                   make_uint4(__float_as_uint(res[0]), __float_as_uint(res[1]),
                              __float_as_uint(res[2]), __float_as_uint(res[3])));
    }
    return;
  }
  char* out = reinterpret_cast<char*>(P.out) + row_qo * sizeof(T) + c * 16;
  if constexpr (sizeof(T) == 2) {
    uint4 u;
    u.x = pack_bf16x2(res[0], res[1]);
    u.y = pack_bf16x2(res[2], res[3]);
    u.z = pack_bf16x2(res[4], res[5]);
    u.w = pack_bf16x2(res[6], res[7]);
    st16(out, u);
  } else {
    st16(out, make_uint4(__float_as_uint(res[0]), __float_as_uint(res[1]),
                         __float_as_uint(res[2]), __float_as_uint(res[3])));
  }
}

template <TilePolicy kPolicy, int NW, int DEPTH = PA_VALU_DEPTH, bool kTail = false>
hipError_t launch_valu(const DecodeParams& p, int dtype, int D, hipStream_t stream) {
  const dim3 grid(p.Hq * p.max_q, p.pass_parts, p.pass_items), block(NW * kWave);
  if (dtype == 1 && D == 128)
    hipLaunchKernelGGL((decode_valu_kernel<uint16_t, 128, NW, DEPTH, kPolicy, kTail>), grid, block, 0,
                       stream, p);
  else if (dtype == 1 && D == 64)
    hipLaunchKernelGGL((decode_valu_kernel<uint16_t, 64, NW, DEPTH, kPolicy, kTail>), grid, block, 0,
                       stream, p);
  else if (dtype == 0 && D == 128) {
    // fp32 rows of 128 need ~220 registers: at most 8 waves per workgroup
    if constexpr (NW <= 8)
      hipLaunchKernelGGL((decode_valu_kernel<float, 128, NW, DEPTH, kPolicy, kTail>), grid, block, 0,
                         stream, p);
    else
      return hipErrorInvalidValue;
  }
  else if (dtype == 0 && D == 64)
    hipLaunchKernelGGL((decode_valu_kernel<float, 64, NW, DEPTH, kPolicy, kTail>), grid, block, 0,
                       stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_decode_valu(const DecodeParams& p, int dtype, int D, hipStream_t stream) {
  constexpr int TD = PA_VALU_TAIL_DEPTH;
  if (p.tail_pass)
    return p.shared_kv
               ? launch_valu<TilePolicy::kShared, PA_VALU_TAIL_WAVES, TD, true>(p, dtype, D, stream)
               : launch_valu<TilePolicy::kStream, PA_VALU_TAIL_WAVES, TD, true>(p, dtype, D, stream);
  if (p.few_items)
    return p.shared_kv ? launch_valu<TilePolicy::kShared, PA_VALU_WAVES_FEW>(p, dtype, D, stream)
                       : launch_valu<TilePolicy::kStream, PA_VALU_WAVES_FEW>(p, dtype, D, stream);
  return p.shared_kv ? launch_valu<TilePolicy::kShared, PA_VALU_WAVES>(p, dtype, D, stream)
                     : launch_valu<TilePolicy::kStream, PA_VALU_WAVES>(p, dtype, D, stream);
}

}  // namespace pa
