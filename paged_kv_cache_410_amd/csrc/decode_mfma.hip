// Paged decode attention for grouped query heads, matrix-core path
// (bf16, head_dim 128, G = Hq / Hkv query heads per kv head).
//
// Method: as the vector path ("Why OS Virtual Memory Paging Saved LLM
// Inference" (a8q9.cn), section 2: K/V gathered block by block through the
// block table; online softmax over blocks). With G query heads sharing one
// kv head, each 16-token K tile meets a G x 128 query block: a small, real
// contraction, done on the MFMA units so that every K/V byte is read once
// for all G heads.
//
// Layouts (wave64; lane = 16 * rg + col, rg = lane / 16, col = lane % 16):
//   S^T = K Q^T with v_mfma_f32_16x16x32_bf16, 4 steps over D (kk = 0..3):
//     A (16 tokens x 32 dims): lane holds K[t = col][32 kk + 8 rg + 0..7]
//     B (32 dims x 16 heads):  lane holds Q[q = col][32 kk + 8 rg + 0..7]
//     result: lane holds S^T[t = 4 rg + i][q = col], i = 0..3
//   So every lane owns one query head (col) and 4 tokens: the softmax max is
//   an in-lane max plus a max over the 4 row groups.
//   O^T = V^T P^T with v_mfma_f32_16x16x16_bf16 (K dimension = 16 tokens):
//     V is loaded row-wise: lane holds V[t = 4 rg + j][8 col + 0..7], j = 0..3
//     (each load instruction reads 4 whole 256-byte rows).
//     For output tile e (e = 0..7) the A operand (16 "dims" x 16 tokens) is
//     {V[4 rg + j][8 col + e]}_j, i.e. row m = col stands for dim 8 m + e;
//     it is assembled from the loaded registers with byte permutes.
//     B (16 tokens x 16 heads): lane holds P^T[t = 4 rg + j][q = col] = the
//     lane's own 4 probabilities, rounded to bf16.
//     result tile e: lane holds O^T[d = 8 (4 rg + i) + e][q = col].
//   Every accumulator a lane holds belongs to its own query head, so the
//   online-softmax rescale is a per-lane multiply.
// Heads past G in a 16-wide group are zero-padded and never written.
#include "pa_device.h"
#include "pa_launch.h"

// Waves per workgroup and K/V tiles in flight per wave.
#ifndef PA_MFMA_WAVES
#define PA_MFMA_WAVES 2
#endif
#ifndef PA_MFMA_DEPTH
#define PA_MFMA_DEPTH 2
#endif
// Minimum waves per SIMD the register allocation must allow.
#ifndef PA_MFMA_MIN_WAVES
#define PA_MFMA_MIN_WAVES 3
#endif

namespace pa {

namespace {

__device__ __forceinline__ uint32_t pack_lo16(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x05040100u);  // (x.lo, y.lo)
}
__device__ __forceinline__ uint32_t pack_hi16(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x07060302u);  // (x.hi, y.hi)
}
__device__ __forceinline__ uint32_t word(const uint4& u, int k) {
  return k == 0 ? u.x : k == 1 ? u.y : k == 2 ? u.z : u.w;
}

}  // namespace

template <int NW, int DEPTH>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(PA_MFMA_MIN_WAVES)))
void decode_mfma_kernel(DecodeParams P) {
  constexpr int D = 128;
  constexpr int kRowBytes = D * 2;
  constexpr int kPad = 4;  // LDS row padding (floats) against bank conflicts

  const int lane = threadIdx.x & (kWave - 1);
  const int w = wave_id();
  const int col = lane & 15;
  const int rg = lane >> 4;

  const GridPos gp = grid_pos();
  const int p = gp.y;
  const int QG = mfma_q_groups(P.G);
  const int g = gp.x / QG;
  const int sub = gp.x % QG;
  const int s = gp.z;
  const int q0 = g * P.G + sub * 16;           // first query head of this group
  const int gsub = min(16, P.G - sub * 16);     // real heads in the group

  const int32_t* bt_row = P.block_tables + (size_t)s * P.MB;
  const int bpp = P.partition / kBlock;  // blocks per partition (0: no split)
  const int blk_begin = p * bpp;
  const int first = blk_begin + w;       // this wave's blocks: first, first + NW, ...

  // Start-up loads, issued together before anything waits on them: the query
  // group, the wave's first 64 block ids (bounded by the partition's table
  // range, as the context length is not known yet) and the context length.
  // B operand of S^T: Q[q0 + col][32 kk + 8 rg ..], zero for padded heads.
  bf16x8_t qop[4];
  {
    const char* qrow = reinterpret_cast<const char*>(P.q) +
                       ((size_t)s * P.Hq + q0 + min(col, gsub - 1)) * kRowBytes;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      uint4 u = ld16(qrow + (32 * kk + 8 * rg) * 2);
      if (col >= gsub) u = make_uint4(0, 0, 0, 0);
      qop[kk] = __builtin_bit_cast(bf16x8_t, u);
    }
  }
  const int ids0 = first_chunk_ids(bt_row, first, NW, bpp > 0 ? min(P.MB, blk_begin + bpp) : P.MB,
                                   lane);
  const int ctx = P.context_lens[s];

  const bool bad_ctx = ctx < 0 || ctx > P.ctx_limit;
  const int nblk = bad_ctx ? 0 : (ctx + kBlock - 1) / kBlock;
  const int blk_end = bpp > 0 ? min(nblk, blk_begin + bpp) : nblk;
  const int nparts_s = bpp > 0 ? (nblk + bpp - 1) / bpp : (nblk > 0 ? 1 : 0);
  if (p >= max(nparts_s, 1)) return;  // partition past this sequence's end

  float m = -INFINITY, lsum = 0.0f;
  f32x4_t acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  bool bad = bad_ctx;

  const char* kbase = reinterpret_cast<const char*>(P.k_cache);
  const char* vbase = reinterpret_cast<const char*>(P.v_cache);
  const size_t head_off = (size_t)g * kBlock * kRowBytes;
  const size_t block_stride = (size_t)P.Hkv * kBlock * kRowBytes;
  const int k_lane = col * kRowBytes + 8 * rg * 2;       // + 64 B per kk
  const int v_lane = (4 * rg) * kRowBytes + 8 * col * 2;  // + 1 row per j

  // Issue the loads of physical block b's tile (logical block blk) into
  // (kb, vb). An id outside the pool marks the group bad and loads nothing;
  // so does a block that does not exist (an empty ring refill).
  auto load = [&](uint4 (&kb)[4], uint4 (&vb)[4], int b, int blk, bool exists) {
    const bool valid = b >= 0 && b < P.NB;
    bad |= exists && !valid;
    const size_t off = (size_t)(valid ? b : 0) * block_stride + head_off;
    // only the block's rows inside the context are fetched (the rest read as 0)
    const int rows = min(kBlock, ctx - blk * kBlock);
    const int bytes = exists && valid ? rows * kRowBytes : 0;
    const rsrc_t rk = make_rsrc(kbase + off, bytes);
    const rsrc_t rv = make_rsrc(vbase + off, bytes);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) kb[kk] = ld16(rk, k_lane + kk * 64);
#pragma unroll
    for (int j = 0; j < 4; ++j) vb[j] = ld16(rv, v_lane + j * kRowBytes);
  };

  auto consume = [&](const uint4 (&kb)[4], const uint4 (&vbin)[4], int blk) {
    f32x4_t st = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kb[kk]), qop[kk],
                                                  st, 0, 0, 0);
    const int tok0 = blk * kBlock + 4 * rg;
    const bool partial = blk * kBlock + kBlock > ctx;  // wave-uniform
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = st[i] * P.qscale;
      if (partial && tok0 + i >= ctx) x[i] = -INFINITY;
    }
    uint4 vb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      vb[j] = vbin[j];
      // rows past the context may hold anything (even NaN): select, not multiply
      if (partial && tok0 + j >= ctx) vb[j] = make_uint4(0, 0, 0, 0);
    }
    const float mx = rows_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = exp2_fast(m - m_use);
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = exp2_fast(x[i] - m_use);
    lsum = lsum * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
    m = m_new;
    const uint32_t p01 = pack_bf16x2(pr[0], pr[1]);
    const uint32_t p23 = pack_bf16x2(pr[2], pr[3]);
    const s16x4_t pop = __builtin_bit_cast(s16x4_t, make_uint2(p01, p23));
#pragma unroll
    for (int k = 0; k < 4; ++k) {  // 32-bit word k of each V chunk: dims 2k, 2k+1
      const uint32_t w0 = word(vb[0], k), w1 = word(vb[1], k);
      const uint32_t w2 = word(vb[2], k), w3 = word(vb[3], k);
      const s16x4_t a_lo = __builtin_bit_cast(s16x4_t, make_uint2(pack_lo16(w0, w1), pack_lo16(w2, w3)));
      const s16x4_t a_hi = __builtin_bit_cast(s16x4_t, make_uint2(pack_hi16(w0, w1), pack_hi16(w2, w3)));
      acc[2 * k] *= alpha;
      acc[2 * k + 1] *= alpha;
      acc[2 * k] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_lo, pop, acc[2 * k], 0, 0, 0);
      acc[2 * k + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_hi, pop, acc[2 * k + 1], 0, 0, 0);
    }
  };

  // This wave's blocks: first + k * NW, k < nk, through a ring of DEPTH tiles.
  {
    const int nk = first < blk_end ? (blk_end - first + NW - 1) / NW : 0;
    uint4 kb[DEPTH][4], vb[DEPTH][4];
    block_pipeline<DEPTH>(
        bt_row, first, NW, nk, lane, ids0,
        [&](int d, int b, int k, bool exists) { load(kb[d], vb[d], b, first + k * NW, exists); },
        [&](int d, int k) { consume(kb[d], vb[d], first + k * NW); });
  }


  lsum = rows_sum(lsum);  // per query head: sum over the 4 row groups

  // Waves -> LDS -> one merged state per (head, dim).
  __shared__ float sm_o[NW][16][D + kPad];
  __shared__ float sm_m[NW][16], sm_l[NW][16];
  __shared__ int sm_bad[NW];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float* dst = &sm_o[w][col][8 * (4 * rg + i)];
    // tile e holds dim 8 (4 rg + i) + e
    *reinterpret_cast<float4*>(dst) = make_float4(acc[0][i], acc[1][i], acc[2][i], acc[3][i]);
    *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[4][i], acc[5][i], acc[6][i], acc[7][i]);
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
  const bool split_out = P.partition > 0 && nparts_s > 1;
  // thread -> (head qq, 8-dim chunk ch)
  for (int t = threadIdx.x; t < 16 * 16; t += NW * kWave) {
    const int qq = t >> 4, ch = t & 15;
    if (qq >= gsub) continue;
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
    const int h = q0 + qq;
    if (split_out) {
      const size_t part = ((size_t)s * P.Hq + h) * P.n_parts + p;
      float* dst = P.ws_o + part * D + 8 * ch;
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[e] = any_bad ? __builtin_nanf("") : ov[e];
      if (ch == 0) {
        P.ws_ml[2 * part] = any_bad ? 0.0f : M;
        P.ws_ml[2 * part + 1] = any_bad ? __builtin_nanf("") : L;
      }
    } else {
      const float inv = L > 0.0f ? 1.0f / L : 0.0f;
      float res[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) res[e] = any_bad ? __builtin_nanf("") : ov[e] * inv;
      uint4 u;
      u.x = pack_bf16x2(res[0], res[1]);
      u.y = pack_bf16x2(res[2], res[3]);
      u.z = pack_bf16x2(res[4], res[5]);
      u.w = pack_bf16x2(res[6], res[7]);
      st16(reinterpret_cast<char*>(P.out) + (((size_t)s * P.Hq + h) * D + 8 * ch) * 2, u);
    }
  }
}

hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t stream) {
  constexpr int NW = PA_MFMA_WAVES;
  constexpr int DEPTH = PA_MFMA_DEPTH;
  const dim3 grid(p.Hkv * mfma_q_groups(p.G), p.n_parts, p.B), block(NW * kWave);
  hipLaunchKernelGGL((decode_mfma_kernel<NW, DEPTH>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
