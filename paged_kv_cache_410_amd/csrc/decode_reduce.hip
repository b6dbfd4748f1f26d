// Split-context merge: combines the per-partition partial results of a
// (sequence, query head) into the final output row.
//
// Each partition j left (m_j, l_j, O_j): its running max and softmax sum in
// the log2 domain and its unnormalised output row (for bf16 I/O an fp16 row
// of an equivalent, rescaled state). With M = max_j m_j and w_j = 2^(m_j - M),
// the full-context result is
//     out = (sum_j w_j O_j) / (sum_j w_j l_j),
// the same online-softmax rescaling the decode kernels apply between blocks,
// applied once more between partitions. (The pages describe attention run
// block by block; partitioning long contexts across workgroups is this
// library's way to spread one sequence over many compute units.)
//
// One workgroup of RW waves per (query head, query row). Wave w takes
// partitions w, w + RW, ... in rounds of kUnroll: lane i loads the (m, l) of
// the round's i-th partition while every lane loads its dims of all the
// round's rows, in one round trip; the wave's running max moves once per
// round (the rows summed before are rescaled, as between blocks in the
// decode kernels), the weights are broadcast with readlane. The waves' states
// are merged through LDS.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr int kReduceWaves = 4;

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<kDppXor1>(x));
  x = fmaxf(x, dpp<kDppXor2>(x));
  x = fmaxf(x, dpp<kDppHalfMirror>(x));
  x = fmaxf(x, dpp<kDppMirror>(x));
  return rows_max(x);
}

// T: the output's element type; E: the partial rows' (fp16 for bf16 output,
// fp32 for fp32), chosen at launch.
template <typename T, typename E, int D>
__global__ __launch_bounds__(kReduceWaves * kWave) void decode_reduce_kernel(DecodeParams P) {
  constexpr int RW = kReduceWaves;
  constexpr int DPL = D / kWave;  // output dims per lane
  constexpr int kUnroll = 16;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = wave_id();
  const int h = blockIdx.x;
  const int i = blockIdx.y;  // query row of the sequence (0 for decode)
  const int s = blockIdx.z;

  const SeqRows sr = seq_rows(P, s);
  if (i >= min(sr.n, P.max_q) || sr.bad) return;  // no row, or NaN written already
  const int nblk = (sr.row_ctx(i) + kBlock - 1) / kBlock;
  const int bpp = P.partition / kBlock;
  const int np = (nblk + bpp - 1) / bpp;
  if (np <= 1) return;  // the attention kernel wrote the final row itself

  const int row = sr.first + i;
  // partial j of this row and head sits at slot part_slot(row, h, j): Hq slots apart
  const size_t base = part_slot(P, row, h, 0);
  const size_t jstride = P.Hq;
  const float* ml = P.ws_ml + 2 * base;
  const E* po = static_cast<const E*>(P.ws_o) + base * D + lane * DPL;

  // One pass: each round, every lane loads the (m, l) of one of the wave's
  // next kUnroll partitions while all lanes load those partitions' rows; the
  // running max moves once per round and rescales what was summed before
  // (the online-softmax merge), so the rows never wait for a max pass.
  // This wave's partitions: j = w + RW * i, i < nw.
  const int nw = w < np ? (np - w + RW - 1) / RW : 0;
  float Mw = -INFINITY, lw = 0.0f;
  float acc[DPL];
#pragma unroll
  for (int d = 0; d < DPL; ++d) acc[d] = 0.0f;
  for (int i0 = 0; i0 < nw; i0 += kUnroll) {
    const int cnt = min(kUnroll, nw - i0);
    float mi = -INFINITY, li = 0.0f;
    if (lane < cnt) {
      const int j = w + RW * (i0 + lane);
      mi = ml[2 * j * jstride];
      li = ml[2 * j * jstride + 1];
    }
    float v[kUnroll][DPL];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int k = min(u, cnt - 1);  // repeats are weighted by 0 below
      const E* src = po + (size_t)(w + RW * (i0 + k)) * jstride * D;
#pragma unroll
      for (int d = 0; d < DPL; ++d) v[u][d] = elem_f32(src[d]);
    }
    const float Mn = fmaxf(Mw, wave_max(mi));
    const float m_use = (Mn == -INFINITY) ? 0.0f : Mn;
    const float a = exp2_fast(Mw - m_use);  // rescale of the earlier rounds
    const float wi = lane < cnt ? exp2_fast(mi - m_use) : 0.0f;
    lw = lw * a + group_sum<kWave>(wi * li);
#pragma unroll
    for (int d = 0; d < DPL; ++d) acc[d] *= a;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float wk = u < cnt ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wi), u))
                               : 0.0f;
#pragma unroll
      for (int d = 0; d < DPL; ++d) acc[d] = fmaf(wk, v[u][d], acc[d]);
    }
    Mw = Mn;
  }

  // The waves' states, each relative to its own max, merged through LDS.
  __shared__ float sm_acc[RW][D];
  __shared__ float sm_l[RW], sm_m[RW];
#pragma unroll
  for (int d = 0; d < DPL; ++d) sm_acc[w][lane * DPL + d] = acc[d];
  if (lane == 0) {
    sm_l[w] = lw;
    sm_m[w] = Mw;
  }
  __syncthreads();
  if (w != 0) return;
  float M = sm_m[0];
#pragma unroll
  for (int v = 1; v < RW; ++v) M = fmaxf(M, sm_m[v]);
  const float m_use = (M == -INFINITY) ? 0.0f : M;
  float L = 0.0f;
#pragma unroll
  for (int d = 0; d < DPL; ++d) acc[d] = 0.0f;
#pragma unroll
  for (int v = 0; v < RW; ++v) {
    const float sc = exp2_fast(sm_m[v] - m_use);
    L += sm_l[v] * sc;
#pragma unroll
    for (int d = 0; d < DPL; ++d) acc[d] += sm_acc[v][lane * DPL + d] * sc;
  }
  const float inv = 1.0f / L;
  char* out = reinterpret_cast<char*>(P.out) + (((size_t)row * P.Hq + h) * D + lane * DPL) * sizeof(T);
  if constexpr (sizeof(T) == 2) {
    if constexpr (DPL == 2) {
      *reinterpret_cast<uint32_t*>(out) = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    } else {
      const uint32_t pr = pack_bf16x2(acc[0] * inv, 0.0f);
      *reinterpret_cast<uint16_t*>(out) = (uint16_t)(pr & 0xffffu);
    }
  } else {
#pragma unroll
    for (int d = 0; d < DPL; ++d) reinterpret_cast<float*>(out)[d] = acc[d] * inv;
  }
}

hipError_t launch_decode_reduce(const DecodeParams& p, int dtype, int D, hipStream_t stream) {
  const dim3 grid(p.Hq, p.max_q, p.B), block(kReduceWaves * kWave);
  // bf16 output: fp16 partial rows; fp32 output: fp32 rows
  if (p.part_f32 != (dtype == 0)) return hipErrorInvalidValue;
  if (dtype == 1 && D == 128)
    hipLaunchKernelGGL((decode_reduce_kernel<uint16_t, _Float16, 128>), grid, block, 0, stream, p);
  else if (dtype == 1 && D == 64)
    hipLaunchKernelGGL((decode_reduce_kernel<uint16_t, _Float16, 64>), grid, block, 0, stream, p);
  else if (dtype == 0 && D == 128)
    hipLaunchKernelGGL((decode_reduce_kernel<float, float, 128>), grid, block, 0, stream, p);
  else if (dtype == 0 && D == 64)
    hipLaunchKernelGGL((decode_reduce_kernel<float, float, 64>), grid, block, 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
