// Split-context merge: combines the per-partition partial results of a
// (sequence, query head) into the final output row.
//
// Each partition j left (m_j, l_j, O_j): its running max and softmax sum in
// the log2 domain and its unnormalised output row. With M = max_j m_j and
// w_j = 2^(m_j - M), the full-context result is
//     out = (sum_j w_j O_j) / (sum_j w_j l_j),
// the same online-softmax rescaling the decode kernels apply between blocks,
// applied once more between partitions. (The pages describe attention run
// block by block; partitioning long contexts across workgroups is this
// library's way to spread one sequence over many compute units.)
//
// One workgroup of RW waves per (query head, query row). Every wave finds M
// over all partitions; wave w then accumulates partitions w, w + RW, ...,
// reading kUnroll partial rows per round trip (lane i holds w_j for the i-th
// partition of the wave's current chunk, broadcast with readlane, while every
// lane accumulates its own dims of the output row); the waves' sums are
// combined through LDS.
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

template <typename T, int D>
__global__ __launch_bounds__(kReduceWaves * kWave) void decode_reduce_kernel(DecodeParams P) {
  constexpr int RW = kReduceWaves;
  constexpr int DPL = D / kWave;  // output dims per lane
  constexpr int kUnroll = 8;
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
  const size_t base = ((size_t)row * P.Hq + h) * P.n_parts;
  const float* ml = P.ws_ml + 2 * base;
  const float* po = P.ws_o + base * D + lane * DPL;

  float M = -INFINITY;
  for (int j = lane; j < np; j += kWave) M = fmaxf(M, ml[2 * j]);
  M = wave_max(M);
  const float m_use = (M == -INFINITY) ? 0.0f : M;

  // this wave's partitions: j = w + RW * i, i < nw
  const int nw = w < np ? (np - w + RW - 1) / RW : 0;
  float lpart = 0.0f;
  float acc[DPL];
#pragma unroll
  for (int d = 0; d < DPL; ++d) acc[d] = 0.0f;
  for (int i0 = 0; i0 < nw; i0 += kWave) {
    const int i = i0 + lane;
    float wj = 0.0f;
    if (i < nw) {
      const int j = w + RW * i;
      wj = exp2_fast(ml[2 * j] - m_use);
      lpart += wj * ml[2 * j + 1];
    }
    const int cnt = min(kWave, nw - i0);
    for (int k0 = 0; k0 < cnt; k0 += kUnroll) {
      float v[kUnroll][DPL];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int k = min(k0 + u, cnt - 1);  // repeats are weighted by 0 below
        const float* src = po + (size_t)(w + RW * (i0 + k)) * D;
#pragma unroll
        for (int d = 0; d < DPL; ++d) v[u][d] = src[d];
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const float wk = k0 + u < cnt
                             ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wj), k0 + u))
                             : 0.0f;
#pragma unroll
        for (int d = 0; d < DPL; ++d) acc[d] = fmaf(wk, v[u][d], acc[d]);
      }
    }
  }

  __shared__ float sm_acc[RW][D];
  __shared__ float sm_l[RW];
#pragma unroll
  for (int d = 0; d < DPL; ++d) sm_acc[w][lane * DPL + d] = acc[d];
  const float lw = group_sum<kWave>(lpart);
  if (lane == 0) sm_l[w] = lw;
  __syncthreads();
  if (w != 0) return;
  float L = 0.0f;
#pragma unroll
  for (int v = 0; v < RW; ++v) L += sm_l[v];
#pragma unroll
  for (int d = 0; d < DPL; ++d) {
    float t = 0.0f;
#pragma unroll
    for (int v = 0; v < RW; ++v) t += sm_acc[v][lane * DPL + d];
    acc[d] = t;
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
  if (dtype == 1 && D == 128)
    hipLaunchKernelGGL((decode_reduce_kernel<uint16_t, 128>), grid, block, 0, stream, p);
  else if (dtype == 1 && D == 64)
    hipLaunchKernelGGL((decode_reduce_kernel<uint16_t, 64>), grid, block, 0, stream, p);
  else if (dtype == 0 && D == 128)
    hipLaunchKernelGGL((decode_reduce_kernel<float, 128>), grid, block, 0, stream, p);
  else if (dtype == 0 && D == 64)
    hipLaunchKernelGGL((decode_reduce_kernel<float, 64>), grid, block, 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
