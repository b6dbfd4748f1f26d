// Checks of the preconditions the write, copy and attention calls take on
// trust, for debugging a caller: each counts the violating entries of its
// input on the device. The calls they guard are these:
//   - the cache write fills the slots the block table maps new tokens to
//     ("Why OS Virtual Memory Paging Saved LLM Inference" (a8q9.cn),
//     section 2): two tokens of one call must not share a slot;
//   - copy-on-write gives a branch a private copy of a shared block before
//     it writes (same page, section 3): the copies of one call must not
//     write one block twice, nor write a block another copy reads;
//   - attention reads each sequence's blocks through its table (section 2):
//     every entry below the context length must name a pool block, and the
//     length must lie within the table and the caller's bound.
//   - shared-prefix decode reads a group's shared blocks once, through its
//     first member's table (section 3: sharers point at the same blocks):
//     the groups must cover the batch in order, and every member must share
//     the same whole blocks, inside its own context.
// Each check is two launches on the caller's stream: one thread clears the
// counter, then the count is added up with one atomic add per wave.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

namespace {

__global__ void clear_count_kernel(int32_t* count) { *count = 0; }

// Adds this wave's violations (one flag per lane) to the counter.
__device__ __forceinline__ void count_violations(bool bad, int32_t* count) {
  const uint64_t mask = __builtin_amdgcn_ballot_w64(bad);
  const int lane = threadIdx.x & (kWave - 1);
  if (lane == 0 && mask != 0) atomicAdd(count, (int32_t)__builtin_popcountll(mask));
}

// Token i violates when its slot is non-negative and an earlier token of the
// call has the same slot. The loop over earlier tokens is uniform across the
// wave, so every slot read is one broadcast load.
__global__ void check_slots_kernel(const int32_t* __restrict__ slots, int32_t T,
                                   int32_t* count) {
  const int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  const int32_t wave_first = i - (int32_t)(threadIdx.x & (kWave - 1));
  const int32_t mine = i < T ? slots[i] : -1;
  bool dup = false;
  const int32_t jmax = min(T, wave_first + kWave);
  for (int32_t j = 0; j < jmax; ++j) {
    const int32_t other = slots[j];
    dup |= j < i && mine >= 0 && other == mine;
  }
  count_violations(i < T && dup, count);
}

// Pair i (src, dst) with both ids inside [0, NB) (others are skipped by the
// copy) violates when an earlier such pair has the same destination, or when
// any such pair reads the block it writes.
__global__ void check_pairs_kernel(const int32_t* __restrict__ pairs, int32_t n, int32_t NB,
                                   int32_t* count) {
  const int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  auto live = [&](int32_t src, int32_t dst) {
    return src >= 0 && src < NB && dst >= 0 && dst < NB;
  };
  const int32_t src_i = i < n ? pairs[2 * i] : -1;
  const int32_t dst_i = i < n ? pairs[2 * i + 1] : -1;
  const bool mine = i < n && live(src_i, dst_i);
  bool bad = false;
  for (int32_t j = 0; j < n; ++j) {
    const int32_t src_j = pairs[2 * j];
    const int32_t dst_j = pairs[2 * j + 1];
    if (!live(src_j, dst_j)) continue;
    bad |= mine && ((j < i && dst_j == dst_i) || src_j == dst_i);
  }
  count_violations(bad, count);
}

// Sequence s violates when its context length is negative or above
// min(max_ctx, MB * 16), or when a table entry below ceil(length / 16)
// lies outside [0, NB).
__global__ void check_tables_kernel(const int32_t* __restrict__ bt,
                                    const int32_t* __restrict__ ctx_lens, int32_t B, int32_t MB,
                                    int32_t NB, int32_t ctx_limit, int32_t* count) {
  const int32_t s = blockIdx.x * blockDim.x + threadIdx.x;
  bool bad = false;
  if (s < B) {
    const int32_t L = ctx_lens[s];
    if (L < 0 || L > ctx_limit) {
      bad = true;
    } else {
      const int32_t* row = bt + (size_t)s * MB;
      for (int32_t j = 0; j < (L + kBlock - 1) / kBlock; ++j) {
        const int32_t b = row[j];
        bad |= b < 0 || b >= NB;
      }
    }
  }
  count_violations(bad, count);
}

// Group j violates when its bounds are out of order or outside [0, B], when
// it is empty or larger than max_group, or (j = 0, j = n - 1) when the groups
// do not start at 0 and end at B. Each member s of a well-formed group
// violates when its shared length differs from the first member's, is not a
// multiple of 16, exceeds its context or its table, or when one of its first
// S / 16 table entries differs from the first member's.
__global__ void check_groups_kernel(const int32_t* __restrict__ group_start,
                                    const int32_t* __restrict__ seq_shared,
                                    const int32_t* __restrict__ bt,
                                    const int32_t* __restrict__ ctx_lens, int32_t B,
                                    int32_t n_groups, int32_t max_group, int32_t MB,
                                    int32_t* count) {
  const int32_t j = blockIdx.x * blockDim.x + threadIdx.x;
  int32_t bad = 0;
  if (j < n_groups) {
    const int32_t a = group_start[j], b = group_start[j + 1];
    const bool ok = a >= 0 && b <= B && b > a && b - a <= max_group && (j > 0 || a == 0) &&
                    (j < n_groups - 1 || b == B);
    if (!ok) {
      bad = 1;
    } else {
      const int32_t S = seq_shared[a];
      const int32_t* first = bt + (size_t)a * MB;
      for (int32_t s = a; s < b; ++s) {
        const int32_t Ss = seq_shared[s];
        bool m = Ss != S || Ss < 0 || Ss % kBlock != 0 || Ss > ctx_lens[s] || Ss / kBlock > MB;
        if (!m) {
          const int32_t* row = bt + (size_t)s * MB;
          for (int32_t k = 0; k < Ss / kBlock; ++k) m |= row[k] != first[k];
        }
        bad += m ? 1 : 0;
      }
    }
  }
  // a lane may count several members: add the wave's sum
  int32_t sum = bad;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  if ((threadIdx.x & (kWave - 1)) == 0 && sum != 0) atomicAdd(count, sum);
}

constexpr int kThreads = 256;

}  // namespace

hipError_t launch_check_slots(const int32_t* slots, int32_t T, int32_t* count,
                              hipStream_t stream) {
  hipLaunchKernelGGL(clear_count_kernel, dim3(1), dim3(1), 0, stream, count);
  if (T > 0)
    hipLaunchKernelGGL(check_slots_kernel, dim3((T + kThreads - 1) / kThreads), dim3(kThreads), 0,
                       stream, slots, T, count);
  return hipGetLastError();
}

hipError_t launch_check_pairs(const int32_t* pairs, int32_t n, int32_t NB, int32_t* count,
                              hipStream_t stream) {
  hipLaunchKernelGGL(clear_count_kernel, dim3(1), dim3(1), 0, stream, count);
  if (n > 0)
    hipLaunchKernelGGL(check_pairs_kernel, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0,
                       stream, pairs, n, NB, count);
  return hipGetLastError();
}

hipError_t launch_check_tables(const int32_t* bt, const int32_t* ctx_lens, int32_t B, int32_t MB,
                               int32_t NB, int32_t ctx_limit, int32_t* count,
                               hipStream_t stream) {
  hipLaunchKernelGGL(clear_count_kernel, dim3(1), dim3(1), 0, stream, count);
  if (B > 0)
    hipLaunchKernelGGL(check_tables_kernel, dim3((B + kThreads - 1) / kThreads), dim3(kThreads),
                       0, stream, bt, ctx_lens, B, MB, NB, ctx_limit, count);
  return hipGetLastError();
}

hipError_t launch_check_groups(const int32_t* group_start, const int32_t* seq_shared,
                               const int32_t* bt, const int32_t* ctx_lens, int32_t B,
                               int32_t n_groups, int32_t max_group, int32_t MB, int32_t* count,
                               hipStream_t stream) {
  hipLaunchKernelGGL(clear_count_kernel, dim3(1), dim3(1), 0, stream, count);
  if (n_groups > 0)
    hipLaunchKernelGGL(check_groups_kernel, dim3((n_groups + kThreads - 1) / kThreads),
                       dim3(kThreads), 0, stream, group_start, seq_shared, bt, ctx_lens, B,
                       n_groups, max_group, MB, count);
  return hipGetLastError();
}

}  // namespace pa
