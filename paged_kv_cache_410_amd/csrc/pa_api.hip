// C ABI of the paged decode attention library: argument validation, kernel
// choice, grid and workspace layout. Every check here runs on the host before
// anything is launched; a failed check launches nothing.
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "pa.h"
#include "pa_launch.h"

// pa_decode_shared in one pass where it can (1), or always as a group pass
// and a tail pass (0, for measurement).
#ifndef PA_FOLD_TAILS
#define PA_FOLD_TAILS 1
#endif

namespace {

// Scratch of pa_decode_noalloc: the split-context partials of callers that
// cannot allocate. Each GPU the library runs on holds its own copy from the
// time the library's code is loaded there until the process ends. In host
// code `scratch` names a host-side stand-in, not device memory: only the
// address hipGetSymbolAddress returns for the current device is passed to
// kernels.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];  // per device, null until looked up
std::mutex g_scratch_mu;

// Device address of the current device's scratch (looked up once per device).
pa_status device_scratch(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PA_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return PA_EUNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PA_EHIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return PA_OK;
}

constexpr int32_t kBs = 16;
constexpr int32_t kMaxGridYZ = 65535;
constexpr size_t kAlign = 256;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int32_t elem_bytes(pa_dtype dt) { return dt == PA_F32 ? 4 : 2; }
bool dtype_ok(pa_dtype dt) { return dt == PA_F32 || dt == PA_BF16; }

// Partitions the grid covers for a split of `partition` tokens (1 = no split).
int64_t grid_parts(int32_t max_ctx, int32_t partition) {
  if (partition <= 0 || max_ctx <= partition) return 1;
  return ((int64_t)max_ctx + partition - 1) / partition;
}

// Partitions of the shared part of pa_decode_shared (0 when nothing is shared).
int64_t shared_parts(int32_t max_shared, int32_t partition) {
  if (max_shared <= 0) return 0;
  return partition > 0 ? ((int64_t)max_shared + partition - 1) / partition : 1;
}

int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

}  // namespace

extern "C" {

const char* pa_status_str(pa_status s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_EINVAL: return "invalid argument";
    case PA_EUNSUPPORTED: return "unsupported configuration";
    case PA_EWORKSPACE: return "workspace missing or too small";
    case PA_EHIP: return "HIP launch failure";
    case PA_ENOBLOCKS: return "not enough free KV blocks";
  }
  return "unknown status";
}

pa_status pa_slot_mapping(int32_t* slot_mapping, const int32_t* block_tables,
                          const int32_t* seq_ids, const int32_t* positions, int32_t T, int32_t B,
                          int32_t MB, int32_t bs, hipStream_t stream) {
  if (T < 0 || B < 0 || MB < 0) return PA_EINVAL;
  if (bs != kBs) return bs > 0 ? PA_EUNSUPPORTED : PA_EINVAL;
  if (!seq_ids && T > B) return PA_EINVAL;
  if (T == 0) return PA_OK;
  if (!slot_mapping || !positions || (B > 0 && MB > 0 && !block_tables)) return PA_EINVAL;
  return pa::launch_slot_mapping(slot_mapping, block_tables, seq_ids, positions, T, B, MB,
                                 stream) == hipSuccess
             ? PA_OK
             : PA_EHIP;
}

pa_status pa_write_kv(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                      const int32_t* slot_mapping, int32_t T, int32_t NB, int32_t Hkv, int32_t D,
                      int32_t bs, pa_dtype dt, hipStream_t stream) {
  if (T < 0 || NB < 0 || Hkv <= 0 || D <= 0 || !dtype_ok(dt)) return PA_EINVAL;
  if (bs != kBs) return bs > 0 ? PA_EUNSUPPORTED : PA_EINVAL;
  if (D != 64 && D != 128) return PA_EUNSUPPORTED;
  if (T == 0) return PA_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping) return PA_EINVAL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_EINVAL;
  if ((int64_t)T * Hkv * D * elem_bytes(dt) / 16 > (int64_t)INT32_MAX * 256) return PA_EUNSUPPORTED;
  return pa::launch_write_kv(k_new, v_new, k_cache, v_cache, slot_mapping, T, NB, Hkv,
                             D * elem_bytes(dt), stream) == hipSuccess
             ? PA_OK
             : PA_EHIP;
}

pa_status pa_append_kv(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                       int32_t* slot_mapping, const int32_t* block_tables, const int32_t* seq_ids,
                       const int32_t* positions, int32_t T, int32_t B, int32_t MB, int32_t NB,
                       int32_t Hkv, int32_t D, int32_t bs, pa_dtype dt, hipStream_t stream) {
  if (T < 0 || B < 0 || MB < 0 || NB < 0 || Hkv <= 0 || D <= 0 || !dtype_ok(dt)) return PA_EINVAL;
  if (bs != kBs) return bs > 0 ? PA_EUNSUPPORTED : PA_EINVAL;
  if (D != 64 && D != 128) return PA_EUNSUPPORTED;
  if (!seq_ids && T > B) return PA_EINVAL;
  if (T == 0) return PA_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !positions) return PA_EINVAL;
  if (B > 0 && MB > 0 && !block_tables) return PA_EINVAL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_EINVAL;
  if ((int64_t)T * Hkv * D * elem_bytes(dt) / 16 > (int64_t)INT32_MAX * 256) return PA_EUNSUPPORTED;
  return pa::launch_append_kv(k_new, v_new, k_cache, v_cache, slot_mapping, block_tables, seq_ids,
                              positions, T, B, MB, NB, Hkv, D * elem_bytes(dt), stream) == hipSuccess
             ? PA_OK
             : PA_EHIP;
}

pa_status pa_check_slots(const int32_t* slot_mapping, int32_t T, int32_t* count,
                         hipStream_t stream) {
  if (T < 0 || !count || (T > 0 && !slot_mapping)) return PA_EINVAL;
  return pa::launch_check_slots(slot_mapping, T, count, stream) == hipSuccess ? PA_OK : PA_EHIP;
}

pa_status pa_check_pairs(const int32_t* pairs, int32_t n, int32_t NB, int32_t* count,
                         hipStream_t stream) {
  if (n < 0 || NB < 0 || !count || (n > 0 && !pairs)) return PA_EINVAL;
  return pa::launch_check_pairs(pairs, n, NB, count, stream) == hipSuccess ? PA_OK : PA_EHIP;
}

pa_status pa_check_tables(const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                          int32_t MB, int32_t NB, int32_t max_ctx, int32_t bs, int32_t* count,
                          hipStream_t stream) {
  if (B < 0 || MB < 0 || NB < 0 || max_ctx < 0 || !count) return PA_EINVAL;
  if (bs != kBs) return bs > 0 ? PA_EUNSUPPORTED : PA_EINVAL;
  if (B > 0 && (!context_lens || (MB > 0 && !block_tables))) return PA_EINVAL;
  const int64_t cap = (int64_t)MB * kBs;
  const int32_t limit = (int32_t)(cap < max_ctx ? cap : max_ctx);
  return pa::launch_check_tables(block_tables, context_lens, B, MB, NB, limit, count, stream) ==
                 hipSuccess
             ? PA_OK
             : PA_EHIP;
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t n, int32_t NB,
                         int32_t Hkv, int32_t D, int32_t bs, pa_dtype dt, hipStream_t stream) {
  if (n < 0 || NB < 0 || Hkv <= 0 || D <= 0 || !dtype_ok(dt)) return PA_EINVAL;
  if (bs != kBs) return bs > 0 ? PA_EUNSUPPORTED : PA_EINVAL;
  if (D != 64 && D != 128) return PA_EUNSUPPORTED;
  if (n == 0) return PA_OK;
  if (!k_cache || !v_cache || !pairs) return PA_EINVAL;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return PA_EINVAL;
  const size_t block_bytes = (size_t)Hkv * kBs * D * elem_bytes(dt);
  for (int32_t done = 0; done < n; done += kMaxGridYZ) {
    const int32_t cnt = n - done < kMaxGridYZ ? n - done : kMaxGridYZ;
    if (pa::launch_copy_blocks(k_cache, v_cache, pairs + 2 * (size_t)done, cnt, NB, block_bytes,
                               stream) != hipSuccess)
      return PA_EHIP;
  }
  return PA_OK;
}

pa_status pa_check_groups(const int32_t* group_start, const int32_t* seq_shared,
                          const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                          int32_t n_groups, int32_t max_group, int32_t MB, int32_t bs,
                          int32_t* count, hipStream_t stream) {
  if (B < 0 || n_groups < 0 || max_group < 1 || MB < 0 || !count) return PA_EINVAL;
  if (bs != kBs) return bs > 0 ? PA_EUNSUPPORTED : PA_EINVAL;
  if (n_groups > 0 && (!group_start || !seq_shared || !context_lens || (MB > 0 && !block_tables)))
    return PA_EINVAL;
  return pa::launch_check_groups(group_start, seq_shared, block_tables, context_lens, B, n_groups,
                                 max_group, MB, count, stream) == hipSuccess
             ? PA_OK
             : PA_EHIP;
}

int32_t pa_decode_default_partition(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                    int32_t max_ctx) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || max_ctx <= 0) return 0;
  const int32_t G = Hq / Hkv;
  const int64_t units = (int64_t)B * (G >= 2 ? (int64_t)Hkv * pa::mfma_q_groups(G) : Hq);
  const int64_t cus = device_cus();
  // At least 4 unsplit (sequence, head) workgroups per CU keep every CU
  // busy: no split. For grouped heads (the matrix-core kernels, whose
  // unsplit workgroups stream a whole context on 8 waves) contexts up to
  // 2048 tokens are not split at all: there the partial rows and the merge
  // cost more than the added workgroups gain. Measured, 32 query heads:
  // with 8 kv heads, 128 sequences of lognormal lengths up to 2048, 61 us
  // unsplit against 94 at 512-token partitions; 128 of 512-4096 tokens, 201
  // against 212; 16 of up to 2048, 27.5 against 29.9; 16 of 2048-8192, 85.5
  // against 65.2 (split); 48 of 2048-8192, 186 against 167 (split). With 32
  // kv heads, 32 sequences (1024 workgroups) of 128-2048 tokens, 95.6 against
  // 102.5; of 512-4096, 195.7 against 200.8; 16 of 512-4096, 106.6 against
  // 109.3.
  if (units >= 4 * cus || max_ctx <= 512) return 0;
  if (G >= 2 && max_ctx <= 2048) return 0;
  return 512;
}

size_t pa_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t D, int32_t max_ctx,
                                 int32_t partition) {
  if (B <= 0 || Hq <= 0 || D <= 0 || max_ctx <= 0 || partition <= 0) return 0;
  const int64_t parts = grid_parts(max_ctx, partition);
  if (parts <= 1) return 0;
  const size_t rows = (size_t)B * Hq * (size_t)parts;
  // (m, l) in fp32, then the rows; a row takes D elements of the I/O dtype,
  // sized here for fp32 so that one size serves both dtypes
  return align_up(rows * 2 * sizeof(float)) + rows * (size_t)D * sizeof(float);
}

}  // extern "C"

namespace {

// Shared body of pa_decode (query_start == NULL: one query row per sequence)
// and pa_multi_query (rows query_start[s] .. query_start[s+1]-1 of sequence s).
pa_status attention(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens,
                    const int32_t* query_start, int32_t B, int32_t rows, int32_t max_q, int32_t Hq,
                    int32_t Hkv, int32_t D, int32_t bs, int32_t NB, int32_t MB, int32_t max_ctx,
                    float scale, int32_t partition, void* workspace, size_t workspace_bytes,
                    uint32_t flags, pa_dtype dt, hipStream_t stream, bool use_scratch = false) {
  if (B < 0 || rows < 0 || max_q < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || NB < 0 || MB < 0 ||
      max_ctx < 0 || !dtype_ok(dt) || (flags & ~PA_KV_SHARED) != 0 || !__builtin_isfinite(scale))
    return PA_EINVAL;
  if (Hq % Hkv != 0) return PA_EINVAL;
  if (partition < 0 || partition % kBs != 0) return PA_EINVAL;
  if (bs != kBs) return bs > 0 ? PA_EUNSUPPORTED : PA_EINVAL;
  if (D != 64 && D != 128) return PA_EUNSUPPORTED;
  if (B > kMaxGridYZ || max_q > kMaxGridYZ) return PA_EUNSUPPORTED;  // grid z / merge grid y
  if ((int64_t)Hq * max_q > INT32_MAX) return PA_EUNSUPPORTED;      // grid x
  if (B == 0 || rows == 0 || max_q == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !context_lens || (MB > 0 && !block_tables))
    return PA_EINVAL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_EINVAL;

  const int64_t parts = grid_parts(max_ctx, partition);
  const size_t need = pa_decode_workspace_bytes(rows, Hq, D, max_ctx, partition);
  if (use_scratch && need > 0) {
    // the library's own scratch in place of a caller's workspace
    if (need > PA_NOALLOC_SCRATCH_BYTES) return PA_EWORKSPACE;
    const pa_status st = device_scratch(&workspace);
    if (st != PA_OK) return st;
    workspace_bytes = PA_NOALLOC_SCRATCH_BYTES;
  }
  if (need > 0 && (!workspace || workspace_bytes < need)) return PA_EWORKSPACE;
  if (need > 0 && ((uintptr_t)workspace % kAlign) != 0) return PA_EINVAL;
  if (parts > kMaxGridYZ) return PA_EUNSUPPORTED;  // grid y

  pa::DecodeParams p{};
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.query_start = query_start;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.D = D;
  p.NB = NB;
  p.MB = MB;
  const int64_t cap = (int64_t)MB * kBs;
  p.ctx_limit = (int32_t)(cap < max_ctx ? cap : max_ctx);
  p.partition = parts > 1 ? partition : 0;
  p.n_parts = (int32_t)parts;
  p.pass_parts = (int32_t)parts;
  p.pass_items = B;
  // few long work items: wider workgroups (measured on the 7B-shape batch:
  // 2048 (sequence, head) items, 176 vs 180 us; the 13B-shape's 5120 items
  // keep 8 waves; fp32 rows of 128 keep 8 waves for registers)
  p.few_items = parts == 1 && !(dt == PA_F32 && D == 128) &&
                        (int64_t)B * Hq * max_q <= 8 * (int64_t)device_cus()
                    ? 1
                    : 0;
  p.max_q = max_q;
  p.rows = rows;
  p.n_tiles = (int32_t)(((int64_t)max_q * p.G + 15) / 16);
  p.qscale = scale * 1.4426950408889634f;
  p.shared_kv = (flags & PA_KV_SHARED) ? 1 : 0;
  if (parts > 1) {
    const size_t nrows = (size_t)rows * Hq * (size_t)parts;
    p.ws_ml = static_cast<float*>(workspace);
    p.ws_o = static_cast<char*>(workspace) + align_up(nrows * 2 * sizeof(float));
  }

  // The matrix-core kernels serve a kv head's columns (query rows x group
  // heads) 16 at a time; a single column per kv head (one query head, one
  // row) goes to the vector kernel. bf16: past 16 columns per kv head the
  // chunk kernel takes over; in fp32, one workgroup per 16-column tile.
  const bool several = p.G >= 2 || max_q >= 2;
  const bool mfma = dt == PA_BF16 && several;
  const bool mfma32 = dt == PA_F32 && several;
  if ((mfma || mfma32) && (int64_t)Hkv * p.n_tiles > INT32_MAX) return PA_EUNSUPPORTED;
  // partial rows: fp32 for fp32 I/O, scaled fp16 for bf16 (every kernel)
  p.part_f32 = dt == PA_F32;
  hipError_t err = mfma     ? pa::launch_decode_mfma(p, stream)
                   : mfma32 ? pa::launch_decode_mfma_f32(p, stream)
                            : pa::launch_decode_valu(p, dt, D, stream);
  if (err != hipSuccess) return PA_EHIP;
  if (parts > 1) {
    err = pa::launch_decode_reduce(p, dt, D, stream);
    if (err != hipSuccess) return PA_EHIP;
  }
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                    int32_t Hq, int32_t Hkv, int32_t D, int32_t bs, int32_t NB, int32_t MB,
                    int32_t max_ctx, float scale, int32_t partition, void* workspace,
                    size_t workspace_bytes, uint32_t flags, pa_dtype dt, hipStream_t stream) {
  return attention(out, q, k_cache, v_cache, block_tables, context_lens, nullptr, B, B, 1, Hq, Hkv,
                   D, bs, NB, MB, max_ctx, scale, partition, workspace, workspace_bytes, flags, dt,
                   stream);
}

pa_status pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                            int32_t Hq, int32_t Hkv, int32_t D, int32_t bs, int32_t NB,
                            int32_t MB, int32_t max_ctx, float scale, int32_t partition,
                            uint32_t flags, pa_dtype dt, hipStream_t stream) {
  return attention(out, q, k_cache, v_cache, block_tables, context_lens, nullptr, B, B, 1, Hq, Hkv,
                   D, bs, NB, MB, max_ctx, scale, partition, nullptr, 0, flags, dt, stream,
                   /*use_scratch=*/true);
}

int32_t pa_decode_shared_default_partition(int32_t n_groups, int32_t Hq, int32_t Hkv,
                                           int32_t max_group, int32_t max_shared) {
  if (n_groups <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || max_group < 1 || max_shared <= 0)
    return 0;
  // group-pass workgroups: one per (group, kv head) for one 16-column tile,
  // one per 8 tiles on the chunk kernel
  const int64_t tiles = ((int64_t)max_group * (Hq / Hkv) + 15) / 16;
  const int64_t items = (int64_t)n_groups * Hkv * (tiles > 1 ? (tiles + 7) / 8 : 1);
  // at least one per CU: one partition (measured best on the 16 x 8 COW and
  // 8 x 16 prefix MHA batches); fewer: two (a 64/8-head COW batch of 128
  // workgroups: 39.7 us against 46.0 unsplit and 43.4 with four)
  if (items >= device_cus()) return 0;
  const int32_t half = (max_shared / 2 + kBs - 1) / kBs * kBs;
  return half >= max_shared ? 0 : half;
}

size_t pa_decode_shared_workspace_bytes(int32_t B, int32_t Hq, int32_t D, int32_t max_shared,
                                        int32_t partition) {
  if (B <= 0 || Hq <= 0 || D <= 0 || max_shared < 0 || partition < 0) return 0;
  const int64_t nps = shared_parts(max_shared, partition);
  if (nps == 0) return 0;
  const size_t rows = (size_t)B * Hq * (size_t)nps;
  return align_up(rows * 2 * sizeof(float)) + rows * (size_t)D * sizeof(float);
}

pa_status pa_decode_shared(void* out, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* context_lens,
                           const int32_t* group_start, const int32_t* seq_shared, int32_t B,
                           int32_t n_groups, int32_t max_group, int32_t max_shared, int32_t Hq,
                           int32_t Hkv, int32_t D, int32_t bs, int32_t NB, int32_t MB,
                           int32_t max_ctx, float scale, int32_t partition, void* workspace,
                           size_t workspace_bytes, uint32_t flags, pa_dtype dt,
                           hipStream_t stream) {
  if (B < 0 || n_groups < 0 || max_group < 1 || max_shared < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 ||
      NB < 0 || MB < 0 || max_ctx < 0 || !dtype_ok(dt) ||
      (flags & ~(PA_KV_SHARED | PA_KV_SHARED_GROUPS)) != 0 || !__builtin_isfinite(scale))
    return PA_EINVAL;
  if (Hq % Hkv != 0) return PA_EINVAL;
  if (partition < 0 || partition % kBs != 0 || max_shared % kBs != 0) return PA_EINVAL;
  if (max_shared > max_ctx) return PA_EINVAL;
  if (bs != kBs) return bs > 0 ? PA_EUNSUPPORTED : PA_EINVAL;
  if (D != 64 && D != 128) return PA_EUNSUPPORTED;
  // the group pass runs on the matrix-core kernels: in bf16 the decode kernel
  // for one 16-column tile of (member, query head) pairs per kv head and the
  // chunk kernel for more, in fp32 the fp32 kernel (one workgroup per tile)
  const int32_t G = Hq / Hkv;
  const bool f32 = dt == PA_F32;
  if (B > kMaxGridYZ || n_groups > kMaxGridYZ || max_group > kMaxGridYZ) return PA_EUNSUPPORTED;
  const int64_t group_tiles = ((int64_t)max_group * G + 15) / 16;
  if ((int64_t)Hkv * group_tiles > INT32_MAX) return PA_EUNSUPPORTED;
  if (B == 0) return PA_OK;
  if (n_groups == 0) return PA_EINVAL;
  if (!out || !q || !k_cache || !v_cache || !context_lens || !group_start || !seq_shared ||
      (MB > 0 && !block_tables))
    return PA_EINVAL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_EINVAL;
  const int64_t nps = shared_parts(max_shared, partition);
  if (nps > kMaxGridYZ) return PA_EUNSUPPORTED;
  const size_t need = pa_decode_shared_workspace_bytes(B, Hq, D, max_shared, partition);
  if (need > 0 && (!workspace || workspace_bytes < need)) return PA_EWORKSPACE;
  if (need > 0 && ((uintptr_t)workspace % kAlign) != 0) return PA_EINVAL;

  pa::DecodeParams p{};
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = G;
  p.D = D;
  p.NB = NB;
  p.MB = MB;
  const int64_t cap = (int64_t)MB * kBs;
  p.ctx_limit = (int32_t)(cap < max_ctx ? cap : max_ctx);
  p.rows = B;
  p.qscale = scale * 1.4426950408889634f;
  p.shared_kv = (flags & PA_KV_SHARED) ? 1 : 0;
  p.seq_shared = seq_shared;
  p.n_parts = nps > 0 ? (int32_t)nps : 1;  // partial slots per (row, head)
  if (nps > 0) {
    const size_t nrows = (size_t)B * Hq * (size_t)nps;
    p.ws_ml = static_cast<float*>(workspace);
    p.ws_o = static_cast<char*>(workspace) + align_up(nrows * 2 * sizeof(float));
  }

  // One partition of the shared part and one column tile per kv head: a
  // single pass, each group's workgroup reading its shared blocks and then
  // every member's own blocks, writing the final rows (the workspace goes
  // unused). bf16 only.
  if (PA_FOLD_TAILS && !f32 && nps <= 1 && group_tiles == 1) {
    pa::DecodeParams g = p;
    g.group_start = group_start;
    g.fold_tails = 1;
    g.shared_kv = (flags & PA_KV_SHARED_GROUPS) ? 1 : 0;
    g.tail_shared_kv = (flags & PA_KV_SHARED) ? 1 : 0;
    g.max_q = max_group;
    g.n_tiles = 1;
    g.partition = 0;
    g.pass_parts = 1;
    g.pass_items = n_groups;
    g.n_cus = device_cus();
    return pa::launch_decode_mfma(g, stream) == hipSuccess ? PA_OK : PA_EHIP;
  }
  // 1. group pass: each group's shared tokens, read once for all its members
  if (nps > 0) {
    pa::DecodeParams g = p;
    g.group_start = group_start;
    g.shared_kv = (flags & PA_KV_SHARED_GROUPS) ? 1 : 0;
    g.max_q = max_group;
    g.n_tiles = (int32_t)group_tiles;
    g.part_f32 = f32;
    g.partition = nps > 1 ? partition : 0;
    g.part_base = 0;
    g.always_partial = 1;
    g.pass_parts = (int32_t)nps;
    g.pass_items = n_groups;
    if ((f32 ? pa::launch_decode_mfma_f32(g, stream) : pa::launch_decode_mfma(g, stream)) !=
        hipSuccess)
      return PA_EHIP;
  }
  // 2. tail pass: each sequence's own tokens past its shared ones, merged
  //    with its row's group-pass partials into the final row
  pa::DecodeParams t = p;
  t.tail_pass = 1;
  t.shared_partition = nps > 1 ? partition : 0;
  t.max_q = 1;
  t.n_tiles = (G + 15) / 16;
  t.part_f32 = f32;  // as the group pass wrote them
  t.partition = 0;
  t.pass_parts = 1;
  t.pass_items = B;
  // The tail pass: one query head per workgroup on the vector kernel for one
  // head per kv head; else a kv head's query heads on the matrix cores, 16
  // per workgroup in fp32, at most 16 in bf16 (past 16, bf16 goes to the
  // vector kernel: the decode kernel takes one tile per kv head)
  const bool valu_tail = G == 1 || (!f32 && G > 16);
  const hipError_t e = valu_tail ? pa::launch_decode_valu(t, dt, D, stream)
                       : f32     ? pa::launch_decode_mfma_f32(t, stream)
                                 : pa::launch_decode_mfma(t, stream);
  if (e != hipSuccess) return PA_EHIP;
  return PA_OK;
}

pa_status pa_multi_query(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens,
                         const int32_t* query_start, int32_t B, int32_t Tq, int32_t max_q,
                         int32_t Hq, int32_t Hkv, int32_t D, int32_t bs, int32_t NB, int32_t MB,
                         int32_t max_ctx, float scale, int32_t partition, void* workspace,
                         size_t workspace_bytes, uint32_t flags, pa_dtype dt,
                         hipStream_t stream) {
  if (B > 0 && Tq > 0 && !query_start) return PA_EINVAL;
  return attention(out, q, k_cache, v_cache, block_tables, context_lens, query_start, B, Tq,
                   max_q, Hq, Hkv, D, bs, NB, MB, max_ctx, scale, partition, workspace,
                   workspace_bytes, flags, dt, stream);
}

}  // extern "C"
