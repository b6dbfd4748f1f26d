// Host-side KV block bookkeeping: free list, per-sequence block tables,
// reference counts and copy-on-write.
//
// Method: "Why OS Virtual Memory Paging Saved LLM Inference" (a8q9.cn),
// section 2 (a block table per sequence, as a page table; physical blocks
// taken one at a time, only when a token needs one) and section 3 (branches
// share physical prompt blocks; a branch about to write into a shared block
// gets a private block first). "Can OS paging techniques reduce LLM serving
// memory waste?" (inquiringlines.com), mechanism paragraph (a manager keeps
// the per-request tables; requests may share blocks).
//
// Sharing is tracked with per-block reference counts. The free list is a
// deque: blocks are taken from its front and freed blocks return to its
// front. An append that cannot be satisfied changes nothing.
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"

struct pa_block_manager {
  int32_t num_blocks = 0;
  int32_t block_size = 16;
  std::deque<int32_t> free_list;
  std::vector<int32_t> ref;
  struct Seq {
    std::vector<int32_t> table;
    int32_t len = 0;
  };
  std::unordered_map<int32_t, Seq> seqs;
  int32_t next_id = 0;

  int32_t alloc() {
    const int32_t b = free_list.front();
    free_list.pop_front();
    ref[b] = 1;
    return b;
  }

  // Fresh blocks an append of n tokens to `sq` takes, the copy included.
  int64_t blocks_needed(const Seq& sq, int32_t n) const {
    const int64_t p = sq.len, bs = block_size;
    int64_t need = 0;
    if (n > 0 && p % bs != 0 && ref[sq.table[p / bs]] > 1) need += 1;
    const int64_t first_new = (p + bs - 1) / bs;
    const int64_t last_needed = (p + n + bs - 1) / bs;
    if (last_needed > first_new) need += last_needed - first_new;
    return need;
  }
};

namespace {
pa_block_manager::Seq* find(pa_block_manager* bm, int32_t seq) {
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? nullptr : &it->second;
}
const pa_block_manager::Seq* find(const pa_block_manager* bm, int32_t seq) {
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? nullptr : &it->second;
}
}  // namespace

extern "C" {

pa_status pa_bm_create(pa_block_manager** out, int32_t num_blocks, int32_t block_size,
                       const int32_t* free_order) {
  if (!out || num_blocks < 0 || block_size <= 0) return PA_EINVAL;
  *out = nullptr;
  pa_block_manager* bm = new (std::nothrow) pa_block_manager();
  if (!bm) return PA_EINVAL;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->ref.assign(num_blocks, 0);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete bm;
        return PA_EINVAL;  // not a permutation
      }
      seen[b] = 1;
      bm->free_list.push_back(b);
    }
  } else {
    for (int32_t b = 0; b < num_blocks; ++b) bm->free_list.push_back(b);
  }
  *out = bm;
  return PA_OK;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

pa_status pa_bm_add_seq(pa_block_manager* bm, int32_t* seq) {
  if (!bm || !seq) return PA_EINVAL;
  const int32_t id = bm->next_id++;
  bm->seqs[id] = pa_block_manager::Seq{};
  *seq = id;
  return PA_OK;
}

pa_status pa_bm_fork(pa_block_manager* bm, int32_t parent, int32_t* child) {
  if (!bm || !child) return PA_EINVAL;
  const auto* par = find(bm, parent);
  if (!par) return PA_EINVAL;
  pa_block_manager::Seq copy = *par;
  for (int32_t b : copy.table) bm->ref[b] += 1;
  const int32_t id = bm->next_id++;
  bm->seqs[id] = std::move(copy);
  *child = id;
  return PA_OK;
}

pa_status pa_bm_append(pa_block_manager* bm, int32_t seq, int32_t n, int32_t* slots,
                       int32_t* pair, int32_t* n_pairs) {
  if (!bm || n < 0 || (n > 0 && !slots) || !pair || !n_pairs) return PA_EINVAL;
  auto* sq = find(bm, seq);
  if (!sq) return PA_EINVAL;
  if ((int64_t)sq->len + n > INT32_MAX) return PA_EINVAL;
  if (bm->blocks_needed(*sq, n) > (int64_t)bm->free_list.size()) return PA_ENOBLOCKS;
  const int32_t bs = bm->block_size;
  *n_pairs = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t p = sq->len;
    if (p % bs == 0) {
      sq->table.push_back(bm->alloc());
    } else {
      int32_t& b = sq->table[p / bs];
      if (bm->ref[b] > 1) {
        const int32_t nb = bm->alloc();
        pair[0] = b;
        pair[1] = nb;
        *n_pairs = 1;
        bm->ref[b] -= 1;
        b = nb;
      }
    }
    slots[i] = sq->table[p / bs] * bs + p % bs;
    sq->len = p + 1;
  }
  return PA_OK;
}

pa_status pa_bm_free_seq(pa_block_manager* bm, int32_t seq) {
  if (!bm) return PA_EINVAL;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_EINVAL;
  for (int32_t b : it->second.table) {
    bm->ref[b] -= 1;
    if (bm->ref[b] == 0) bm->free_list.push_front(b);
  }
  bm->seqs.erase(it);
  return PA_OK;
}

pa_status pa_bm_seq_len(const pa_block_manager* bm, int32_t seq, int32_t* len) {
  if (!bm || !len) return PA_EINVAL;
  const auto* sq = find(bm, seq);
  if (!sq) return PA_EINVAL;
  *len = sq->len;
  return PA_OK;
}

pa_status pa_bm_num_free(const pa_block_manager* bm, int32_t* n) {
  if (!bm || !n) return PA_EINVAL;
  *n = (int32_t)bm->free_list.size();
  return PA_OK;
}

pa_status pa_bm_refcount(const pa_block_manager* bm, int32_t block, int32_t* r) {
  if (!bm || !r || block < 0 || block >= bm->num_blocks) return PA_EINVAL;
  *r = bm->ref[block];
  return PA_OK;
}

pa_status pa_bm_block_table(const pa_block_manager* bm, int32_t seq, int32_t* out, int32_t cap,
                            int32_t* n) {
  if (!bm || !n || cap < 0 || (cap > 0 && !out)) return PA_EINVAL;
  const auto* sq = find(bm, seq);
  if (!sq) return PA_EINVAL;
  const int32_t len = (int32_t)sq->table.size();
  for (int32_t i = 0; i < len && i < cap; ++i) out[i] = sq->table[i];
  *n = len;
  return PA_OK;
}

pa_status pa_bm_fill_tables(const pa_block_manager* bm, const int32_t* seqs, int32_t n_seqs,
                            int32_t MB, int32_t* tables, int32_t* lens) {
  if (!bm || n_seqs < 0 || MB < 0 || (n_seqs > 0 && (!seqs || !tables || !lens))) return PA_EINVAL;
  for (int32_t i = 0; i < n_seqs; ++i) {
    const auto* sq = find(bm, seqs[i]);
    if (!sq || (int64_t)sq->table.size() > MB) return PA_EINVAL;
  }
  for (int32_t i = 0; i < n_seqs; ++i) {
    const auto* sq = find(bm, seqs[i]);
    int32_t* row = tables + (size_t)i * MB;
    const int32_t len = (int32_t)sq->table.size();
    for (int32_t j = 0; j < MB; ++j) row[j] = j < len ? sq->table[j] : -1;
    lens[i] = sq->len;
  }
  return PA_OK;
}

}  // extern "C"
