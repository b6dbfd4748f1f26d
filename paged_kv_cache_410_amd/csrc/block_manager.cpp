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
//
// Beam re-forks (a8q9.cn section 3: beam-search branches share prompt
// blocks): pa_bm_fork_into re-points a pruned beam at a surviving beam's
// blocks. Sharing across requests (inquiringlines.com mechanism paragraph;
// prefix caching in the completesystemdesign.dev introduction): a full block
// whose tokens are known (pa_bm_append_tokens) is registered under the key
// (content id of the sequence's previous block, or 0; its token ids). Each
// registration gets a fresh content id that is never reissued, so a key names
// the whole prefix exactly, and an evicted block's descendants can no longer
// be matched. pa_bm_add_seq_cached reuses the longest registered prefix of a
// prompt's full blocks, leaving at least one prompt token to process. A
// registered block released by its last holder is kept, evictable, in
// release order; allocation takes the free list first, then evicts the
// oldest kept block. A block that fills with content already registered
// elsewhere stays private and the sequence follows the registered chain.
#include <algorithm>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"

namespace {

// Registration key: previous block's content id + the block's token ids.
struct Key {
  int64_t parent = 0;
  std::vector<int32_t> tokens;
  bool operator==(const Key& o) const { return parent == o.parent && tokens == o.tokens; }
};
// FNV-1a (Fowler-Noll-Vo, 64-bit) over the key's integers; equality is exact.
struct KeyHash {
  size_t operator()(const Key& k) const {
    uint64_t h = 14695981039346656037ull;
    auto mix = [&h](uint64_t v) {
      for (int i = 0; i < 8; ++i) {
        h ^= (v >> (8 * i)) & 0xffu;
        h *= 1099511628211ull;
      }
    };
    mix((uint64_t)k.parent);
    for (int32_t t : k.tokens) mix((uint64_t)(uint32_t)t);
    return (size_t)h;
  }
};

}  // namespace

struct pa_block_manager {
  int32_t num_blocks = 0;
  int32_t block_size = 16;
  std::deque<int32_t> free_list;
  std::deque<int32_t> kept;            // registered, unheld blocks, oldest release first
  std::vector<int32_t> ref;
  std::vector<int64_t> cid;            // content id of a registered block, 0 otherwise
  std::vector<Key> key_of;             // key of a registered block
  std::unordered_map<Key, int32_t, KeyHash> cached;
  int64_t next_cid = 1;
  struct Seq {
    std::vector<int32_t> table;
    int32_t len = 0;
    int64_t chain = 0;                 // content id of its last full block; -1: unknown content
    std::vector<int32_t> partial;      // token ids in its partly filled last block
  };
  std::unordered_map<int32_t, Seq> seqs;
  int32_t next_id = 0;

  int64_t allocatable() const { return (int64_t)free_list.size() + (int64_t)kept.size(); }

  int32_t alloc() {
    int32_t b;
    if (!free_list.empty()) {
      b = free_list.front();
      free_list.pop_front();
    } else {
      b = kept.front();
      kept.pop_front();
      cached.erase(key_of[b]);
      key_of[b] = Key{};
      cid[b] = 0;
    }
    ref[b] = 1;
    return b;
  }

  void release(int32_t b) {
    ref[b] -= 1;
    if (ref[b] == 0) {
      if (cid[b] != 0)
        kept.push_back(b);
      else
        free_list.push_front(b);
    }
  }

  void hold(int32_t b) {
    if (ref[b] == 0) kept.erase(std::find(kept.begin(), kept.end(), b));
    ref[b] += 1;
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

  // Append n tokens; `tokens` (may be null: content unknown) registers every
  // block they fill. The caller has checked capacity.
  void append(Seq& sq, int32_t n, const int32_t* tokens, int32_t* slots, int32_t* pair,
              int32_t* n_pairs) {
    const int32_t bs = block_size;
    *n_pairs = 0;
    if (n > 0 && !tokens) {
      sq.chain = -1;
      sq.partial.clear();
    }
    for (int32_t i = 0; i < n; ++i) {
      const int32_t p = sq.len;
      if (p % bs == 0) {
        sq.table.push_back(alloc());
      } else {
        int32_t& b = sq.table[p / bs];
        if (ref[b] > 1) {
          const int32_t nb = alloc();
          pair[0] = b;
          pair[1] = nb;
          *n_pairs = 1;
          ref[b] -= 1;
          b = nb;
        }
      }
      slots[i] = sq.table[p / bs] * bs + p % bs;
      sq.len = p + 1;
      if (tokens && sq.chain >= 0) {
        sq.partial.push_back(tokens[i]);
        if (p % bs == bs - 1) register_full(sq, sq.table[p / bs]);
      }
    }
  }

  void register_full(Seq& sq, int32_t b) {
    Key k{sq.chain, std::move(sq.partial)};
    sq.partial.clear();
    auto it = cached.find(k);
    if (it != cached.end()) {
      sq.chain = cid[it->second];
      return;
    }
    const int64_t c = next_cid++;
    cid[b] = c;
    key_of[b] = k;
    cached.emplace(std::move(k), b);
    sq.chain = c;
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
  bm->cid.assign(num_blocks, 0);
  bm->key_of.assign(num_blocks, Key{});
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
  if (bm->blocks_needed(*sq, n) > bm->allocatable()) return PA_ENOBLOCKS;
  bm->append(*sq, n, nullptr, slots, pair, n_pairs);
  return PA_OK;
}

pa_status pa_bm_append_tokens(pa_block_manager* bm, int32_t seq, const int32_t* tokens, int32_t n,
                              int32_t* slots, int32_t* pair, int32_t* n_pairs) {
  if (!bm || n < 0 || (n > 0 && (!slots || !tokens)) || !pair || !n_pairs) return PA_EINVAL;
  auto* sq = find(bm, seq);
  if (!sq) return PA_EINVAL;
  if ((int64_t)sq->len + n > INT32_MAX) return PA_EINVAL;
  if (bm->blocks_needed(*sq, n) > bm->allocatable()) return PA_ENOBLOCKS;
  bm->append(*sq, n, tokens, slots, pair, n_pairs);
  return PA_OK;
}

pa_status pa_bm_add_seq_cached(pa_block_manager* bm, const int32_t* tokens, int32_t n,
                               int32_t* seq, int32_t* n_cached) {
  if (!bm || n < 0 || (n > 0 && !tokens) || !seq || !n_cached) return PA_EINVAL;
  const int32_t bs = bm->block_size;
  pa_block_manager::Seq sq;
  const int32_t full = n > 0 ? (n - 1) / bs : 0;
  Key k;
  for (int32_t i = 0; i < full; ++i) {
    k.parent = sq.chain;
    k.tokens.assign(tokens + (size_t)i * bs, tokens + (size_t)(i + 1) * bs);
    auto it = bm->cached.find(k);
    if (it == bm->cached.end()) break;
    const int32_t b = it->second;
    bm->hold(b);
    sq.table.push_back(b);
    sq.len += bs;
    sq.chain = bm->cid[b];
  }
  const int32_t id = bm->next_id++;
  *n_cached = sq.len;
  bm->seqs[id] = std::move(sq);
  *seq = id;
  return PA_OK;
}

pa_status pa_bm_fork_into(pa_block_manager* bm, int32_t dst, int32_t src) {
  if (!bm) return PA_EINVAL;
  auto* d = find(bm, dst);
  const auto* sr = find(bm, src);
  if (!d || !sr) return PA_EINVAL;
  pa_block_manager::Seq next = *sr;  // copied first: dst may be src
  for (int32_t b : next.table) bm->hold(b);
  std::vector<int32_t> old = std::move(d->table);
  *d = std::move(next);
  for (int32_t b : old) bm->release(b);
  return PA_OK;
}

pa_status pa_bm_free_seq(pa_block_manager* bm, int32_t seq) {
  if (!bm) return PA_EINVAL;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_EINVAL;
  for (int32_t b : it->second.table) bm->release(b);
  bm->seqs.erase(it);
  return PA_OK;
}

pa_status pa_bm_num_cached(const pa_block_manager* bm, int32_t* n) {
  if (!bm || !n) return PA_EINVAL;
  *n = (int32_t)bm->kept.size();
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
  *n = (int32_t)bm->allocatable();
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

pa_status pa_shared_groups(const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                           int32_t MB, int32_t bs, int32_t max_group, int32_t* group_start,
                           int32_t* seq_shared, int32_t* n_groups) {
  if (B < 0 || MB < 0 || bs <= 0 || max_group < 1 || !n_groups ||
      (B > 0 && (!context_lens || !group_start || !seq_shared || (MB > 0 && !block_tables))))
    return PA_EINVAL;
  *n_groups = 0;
  if (B == 0) return PA_OK;
  int32_t ng = 0;
  group_start[0] = 0;
  for (int32_t s = 0; s < B;) {
    const int32_t* first = block_tables + (size_t)s * MB;
    // whole blocks inside the first member's context, with valid ids
    int32_t k = context_lens[s] > 0 ? context_lens[s] / bs : 0;
    if (k > MB) k = MB;
    for (int32_t j = 0; j < k; ++j)
      if (first[j] < 0) {
        k = j;
        break;
      }
    int32_t e = s + 1;
    while (e < B && e - s < max_group && k > 0) {
      const int32_t* row = block_tables + (size_t)e * MB;
      int32_t full = context_lens[e] > 0 ? context_lens[e] / bs : 0;
      int32_t lcp = 0;
      const int32_t lim = k < full ? k : full;
      while (lcp < lim && row[lcp] == first[lcp]) ++lcp;
      if (lcp == 0) break;  // shares nothing with the group: next group
      k = lcp;
      ++e;
    }
    const int32_t shared = e - s > 1 ? k * bs : 0;  // a sequence alone shares nothing
    for (int32_t i = s; i < e; ++i) seq_shared[i] = shared;
    group_start[++ng] = e;
    s = e;
  }
  *n_groups = ng;
  return PA_OK;
}

}  // extern "C"
