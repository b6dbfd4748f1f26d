"""KV block bookkeeping oracle: free list, block tables, reference counts, COW.

TEST INFRASTRUCTURE ONLY: the reference against which the native block
manager of the GPU library is checked, and the builder of the block tables
the decode oracle reads. It shares no code with the library.

Follows:
  * "Why OS Virtual Memory Paging Saved LLM Inference" (a8q9.cn), section
    "2. The PagedAttention Architecture": fixed-size physical blocks; a
    per-request table from logical positions to physical blocks, as a page
    table; physical blocks are taken one at a time, only when a new token
    needs one.
  * Same page, section "3. Copy-on-Write for Prompt Sharing": branches of a
    parallel-sampling or beam-search request point at the same physical
    prompt blocks; a branch that writes a new token into a shared block first
    gets a private block of its own.
  * "Can OS paging techniques reduce LLM serving memory waste?"
    (inquiringlines.com), mechanism paragraph: a KV cache manager keeps one
    block table per request and lets requests share blocks.

Readings where the pages are silent (each listed in the design notes):
  * Sharing is tracked with a per-block reference count (the pages describe
    the sharing, not the mechanism). A write into a block whose count is
    above one copies it (count of the old block drops by one); the last
    holder writes in place, as an OS copy-on-write page does.
  * The free list is a deque: allocation pops the front; a block whose count
    reaches zero is pushed back onto the front. The initial order is given
    (a seeded permutation in the workloads), so which physical block a
    sequence receives is deterministic and the native manager can be checked
    against this one entry by entry.
  * Slot of logical position p of a sequence: table[p // bs] * bs + p % bs.
  * An append that cannot be satisfied raises before changing any state.
"""

from collections import deque


class OutOfBlocks(RuntimeError):
    """The free list cannot supply the blocks an operation needs."""


class BlockManager:
    """Per-sequence block tables over a pool of `num_blocks` physical blocks."""

    def __init__(self, num_blocks, block_size=16, free_order=None):
        if num_blocks < 0 or block_size <= 0:
            raise ValueError("bad pool size")
        if free_order is None:
            free_order = range(num_blocks)
        free_order = [int(b) for b in free_order]
        if sorted(free_order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of range(num_blocks)")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = deque(free_order)
        self.ref = [0] * num_blocks
        self.tables = {}
        self.lens = {}
        self._next_id = 0

    # -- allocation -------------------------------------------------------
    def _alloc(self):
        b = self.free.popleft()
        self.ref[b] = 1
        return b

    def add_seq(self):
        sid = self._next_id
        self._next_id += 1
        self.tables[sid] = []
        self.lens[sid] = 0
        return sid

    def _blocks_needed(self, sid, n):
        """Fresh blocks an append of n tokens takes (COW copy included)."""
        p = self.lens[sid]
        bs = self.block_size
        table = self.tables[sid]
        need = 0
        if n > 0 and p % bs != 0 and self.ref[table[p // bs]] > 1:
            need += 1  # the shared, partly filled last block gets copied
        # blocks that start inside [p, p + n): logical block indices
        first_new = (p + bs - 1) // bs
        last_needed = (p + n + bs - 1) // bs
        need += max(0, last_needed - first_new)
        return need

    def append(self, sid, n=1):
        """Append n tokens to sequence sid.

        Returns (slots, pairs): the physical slot of each new token, and the
        (src, dst) block copies the caller must perform before writing them.
        """
        if n < 0:
            raise ValueError("n must be >= 0")
        if self._blocks_needed(sid, n) > self.num_free():
            raise OutOfBlocks(f"sequence {sid}: {n} tokens need more blocks than are free")
        bs = self.block_size
        table = self.tables[sid]
        slots, pairs = [], []
        for _ in range(n):
            p = self.lens[sid]
            if p % bs == 0:
                table.append(self._alloc())
            else:
                b = table[p // bs]
                if self.ref[b] > 1:
                    nb = self._alloc()
                    pairs.append((b, nb))
                    self.ref[b] -= 1
                    table[p // bs] = nb
            slots.append(table[p // bs] * bs + p % bs)
            self.lens[sid] = p + 1
        return slots, pairs

    def fork(self, parent):
        """A new sequence sharing every block of `parent` (counts go up)."""
        child = self.add_seq()
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1
        return child

    def free_seq(self, sid):
        """Drop sequence sid; blocks no one else holds go back to the free list."""
        for b in self.tables.pop(sid):
            if self.ref[b] <= 0:
                raise RuntimeError(f"block {b} freed with reference count {self.ref[b]}")
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.appendleft(b)
        del self.lens[sid]

    # -- views ------------------------------------------------------------
    def num_free(self):
        return len(self.free)

    def block_table(self, sid):
        return list(self.tables[sid])

    def seq_len(self, sid):
        return self.lens[sid]

    def refcount(self, b):
        return self.ref[b]

    def tables_array(self, sids, max_blocks):
        """int32-compatible nested lists [len(sids)][max_blocks], unused = -1."""
        out = []
        for sid in sids:
            t = self.tables[sid]
            if len(t) > max_blocks:
                raise ValueError("table longer than max_blocks")
            out.append(t + [-1] * (max_blocks - len(t)))
        return out


class PrefixBlockManager(BlockManager):
    """Block manager with beam re-forks and cross-request prefix sharing.

    Follows, beyond the base class:
      * "Why OS Virtual Memory Paging Saved LLM Inference" (a8q9.cn), section
        3: beam-search branches share physical prompt blocks; here a pruned
        beam is re-pointed at a surviving beam's blocks (fork_into).
      * "Can OS paging techniques reduce LLM serving memory waste?"
        (inquiringlines.com), mechanism paragraph: requests share KV blocks
        within and across a batch; "vLLM & PagedAttention"
        (completesystemdesign.dev), introduction: prefix caching.

    Readings where the pages are silent (each listed in the design notes):
      * A block is shareable across requests once it is full and its content
        is known: it is registered under the key (content id of the previous
        block of its sequence, or 0 at the start; its block_size token ids).
        Every registration gets a fresh content id, never reissued, so the
        key pins the whole prefix exactly (no hashing, no collisions) and an
        evicted block's descendants become unreachable.
      * A new request reuses the longest registered prefix of its prompt's
        full blocks, but always leaves at least one prompt token to process
        (the model needs that token's query to continue).
      * A registered block whose last holder leaves is not freed but kept,
        evictable, in least-recently-released order. Allocation takes the
        free list first, then evicts the oldest kept block (dropping its
        registration). Reusing a kept block takes it out of that order.
      * A block that fills with content already registered under another
        block stays private; the sequence continues the registered chain.
    """

    def __init__(self, num_blocks, block_size=16, free_order=None):
        super().__init__(num_blocks, block_size, free_order)
        self.cached = {}                 # key -> block
        self.key_of = {}                 # block -> key (registered blocks)
        self.cid = {}                    # block -> content id (registered blocks)
        self._next_cid = 1
        self.evictable = deque()         # registered blocks nobody holds, oldest first
        self.chain = {}                  # seq -> content id of its last full block, or None
        self.partial = {}                # seq -> token ids in its partly filled last block

    # -- allocation -------------------------------------------------------
    def num_free(self):
        return len(self.free) + len(self.evictable)

    def _alloc(self):
        if self.free:
            b = self.free.popleft()
        else:
            b = self.evictable.popleft()
            del self.cached[self.key_of.pop(b)]
            del self.cid[b]
        self.ref[b] = 1
        return b

    def _release(self, b):
        if self.ref[b] <= 0:
            raise RuntimeError(f"block {b} freed with reference count {self.ref[b]}")
        self.ref[b] -= 1
        if self.ref[b] == 0:
            if b in self.key_of:
                self.evictable.append(b)
            else:
                self.free.appendleft(b)

    def _hold(self, b):
        if self.ref[b] == 0:
            self.evictable.remove(b)
        self.ref[b] += 1

    # -- sequences --------------------------------------------------------
    def add_seq(self):
        sid = super().add_seq()
        self.chain[sid] = 0
        self.partial[sid] = []
        return sid

    def add_seq_cached(self, tokens):
        """A new sequence whose first blocks are the registered prefix of
        `tokens` (at most (len(tokens) - 1) // block_size of them). Returns
        (seq, n_cached): the prompt's first n_cached tokens are already in the
        cache; append_tokens(seq, tokens[n_cached:]) continues it."""
        sid = self.add_seq()
        bs = self.block_size
        parent = 0
        for i in range((len(tokens) - 1) // bs if len(tokens) else 0):
            key = (parent, tuple(int(t) for t in tokens[i * bs:(i + 1) * bs]))
            b = self.cached.get(key)
            if b is None:
                break
            self._hold(b)
            self.tables[sid].append(b)
            self.lens[sid] += bs
            parent = self.cid[b]
        self.chain[sid] = parent
        return sid, self.lens[sid]

    def fork(self, parent):
        child = super().fork(parent)
        self.chain[child] = self.chain[parent]
        self.partial[child] = list(self.partial[parent])
        return child

    def fork_into(self, dst, src):
        """Beam re-fork: sequence dst drops its blocks and shares src's."""
        for b in self.tables[src]:
            self._hold(b)
        old = self.tables[dst]
        self.tables[dst] = list(self.tables[src])
        self.lens[dst] = self.lens[src]
        self.chain[dst] = self.chain[src]
        self.partial[dst] = list(self.partial[src])
        for b in old:
            self._release(b)

    def free_seq(self, sid):
        for b in self.tables.pop(sid):
            self._release(b)
        del self.lens[sid]
        del self.chain[sid]
        del self.partial[sid]

    def append(self, sid, n=1):
        """Append n tokens of unknown content: the sequence's later blocks
        cannot be registered."""
        out = super().append(sid, n)
        if n > 0:
            self.chain[sid] = None
            self.partial[sid] = []
        return out

    def append_tokens(self, sid, tokens):
        """Append tokens with known ids; every block they fill is registered."""
        bs = self.block_size
        slots, pairs = BlockManager.append(self, sid, len(tokens))
        start = self.lens[sid] - len(tokens)
        for i, t in enumerate(tokens):
            p = start + i
            if self.chain[sid] is None:
                continue
            self.partial[sid].append(int(t))
            if p % bs == bs - 1:                   # the token fills its block
                b = self.tables[sid][p // bs]
                key = (self.chain[sid], tuple(self.partial[sid]))
                self.partial[sid] = []
                hit = self.cached.get(key)
                if hit is not None:
                    self.chain[sid] = self.cid[hit]
                else:
                    c = self._next_cid
                    self._next_cid += 1
                    self.cached[key] = b
                    self.key_of[b] = key
                    self.cid[b] = c
                    self.chain[sid] = c
        return slots, pairs

    def num_cached(self):
        """Registered blocks that no sequence holds (kept, evictable)."""
        return len(self.evictable)
