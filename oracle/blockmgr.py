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
        if self._blocks_needed(sid, n) > len(self.free):
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
