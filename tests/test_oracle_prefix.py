"""Pins for the prefix-sharing block manager oracle (oracle.blockmgr.
PrefixBlockManager), CPU only.

What the pages fix: blocks may be shared within and across requests and the
result must not change ("Can OS paging techniques reduce LLM serving memory
waste?", inquiringlines.com, mechanism paragraph); beam-search branches share
prompt blocks and a writer gets a private copy ("Why OS Virtual Memory Paging
Saved LLM Inference", a8q9.cn, section 3); blocks are taken only when needed
(same page, section 2). The checks below follow from those statements, not
from the oracle's own code: a content model (what each physical slot holds)
must reproduce every live sequence's tokens through its table; reference
counts must match table references; registered blocks must hold exactly the
content their key names; and a shared prefix must cost no new blocks.
"""

import itertools

from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle.blockmgr import OutOfBlocks, PrefixBlockManager

BS = 4


class Model:
    """The manager under test plus an independent record of content."""

    def __init__(self, nb):
        self.bm = PrefixBlockManager(nb, BS)
        self.nb = nb
        self.slot = {}          # physical slot -> token id written there
        self.tokens = {}        # seq -> its logical token ids
        self.unknown = itertools.count(-1, -1)

    def _apply(self, sid, toks, slots, pairs):
        for src, dst in pairs:
            for o in range(BS):
                if src * BS + o in self.slot:
                    self.slot[dst * BS + o] = self.slot[src * BS + o]
        for t, s in zip(toks, slots):
            self.slot[s] = t
        self.tokens[sid] = self.tokens[sid] + list(toks)

    def new(self, prompt):
        sid, n = self.bm.add_seq_cached(prompt)
        self.tokens[sid] = list(prompt[:n])
        rest = prompt[n:]
        slots, pairs = self.bm.append_tokens(sid, rest)
        self._apply(sid, rest, slots, pairs)
        return sid, n

    def append_tokens(self, sid, toks):
        slots, pairs = self.bm.append_tokens(sid, toks)
        self._apply(sid, toks, slots, pairs)

    def append_unknown(self, sid, n):
        toks = [next(self.unknown) for _ in range(n)]
        slots, pairs = self.bm.append(sid, n)
        self._apply(sid, toks, slots, pairs)

    def fork(self, sid):
        c = self.bm.fork(sid)
        self.tokens[c] = list(self.tokens[sid])
        return c

    def fork_into(self, dst, src):
        self.bm.fork_into(dst, src)
        self.tokens[dst] = list(self.tokens[src])

    def free(self, sid):
        self.bm.free_seq(sid)
        del self.tokens[sid]

    def check(self):
        bm = self.bm
        refs = [0] * self.nb
        for sid, toks in self.tokens.items():
            table = bm.block_table(sid)
            assert bm.seq_len(sid) == len(toks)
            assert len(table) == -(-len(toks) // BS)
            for p, t in enumerate(toks):
                assert self.slot.get(table[p // BS] * BS + p % BS) == t, (sid, p)
            for b in table:
                refs[b] += 1
        assert refs == [bm.refcount(b) for b in range(self.nb)]
        free, kept = set(bm.free), set(bm.evictable)
        held = {b for b in range(self.nb) if refs[b] > 0}
        assert len(free) == len(bm.free) and len(kept) == len(bm.evictable)
        assert not (free & kept) and not (free & held) and not (kept & held)
        assert free | kept | held == set(range(self.nb))
        assert bm.num_free() == len(free) + len(kept)
        for b in kept:
            assert b in bm.key_of
        # a registered block holds the tokens its key names
        for key, b in bm.cached.items():
            assert bm.key_of[b] == key
            assert [self.slot.get(b * BS + o) for o in range(BS)] == list(key[1])
        assert len(set(bm.cid.values())) == len(bm.cid)


ALPHABET = st.integers(0, 1)           # tiny alphabet: prefixes collide often
ops = st.lists(st.tuples(st.sampled_from(["new", "tok", "unk", "fork", "into", "free"]),
                         st.integers(0, 7), st.integers(0, 7),
                         st.lists(ALPHABET, min_size=0, max_size=11)),
               min_size=1, max_size=40)


@settings(max_examples=400, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(ops=ops, nb=st.integers(6, 24))
def test_prefix_manager_content_and_counts(ops, nb):
    m = Model(nb)
    live = []
    for op, i, j, toks in ops:
        before = (list(m.bm.free), list(m.bm.evictable), dict(m.bm.cached),
                  [m.bm.refcount(b) for b in range(nb)])
        try:
            if op == "new" or not live:
                sid, _ = m.new(toks or [0])
                live.append(sid)
            elif op == "tok":
                m.append_tokens(live[i % len(live)], toks)
            elif op == "unk":
                m.append_unknown(live[i % len(live)], len(toks))
            elif op == "fork":
                live.append(m.fork(live[i % len(live)]))
            elif op == "into":
                m.fork_into(live[i % len(live)], live[j % len(live)])
            elif op == "free":
                m.free(live.pop(i % len(live)))
        except OutOfBlocks:
            if op == "new" or not live:
                # the request's sequence exists, holding whatever cached prefix
                # it revived; dropping it restores the counts and the set of
                # allocatable blocks (their release order may differ)
                for sid in list(m.tokens):
                    if sid not in live:
                        m.free(sid)
                assert [m.bm.refcount(b) for b in range(nb)] == before[3]
                assert set(m.bm.free) | set(m.bm.evictable) == set(before[0]) | set(before[1])
                assert dict(m.bm.cached) == before[2]
            else:
                # a failed append changes nothing at all
                after = (list(m.bm.free), list(m.bm.evictable), dict(m.bm.cached),
                         [m.bm.refcount(b) for b in range(nb)])
                assert after == before
        m.check()


def test_shared_prefix_costs_no_blocks():
    m = Model(40)
    prompt = list(range(11))                       # 2 full blocks + 3 tokens
    a, n = m.new(prompt)
    assert n == 0
    used = 40 - m.bm.num_free()
    b, n = m.new(prompt[:8] + [50, 51])             # shares the 2 full blocks
    assert n == 8
    assert m.bm.block_table(b)[:2] == m.bm.block_table(a)[:2]
    assert 40 - m.bm.num_free() == used + 1          # only its own third block
    c, n = m.new(prompt[:8])                         # whole prompt cached: keep one token
    assert n == 4
    m.check()


def test_kept_blocks_are_reused_then_evicted_oldest_first():
    m = Model(6)
    a, _ = m.new([1, 1, 1, 1, 2, 2, 2, 2, 3])        # blocks: [1111] [2222] [3]
    blocks = m.bm.block_table(a)
    m.free(a)
    assert m.bm.num_cached() == 2 and m.bm.num_free() == 6
    b, n = m.new([1, 1, 1, 1, 2, 2, 2, 2, 7])        # revives both kept blocks
    assert n == 8 and m.bm.block_table(b)[:2] == blocks[:2]
    assert m.bm.num_cached() == 0
    m.free(b)
    # exhaust the free list: the oldest kept block ([1111], released first) goes first
    c, _ = m.new([9] * 16 + [9])
    assert blocks[0] in m.bm.block_table(c) and blocks[1] not in m.bm.block_table(c)
    m.free(c)
    d, n = m.new([1, 1, 1, 1, 2, 2, 2, 2, 5])        # [1111] is gone: no reuse at all
    assert n == 0
    m.check()


def test_beam_refork_shares_and_releases():
    m = Model(30)
    root, _ = m.new(list(range(6)))
    beams = [m.fork(root) for _ in range(3)]
    for k, bsid in enumerate(beams):
        m.append_tokens(bsid, [100 + k])             # each beam diverges in the partial block
    m.free(root)
    m.fork_into(beams[2], beams[0])                  # beam 2 pruned, replaced by beam 0
    assert m.bm.block_table(beams[2]) == m.bm.block_table(beams[0])
    m.append_tokens(beams[2], [7])                   # a writer into a shared block copies it
    assert m.bm.block_table(beams[2])[-1] != m.bm.block_table(beams[0])[-1]
    m.check()
