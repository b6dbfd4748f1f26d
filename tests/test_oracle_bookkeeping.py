"""Pins for the bookkeeping and cache-op oracles (CPU only).

The block manager is checked against invariants the pages fix (a table per
sequence, blocks taken only when needed, shared blocks copied before a write)
and against a content model: whatever sequence of appends, forks and frees,
reading a live sequence's tokens back through its table after applying the
copy pairs and the writes gives exactly the tokens that sequence was given.
"""

import json
import os

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle import blockmgr, cache_ops

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")


def check_invariants(bm):
    NB, bs = bm.num_blocks, bm.block_size
    counts = np.zeros(NB, np.int64)
    for sid, table in bm.tables.items():
        L = bm.lens[sid]
        assert len(table) == -(-L // bs)              # blocks only as needed
        for b in table:
            counts[b] += 1
    assert np.array_equal(counts, np.asarray(bm.ref))  # ref = number of holders
    free = set(bm.free)
    assert len(free) == len(bm.free)                   # no duplicates
    for b in range(NB):
        assert (b in free) == (bm.ref[b] == 0)          # free <=> unreferenced
    assert len(bm.free) + sum(1 for r in bm.ref if r > 0) == NB


ops = st.lists(st.tuples(st.sampled_from(["add", "append", "fork", "free"]),
                         st.integers(0, 10**6), st.integers(1, 40)), max_size=60)


@settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(ops=ops, seed=st.integers(0, 2**31 - 1))
def test_block_manager_invariants_and_content(ops, seed):
    rng = np.random.default_rng(seed)
    NB, bs = 48, 16
    bm = blockmgr.BlockManager(NB, bs, rng.permutation(NB))
    pool = np.full(NB * bs, -1, np.int64)   # physical slot -> token id
    logical = {}                            # sid -> list of token ids
    next_token = 0
    for op, pick, n in ops:
        live = sorted(bm.tables)
        if op == "add" or not live:
            sid = bm.add_seq()
            logical[sid] = []
            continue
        sid = live[pick % len(live)]
        if op == "append":
            try:
                slots, pairs = bm.append(sid, n)
            except blockmgr.OutOfBlocks:
                check_invariants(bm)
                continue
            for src, dst in pairs:                    # copy before writing
                pool[dst * bs:(dst + 1) * bs] = pool[src * bs:(src + 1) * bs]
            for slot in slots:
                pool[slot] = next_token
                logical[sid].append(next_token)
                next_token += 1
            assert len(pairs) <= 1
        elif op == "fork":
            child = bm.fork(sid)
            logical[child] = list(logical[sid])
        elif op == "free":
            bm.free_seq(sid)
            del logical[sid]
        check_invariants(bm)
        for s, toks in logical.items():
            table = bm.block_table(s)
            seen = [pool[table[p // bs] * bs + p % bs] for p in range(len(toks))]
            assert seen == toks


def test_append_failure_changes_nothing():
    bm = blockmgr.BlockManager(4, 16)
    a = bm.add_seq()
    bm.append(a, 40)  # 3 blocks
    before = (list(bm.free), list(bm.ref), bm.block_table(a), bm.seq_len(a))
    with pytest.raises(blockmgr.OutOfBlocks):
        bm.append(a, 40)  # would need 3 more
    assert before == (list(bm.free), list(bm.ref), bm.block_table(a), bm.seq_len(a))


def test_cow_copies_until_last_holder():
    """Eight samples share a partly filled prompt block: seven writers copy it,
    the eighth writes in place (reading of the copy-on-write section)."""
    bm = blockmgr.BlockManager(80, 16)
    parent = bm.add_seq()
    bm.append(parent, 1024 - 5)
    group = [parent] + [bm.fork(parent) for _ in range(7)]
    last_block = bm.block_table(parent)[-1]
    assert bm.refcount(last_block) == 8
    n_pairs = 0
    for sid in group:
        _, pairs = bm.append(sid, 1)
        n_pairs += len(pairs)
        for src, _ in pairs:
            assert src == last_block
    assert n_pairs == 7
    assert bm.refcount(last_block) == 1
    assert all(bm.refcount(b) == 8 for b in bm.block_table(parent)[:-1])


def test_free_returns_blocks_to_front():
    bm = blockmgr.BlockManager(8, 16, [3, 1, 4, 0, 5, 2, 6, 7])
    a = bm.add_seq()
    bm.append(a, 33)  # blocks 3, 1, 4
    assert bm.block_table(a) == [3, 1, 4]
    bm.free_seq(a)
    assert list(bm.free)[:3] == [4, 1, 3]
    b = bm.add_seq()
    bm.append(b, 1)
    assert bm.block_table(b) == [4]


def test_page_example_internal_fragmentation():
    """The pages' 2048-token reservation that stops at 150 tokens leaves 1898
    slots idle; with 16-token blocks taken on demand the same request holds 10
    blocks and leaves 10 slots idle."""
    facts = json.load(open(GOLDEN))
    ex = facts["internal_fragmentation_example"]
    bs = facts["block_size"]["value"]
    assert ex["reserved_tokens"] - ex["used_tokens"] == ex["idle_slots_contiguous"]
    bm = blockmgr.BlockManager(200, bs)
    s = bm.add_seq()
    bm.append(s, ex["used_tokens"])
    blocks = len(bm.block_table(s))
    assert blocks == ex["derived_paged"]["blocks"]
    assert blocks * bs == ex["derived_paged"]["slots"]
    assert blocks * bs - ex["used_tokens"] == ex["derived_paged"]["idle_slots"]


def test_page_example_token_501_lookback():
    """Producing token 501 attends over 500 cached positions: after the step's
    append the sequence holds 500 tokens and the new slot is position 499."""
    facts = json.load(open(GOLDEN))
    ex = facts["decode_lookback"]
    bm = blockmgr.BlockManager(64, facts["block_size"]["value"])
    s = bm.add_seq()
    bm.append(s, ex["tokens_attended"] - 1)
    slots, _ = bm.append(s, 1)
    assert bm.seq_len(s) == ex["tokens_attended"] == ex["generating_token"] - 1
    table = bm.block_table(s)
    assert slots[0] == table[499 // 16] * 16 + 499 % 16


# ------------------------------------------------------------ cache ops
def test_slot_mapping_agrees_with_block_manager():
    rng = np.random.default_rng(3)
    bm = blockmgr.BlockManager(100, 16, rng.permutation(100))
    seqs = [bm.add_seq() for _ in range(6)]
    want = []
    for s in seqs:
        bm.append(s, int(rng.integers(0, 70)))
    for s in seqs:
        want += bm.append(s, 1)[0]
    bt = np.asarray(bm.tables_array(seqs, 8), np.int32)
    pos = np.asarray([bm.seq_len(s) - 1 for s in seqs], np.int32)
    got = cache_ops.slot_mapping(bt, pos, 16)
    assert got.tolist() == want
    pos[2] = -1
    assert cache_ops.slot_mapping(bt, pos, 16)[2] == -1


def test_slot_mapping_entries_without_a_slot():
    # A table entry names a physical block only when it is >= 0 and its
    # slots fit int32 slot numbers; a position must lie inside the table.
    big = (2**31 - 1 - 15) // 16          # 134217727: slots up to 2^31 - 1
    bt = np.array([[5, -1, 7], [2, 3, 2**28 + 1], [big, big + 1, 0]], np.int32)
    pos = [0, 17, 47, 48, -1, 33, 15, 16, 31, 3]
    seq = [0, 0, 0, 0, 1, 1, 2, 2, 2, 3]
    got = cache_ops.slot_mapping(bt, pos, 16, seq_ids=seq).tolist()
    assert got == [80, -1, 7 * 16 + 15, -1, -1, -1, 2**31 - 1, -1, -1, -1]
    # seq_ids default to the token index
    assert cache_ops.slot_mapping(bt, [1, 20], 16).tolist() == [81, 3 * 16 + 4]


@pytest.mark.parametrize("dt", [np.uint16, np.uint32])
def test_write_kv_touches_only_its_slots(dt):
    rng = np.random.default_rng(5)
    NB, Hkv, bs, D, T = 10, 3, 16, 8, 7
    info = np.iinfo(dt)
    kp = rng.integers(0, info.max, (NB, Hkv, bs, D), dtype=dt, endpoint=True)
    vp = rng.integers(0, info.max, (NB, Hkv, bs, D), dtype=dt, endpoint=True)
    kn = rng.integers(0, info.max, (T, Hkv, D), dtype=dt, endpoint=True)
    vn = rng.integers(0, info.max, (T, Hkv, D), dtype=dt, endpoint=True)
    # NaN payloads and denormals survive as raw bits
    if dt == np.uint16:
        kn[0, 0, :2] = [0x7FC1, 0x0001]
    else:
        kn[0, 0, :2] = [0x7FC00001, 0x00000001]
    slots = rng.choice(NB * bs, T, replace=False).astype(np.int32)
    slots[3] = -1
    k2, v2 = kp.copy(), vp.copy()
    cache_ops.write_kv(k2, v2, kn, vn, slots)
    flat_k = k2.transpose(0, 2, 1, 3).reshape(NB * bs, Hkv, D)  # slot-major view
    flat_k0 = kp.transpose(0, 2, 1, 3).reshape(NB * bs, Hkv, D)
    flat_v = v2.transpose(0, 2, 1, 3).reshape(NB * bs, Hkv, D)
    changed = set()
    for i, s in enumerate(slots):
        if s < 0:
            continue
        changed.add(int(s))
        assert np.array_equal(flat_k[s], kn[i]) and np.array_equal(flat_v[s], vn[i])
    for s in range(NB * bs):
        if s not in changed:
            assert np.array_equal(flat_k[s], flat_k0[s])


def test_copy_blocks_copies_whole_blocks_only():
    rng = np.random.default_rng(6)
    NB, Hkv, bs, D = 12, 2, 16, 4
    kp = rng.integers(0, 2**16, (NB, Hkv, bs, D), dtype=np.uint16)
    vp = rng.integers(0, 2**16, (NB, Hkv, bs, D), dtype=np.uint16)
    pairs = np.array([[1, 7], [1, 8], [4, 2]], np.int32)
    k2, v2 = kp.copy(), vp.copy()
    cache_ops.copy_blocks(k2, v2, pairs)
    for src, dst in pairs:
        assert np.array_equal(k2[dst], kp[src]) and np.array_equal(v2[dst], vp[src])
    untouched = [b for b in range(NB) if b not in pairs[:, 1]]
    assert np.array_equal(k2[untouched], kp[untouched])
    assert np.array_equal(v2[untouched], vp[untouched])
