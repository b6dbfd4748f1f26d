"""Cache-write, block-copy and slot-mapping oracle (raw bit moves, numpy).

TEST INFRASTRUCTURE ONLY; shares no code with the GPU library.

Pools are numpy arrays of shape [num_blocks, num_kv_heads, block_size,
head_dim] holding the raw element bits (uint16 for bf16, float32 or uint32
for fp32). Every operation here is a copy of bits, so results are exact.

  * slot_mapping: "Why OS Virtual Memory Paging Saved LLM Inference"
    (a8q9.cn), section 2: the block table maps a logical token position to a
    physical block. Position p of sequence s sits in logical block p // bs at
    offset p % bs, so its physical slot is table[s][p // bs] * bs + p % bs.
    A negative position means "no token" (padding) and maps to slot -1.
    So does a position past the table's width, or an entry that names no
    block: a negative one (an unused entry), or one whose slots do not fit
    the int32 slot numbers the write takes (above (2^31 - 1 - (bs - 1)) / bs).
  * write_kv: the same section: blocks are filled as tokens are generated.
    The new token's K and V rows land in its slot, all kv heads at once:
    K[slot // bs, g, slot % bs, :] = k_new[i, g, :]. A negative slot is
    skipped (padding).
  * copy_blocks: same page, section 3 (copy-on-write): a branch about to write
    into a shared block first gets a private copy of it. Every (src, dst)
    pair copies the whole block of K and of V, all heads, slots and dims.
"""

import numpy as np


def slot_mapping(block_tables, positions, block_size=16, seq_ids=None):
    """Token i belongs to sequence seq_ids[i] (default: i); a sequence index
    outside the table's rows has no slot either."""
    bt = np.asarray(block_tables, dtype=np.int64)
    pos = np.asarray(positions, dtype=np.int64)
    rows, width = bt.shape if bt.ndim == 2 else (0, 0)
    seq = np.arange(pos.shape[0]) if seq_ids is None else np.asarray(seq_ids, dtype=np.int64)
    largest = (2**31 - 1 - (block_size - 1)) // block_size
    out = np.full(pos.shape, -1, dtype=np.int32)
    for i, (s, p) in enumerate(zip(seq.tolist(), pos.tolist())):
        if s < 0 or s >= rows or p < 0 or p // block_size >= width:
            continue
        b = int(bt[s, p // block_size])
        if b < 0 or b > largest:
            continue
        out[i] = b * block_size + p % block_size
    return out


def write_kv(k_cache, v_cache, k_new, v_new, slot_mapping):
    """In place. k_new, v_new: [T, Hkv, D] with the pools' element type."""
    bs = k_cache.shape[2]
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        b, o = divmod(slot, bs)
        k_cache[b, :, o, :] = k_new[i]
        v_cache[b, :, o, :] = v_new[i]


def copy_blocks(k_cache, v_cache, pairs):
    """In place, pairs applied in order. pairs: [n, 2] of (src, dst)."""
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2).tolist():
        k_cache[dst] = k_cache[src]
        v_cache[dst] = v_cache[src]
