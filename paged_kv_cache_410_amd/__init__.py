"""Paged KV-cache decode attention for AMD Instinct MI355X (gfx950).

Python face of libpa.so (include/pa.h). Each function checks tensor shapes,
dtypes, devices and contiguity, then calls the C function of the same name on
torch's current stream. Every step runs in the library's HIP kernels; torch
provides device memory and streams only.

    slot_mapping(block_tables, positions)                  -> int32 [B]
    write_kv(k_new, v_new, k_cache, v_cache, slot_mapping)    (in place)
    copy_blocks(k_cache, v_cache, pairs)                      (in place)
    decode(q, k_cache, v_cache, block_tables, context_lens, scale, max_ctx,
           partition=None, out=None, workspace=None, shared_kv=False) -> [B, Hq, D]
    multi_query(q, k_cache, v_cache, block_tables, context_lens, query_start,
                scale, max_ctx, max_q, partition=None)   -> [Tq, Hq, D]
    BlockManager(num_blocks, block_size=16, free_order=None)

Pools are [num_blocks, num_kv_heads, 16, head_dim] tensors (fp32 or bf16).
"""

import ctypes

import numpy as np
import torch

from ._lib import (PA_BF16, PA_ENOBLOCKS, PA_EWORKSPACE, PA_F32, PA_KV_SHARED,  # noqa: F401
                   PA_KV_SHARED_GROUPS, PA_NOALLOC_SCRATCH_BYTES, PAError, check, lib)

__all__ = ["slot_mapping", "write_kv", "append_kv", "copy_blocks", "check_slots", "check_pairs",
           "check_tables", "decode", "decode_noalloc", "multi_query", "shares_blocks",
           "decode_workspace_bytes",
           "default_partition", "BlockManager", "PAError", "shared_groups", "decode_shared",
           "decode_shared_workspace_bytes", "check_groups",
           "decode_shared_default_partition", "shared_plan"]

BLOCK_SIZE = 16


def _dt(t):
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: use float32 or bfloat16")


def _dev(*ts):
    dev = ts[0].device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    for t in ts:
        if t.device != dev:
            raise ValueError("tensors must share one device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return dev


def _i32(t, name):
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")
    return t


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def slot_mapping(block_tables, positions, seq_ids=None, out=None):
    """Slot of each (sequence, position): positions [T], seq_ids [T] or None (= 0..T-1)."""
    _i32(block_tables, "block_tables")
    _i32(positions, "positions")
    B, MB = block_tables.shape
    T = positions.shape[0]
    ts = [block_tables, positions]
    if seq_ids is not None:
        _i32(seq_ids, "seq_ids")
        if seq_ids.shape != (T,):
            raise ValueError("seq_ids must match positions")
        ts.append(seq_ids)
    elif T > B:
        raise ValueError("without seq_ids there is one position per sequence")
    if out is None:
        out = torch.empty(T, dtype=torch.int32, device=block_tables.device)
    _i32(out, "out")
    if out.shape != (T,):
        raise ValueError("out must be [T]")
    dev = _dev(*ts, out)
    with torch.cuda.device(dev):
        check(lib().pa_slot_mapping(out.data_ptr(), block_tables.data_ptr(),
                                    seq_ids.data_ptr() if seq_ids is not None else None,
                                    positions.data_ptr(), T, B, MB, BLOCK_SIZE, _stream(dev)),
              "pa_slot_mapping")
    return out


def _pool_dims(k_cache, v_cache):
    if k_cache.dim() != 4 or k_cache.shape != v_cache.shape or k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache and v_cache must be matching [NB, Hkv, 16, D] tensors")
    NB, Hkv, bs, D = k_cache.shape
    return NB, Hkv, bs, D


def write_kv(k_new, v_new, k_cache, v_cache, slot_mapping):
    NB, Hkv, bs, D = _pool_dims(k_cache, v_cache)
    _i32(slot_mapping, "slot_mapping")
    T = slot_mapping.shape[0]
    if k_new.shape != (T, Hkv, D) or v_new.shape != (T, Hkv, D):
        raise ValueError("k_new / v_new must be [T, Hkv, D]")
    if k_new.dtype != k_cache.dtype or v_new.dtype != k_cache.dtype:
        raise TypeError("new rows and pools must share a dtype")
    dev = _dev(k_new, v_new, k_cache, v_cache, slot_mapping)
    with torch.cuda.device(dev):
        check(lib().pa_write_kv(k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(),
                                v_cache.data_ptr(), slot_mapping.data_ptr(), T, NB, Hkv, D, bs,
                                _dt(k_cache), _stream(dev)), "pa_write_kv")


def append_kv(k_new, v_new, k_cache, v_cache, block_tables, positions, seq_ids=None,
              slots_out=None):
    """slot_mapping + write_kv in one launch. Returns slots_out (None if not given)."""
    NB, Hkv, bs, D = _pool_dims(k_cache, v_cache)
    _i32(block_tables, "block_tables")
    _i32(positions, "positions")
    B, MB = block_tables.shape
    T = positions.shape[0]
    ts = [k_new, v_new, k_cache, v_cache, block_tables, positions]
    if seq_ids is not None:
        _i32(seq_ids, "seq_ids")
        if seq_ids.shape != (T,):
            raise ValueError("seq_ids must match positions")
        ts.append(seq_ids)
    elif T > B:
        raise ValueError("without seq_ids there is one position per sequence")
    if slots_out is not None:
        _i32(slots_out, "slots_out")
        if slots_out.shape != (T,):
            raise ValueError("slots_out must be [T]")
        ts.append(slots_out)
    if k_new.shape != (T, Hkv, D) or v_new.shape != (T, Hkv, D):
        raise ValueError("k_new / v_new must be [T, Hkv, D]")
    if k_new.dtype != k_cache.dtype or v_new.dtype != k_cache.dtype:
        raise TypeError("new rows and pools must share a dtype")
    dev = _dev(*ts)
    with torch.cuda.device(dev):
        check(lib().pa_append_kv(k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(),
                                 v_cache.data_ptr(),
                                 slots_out.data_ptr() if slots_out is not None else None,
                                 block_tables.data_ptr(),
                                 seq_ids.data_ptr() if seq_ids is not None else None,
                                 positions.data_ptr(), T, B, MB, NB, Hkv, D, bs, _dt(k_cache),
                                 _stream(dev)), "pa_append_kv")
    return slots_out


def _count(dev, call, name):
    count = torch.empty(1, dtype=torch.int32, device=dev)
    with torch.cuda.device(dev):
        check(call(count.data_ptr(), _stream(dev)), name)
    return int(count.item())          # synchronises


def check_slots(slot_mapping):
    """Tokens of one cache write whose slot repeats an earlier token's (0: none)."""
    _i32(slot_mapping, "slot_mapping")
    dev = _dev(slot_mapping)
    T = slot_mapping.shape[0]
    return _count(dev, lambda c, st: lib().pa_check_slots(slot_mapping.data_ptr(), T, c, st),
                  "pa_check_slots")


def check_pairs(pairs, num_blocks):
    """Copy pairs whose destination repeats or is also a source (0: none)."""
    _i32(pairs, "pairs")
    if pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be [n, 2]")
    dev = _dev(pairs)
    return _count(dev, lambda c, st: lib().pa_check_pairs(pairs.data_ptr(), pairs.shape[0],
                                                          num_blocks, c, st), "pa_check_pairs")


def check_tables(block_tables, context_lens, num_blocks, max_ctx):
    """Sequences with a length out of bounds or a used table entry outside the pool."""
    _i32(block_tables, "block_tables")
    _i32(context_lens, "context_lens")
    B, MB = block_tables.shape
    if context_lens.shape != (B,):
        raise ValueError("context_lens must be [B]")
    dev = _dev(block_tables, context_lens)
    return _count(dev, lambda c, st: lib().pa_check_tables(
        block_tables.data_ptr(), context_lens.data_ptr(), B, MB, num_blocks, max_ctx,
        BLOCK_SIZE, c, st), "pa_check_tables")


def check_groups(group_start, seq_shared, block_tables, context_lens, max_group):
    """Violations of what pa_decode_shared takes on trust (pa_check_groups)."""
    for t, name in ((group_start, "group_start"), (seq_shared, "seq_shared"),
                    (block_tables, "block_tables"), (context_lens, "context_lens")):
        _i32(t, name)
    if block_tables.dim() != 2:
        raise ValueError("block_tables must be [B, MB]")
    B, MB = block_tables.shape
    if context_lens.shape != (B,) or seq_shared.shape != (B,) or group_start.dim() != 1 \
            or group_start.shape[0] < 1:
        raise ValueError("context_lens and seq_shared must be [B], group_start [n_groups + 1]")
    n = group_start.shape[0] - 1
    dev = _dev(group_start, seq_shared, block_tables, context_lens)
    return _count(dev, lambda c, st: lib().pa_check_groups(
        group_start.data_ptr(), seq_shared.data_ptr(), block_tables.data_ptr(),
        context_lens.data_ptr(), B, n, int(max_group), MB, 16, c, st), "pa_check_groups")


def copy_blocks(k_cache, v_cache, pairs):
    NB, Hkv, bs, D = _pool_dims(k_cache, v_cache)
    _i32(pairs, "pairs")
    if pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be [n, 2]")
    dev = _dev(k_cache, v_cache, pairs)
    with torch.cuda.device(dev):
        check(lib().pa_copy_blocks(k_cache.data_ptr(), v_cache.data_ptr(), pairs.data_ptr(),
                                   pairs.shape[0], NB, Hkv, D, bs, _dt(k_cache), _stream(dev)),
              "pa_copy_blocks")


def shares_blocks(block_tables):
    """Whether some physical block appears more than once in the tables
    (host numpy array or tensor): the case for shared_kv=True."""
    bt = np.asarray(block_tables.cpu() if hasattr(block_tables, "cpu") else block_tables)
    ids = bt[bt >= 0]
    return bool(ids.size) and np.unique(ids).size < ids.size


def default_partition(B, Hq, Hkv, D, max_ctx):
    return int(lib().pa_decode_default_partition(B, Hq, Hkv, D, max_ctx))


def decode_workspace_bytes(B, Hq, D, max_ctx, partition):
    return int(lib().pa_decode_workspace_bytes(B, Hq, D, max_ctx, partition))


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, max_ctx, partition=None,
           out=None, workspace=None, shared_kv=False):
    """Single-query decode attention (pa_decode). shared_kv: some block is
    referenced by several sequences (forks, beams, prefix cache); K/V are then
    read through the caches instead of streamed past them (PA_KV_SHARED)."""
    NB, Hkv, bs, D = _pool_dims(k_cache, v_cache)
    _i32(block_tables, "block_tables")
    _i32(context_lens, "context_lens")
    B, Hq, Dq = q.shape
    if Dq != D or q.dtype != k_cache.dtype:
        raise ValueError("q must be [B, Hq, D] with the pools' dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [B, MB] and context_lens [B]")
    MB = block_tables.shape[1]
    if partition is None:
        with torch.cuda.device(q.device):
            partition = default_partition(B, Hq, Hkv, D, max_ctx)
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    need = decode_workspace_bytes(B, Hq, D, max_ctx, partition)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    tensors = [q, k_cache, v_cache, block_tables, context_lens, out]
    if workspace is not None:
        tensors.append(workspace)
    dev = _dev(*tensors)
    with torch.cuda.device(dev):
        check(lib().pa_decode(out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                              block_tables.data_ptr(), context_lens.data_ptr(), B, Hq, Hkv, D, bs,
                              NB, MB, int(max_ctx), float(scale), int(partition), ws_ptr, ws_bytes,
                              PA_KV_SHARED if shared_kv else 0, _dt(q), _stream(dev)), "pa_decode")
    return out


def decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale, max_ctx,
                   partition=None, out=None, shared_kv=False):
    """pa_decode without a workspace (pa_decode_noalloc): split-context
    partials go to the library's per-GPU scratch area, so the C call allocates
    nothing. Pass `out` to allocate nothing here either. Calls that overlap
    in time on one GPU race on the scratch area."""
    NB, Hkv, bs, D = _pool_dims(k_cache, v_cache)
    _i32(block_tables, "block_tables")
    _i32(context_lens, "context_lens")
    B, Hq, Dq = q.shape
    if Dq != D or q.dtype != k_cache.dtype:
        raise ValueError("q must be [B, Hq, D] with the pools' dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [B, MB] and context_lens [B]")
    MB = block_tables.shape[1]
    if partition is None:
        with torch.cuda.device(q.device):
            partition = default_partition(B, Hq, Hkv, D, max_ctx)
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    dev = _dev(q, k_cache, v_cache, block_tables, context_lens, out)
    with torch.cuda.device(dev):
        check(lib().pa_decode_noalloc(out.data_ptr(), q.data_ptr(), k_cache.data_ptr(),
                                      v_cache.data_ptr(), block_tables.data_ptr(),
                                      context_lens.data_ptr(), B, Hq, Hkv, D, bs, NB, MB,
                                      int(max_ctx), float(scale), int(partition),
                                      PA_KV_SHARED if shared_kv else 0, _dt(q), _stream(dev)),
              "pa_decode_noalloc")
    return out


def shared_groups(block_tables, context_lens, max_group):
    """Groups of consecutive sequences that share leading blocks, from host
    tables (pa_shared_groups): (group_start int32 [n_groups + 1], seq_shared
    int32 [B]) as numpy arrays."""
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    if bt.ndim != 2 or cl.shape != (bt.shape[0],):
        raise ValueError("block_tables must be [B, MB] and context_lens [B]")
    B, MB = bt.shape
    gs = np.zeros(B + 1, np.int32)
    sh = np.zeros(B, np.int32)
    n = ctypes.c_int32(0)
    check(lib().pa_shared_groups(bt.ctypes.data, cl.ctypes.data, B, MB, 16, int(max_group),
                                 gs.ctypes.data, sh.ctypes.data, ctypes.byref(n)),
          "pa_shared_groups")
    return gs[:n.value + 1].copy(), sh


def shared_plan(block_tables, context_lens, Hq, Hkv, max_group=16):
    """How a batch whose sequences share leading blocks is decoded with
    decode_shared(), from host tables: the groups of sharers, the shared-part
    partition (the library's choice for the current device) and the two cache
    flags. After grouping, a pass reads through the caches only when blocks
    still repeat within it: groups_overlap when the shared parts of different
    groups overlap (one prefix over several groups), shared_kv when sequences'
    own blocks repeat. Returns None when no sequence shares a block with its
    group. Host numpy arrays in and out (group_start, seq_shared)."""
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    gs, sh = shared_groups(bt, cl, max_group)
    if not sh.any():
        return None
    shared_reads, own_reads = [], []
    for j in range(len(gs) - 1):
        a, b = int(gs[j]), int(gs[j + 1])
        nsh = int(sh[a]) // BLOCK_SIZE
        shared_reads += bt[a, :nsh].tolist()
        for s in range(a, b):
            own_reads += bt[s, nsh:(int(cl[s]) + BLOCK_SIZE - 1) // BLOCK_SIZE].tolist()
    max_shared = int(sh.max())
    return dict(group_start=gs, seq_shared=sh, max_group=int(max_group), max_shared=max_shared,
                partition=decode_shared_default_partition(len(gs) - 1, Hq, Hkv, max_group,
                                                          max_shared),
                groups_overlap=len(set(shared_reads)) < len(shared_reads),
                shared_kv=len(set(own_reads)) < len(own_reads))


def decode_shared_default_partition(n_groups, Hq, Hkv, max_group, max_shared):
    return int(lib().pa_decode_shared_default_partition(n_groups, Hq, Hkv, max_group,
                                                        max_shared))


def decode_shared_workspace_bytes(B, Hq, D, max_shared, partition):
    return int(lib().pa_decode_shared_workspace_bytes(B, Hq, D, max_shared, partition))


def decode_shared(q, k_cache, v_cache, block_tables, context_lens, group_start, seq_shared,
                  scale, max_ctx, max_group, max_shared, partition=None, out=None, workspace=None,
                  shared_kv=False, groups_overlap=False):
    """pa_decode for sequences that share leading blocks (pa_decode_shared):
    group_start int32 [n_groups + 1] and seq_shared int32 [B] on the device,
    as shared_groups() gives them; max_group and max_shared bound them.
    partition splits the shared part (0 = one partition; None = the library's
    choice for the current device). shared_kv: blocks
    past the shared parts are read by several sequences; groups_overlap: the
    shared parts of different groups overlap (PA_KV_SHARED_GROUPS)."""
    NB, Hkv, bs, D = _pool_dims(k_cache, v_cache)
    for t, name in ((block_tables, "block_tables"), (context_lens, "context_lens"),
                    (group_start, "group_start"), (seq_shared, "seq_shared")):
        _i32(t, name)
    B, Hq, Dq = q.shape
    if Dq != D or q.dtype != k_cache.dtype:
        raise ValueError("q must be [B, Hq, D] with the pools' dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,) \
            or seq_shared.shape != (B,) or group_start.dim() != 1:
        raise ValueError("block_tables [B, MB], context_lens and seq_shared [B], "
                         "group_start [n_groups + 1]")
    MB = block_tables.shape[1]
    n_groups = group_start.shape[0] - 1
    if partition is None:
        with torch.cuda.device(q.device):
            partition = decode_shared_default_partition(n_groups, Hq, Hkv, int(max_group),
                                                        int(max_shared))
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    need = decode_shared_workspace_bytes(B, Hq, D, max_shared, partition)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    dev = _dev(q, k_cache, v_cache, block_tables, context_lens, group_start, seq_shared, out,
               workspace)
    with torch.cuda.device(dev):
        check(lib().pa_decode_shared(
            out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            block_tables.data_ptr(), context_lens.data_ptr(), group_start.data_ptr(),
            seq_shared.data_ptr(), B, n_groups, int(max_group), int(max_shared), Hq, Hkv, D, bs,
            NB, MB, int(max_ctx), float(scale), int(partition), workspace.data_ptr(), ws_bytes,
            (PA_KV_SHARED if shared_kv else 0) | (PA_KV_SHARED_GROUPS if groups_overlap else 0),
            _dt(q), _stream(dev)), "pa_decode_shared")
    return out


def multi_query(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, max_ctx,
                max_q, partition=None, out=None, workspace=None, shared_kv=False):
    """Causal attention of several new tokens per sequence (pa_multi_query).

    q [Tq, Hq, D]; query_start int32 [B + 1]: sequence s owns rows
    query_start[s] .. query_start[s+1]-1, the last tokens of its context.
    max_q bounds the rows per sequence. shared_kv as for decode()."""
    NB, Hkv, bs, D = _pool_dims(k_cache, v_cache)
    _i32(block_tables, "block_tables")
    _i32(context_lens, "context_lens")
    _i32(query_start, "query_start")
    Tq, Hq, Dq = q.shape
    if Dq != D or q.dtype != k_cache.dtype:
        raise ValueError("q must be [Tq, Hq, D] with the pools' dtype")
    B = context_lens.shape[0]
    if block_tables.dim() != 2 or block_tables.shape[0] != B or query_start.shape != (B + 1,):
        raise ValueError("block_tables must be [B, MB] and query_start [B + 1]")
    MB = block_tables.shape[1]
    if partition is None:
        with torch.cuda.device(q.device):
            partition = default_partition(max(Tq, 1), Hq, Hkv, D, max_ctx)
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    need = decode_workspace_bytes(Tq, Hq, D, max_ctx, partition)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    tensors = [q, k_cache, v_cache, block_tables, context_lens, query_start, out]
    if workspace is not None:
        tensors.append(workspace)
    dev = _dev(*tensors)
    with torch.cuda.device(dev):
        check(lib().pa_multi_query(out.data_ptr(), q.data_ptr(), k_cache.data_ptr(),
                                   v_cache.data_ptr(), block_tables.data_ptr(),
                                   context_lens.data_ptr(), query_start.data_ptr(), B, Tq,
                                   int(max_q), Hq, Hkv, D, bs, NB, MB, int(max_ctx), float(scale),
                                   int(partition), ws_ptr, ws_bytes,
                                   PA_KV_SHARED if shared_kv else 0, _dt(q), _stream(dev)),
              "pa_multi_query")
    return out


class BlockManager:
    """Host-side block bookkeeping in the native library (pa_bm_* in pa.h)."""

    def __init__(self, num_blocks, block_size=BLOCK_SIZE, free_order=None):
        self._h = ctypes.c_void_p()
        fo = None
        if free_order is not None:
            fo = np.ascontiguousarray(free_order, dtype=np.int32)
            if fo.shape != (num_blocks,):
                raise ValueError("free_order must have num_blocks entries")
        self._destroy = lib().pa_bm_destroy  # held so teardown at exit still finds it
        check(lib().pa_bm_create(ctypes.byref(self._h), num_blocks, block_size,
                                 fo.ctypes.data if fo is not None else None), "pa_bm_create")
        self._fo = fo
        self.num_blocks = num_blocks
        self.block_size = block_size

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._destroy(h)
            self._h = None

    def add_seq(self):
        out = ctypes.c_int32()
        check(lib().pa_bm_add_seq(self._h, ctypes.byref(out)), "pa_bm_add_seq")
        return out.value

    def fork(self, parent):
        out = ctypes.c_int32()
        check(lib().pa_bm_fork(self._h, parent, ctypes.byref(out)), "pa_bm_fork")
        return out.value

    def append(self, sid, n=1):
        slots = np.empty(max(n, 1), dtype=np.int32)
        pair = np.empty(2, dtype=np.int32)
        npairs = ctypes.c_int32()
        st = lib().pa_bm_append(self._h, sid, n, slots.ctypes.data, pair.ctypes.data,
                                ctypes.byref(npairs))
        check(st, "pa_bm_append")
        pairs = [(int(pair[0]), int(pair[1]))] if npairs.value else []
        return slots[:n].tolist(), pairs

    def append_tokens(self, sid, tokens):
        """Append tokens with known ids (their full blocks become shareable)."""
        toks = np.ascontiguousarray(tokens, dtype=np.int32).reshape(-1)
        n = toks.shape[0]
        slots = np.empty(max(n, 1), dtype=np.int32)
        pair = np.empty(2, dtype=np.int32)
        npairs = ctypes.c_int32()
        check(lib().pa_bm_append_tokens(self._h, sid, toks.ctypes.data if n else None, n,
                                        slots.ctypes.data, pair.ctypes.data,
                                        ctypes.byref(npairs)), "pa_bm_append_tokens")
        pairs = [(int(pair[0]), int(pair[1]))] if npairs.value else []
        return slots[:n].tolist(), pairs

    def add_seq_cached(self, tokens):
        """New sequence reusing the registered prefix of `tokens`: (seq, n_cached)."""
        toks = np.ascontiguousarray(tokens, dtype=np.int32).reshape(-1)
        n = toks.shape[0]
        sid, nc = ctypes.c_int32(), ctypes.c_int32()
        check(lib().pa_bm_add_seq_cached(self._h, toks.ctypes.data if n else None, n,
                                         ctypes.byref(sid), ctypes.byref(nc)),
              "pa_bm_add_seq_cached")
        return sid.value, nc.value

    def fork_into(self, dst, src):
        check(lib().pa_bm_fork_into(self._h, dst, src), "pa_bm_fork_into")

    def num_cached(self):
        out = ctypes.c_int32()
        check(lib().pa_bm_num_cached(self._h, ctypes.byref(out)), "pa_bm_num_cached")
        return out.value

    def free_seq(self, sid):
        check(lib().pa_bm_free_seq(self._h, sid), "pa_bm_free_seq")

    def seq_len(self, sid):
        out = ctypes.c_int32()
        check(lib().pa_bm_seq_len(self._h, sid, ctypes.byref(out)), "pa_bm_seq_len")
        return out.value

    def num_free(self):
        out = ctypes.c_int32()
        check(lib().pa_bm_num_free(self._h, ctypes.byref(out)), "pa_bm_num_free")
        return out.value

    def refcount(self, b):
        out = ctypes.c_int32()
        check(lib().pa_bm_refcount(self._h, b, ctypes.byref(out)), "pa_bm_refcount")
        return out.value

    def block_table(self, sid):
        n = ctypes.c_int32()
        check(lib().pa_bm_block_table(self._h, sid, None, 0, ctypes.byref(n)), "pa_bm_block_table")
        buf = np.empty(max(n.value, 1), dtype=np.int32)
        check(lib().pa_bm_block_table(self._h, sid, buf.ctypes.data, n.value, ctypes.byref(n)),
              "pa_bm_block_table")
        return buf[:n.value].tolist()

    def tables_array(self, sids, max_blocks):
        seqs = np.ascontiguousarray(sids, dtype=np.int32)
        tables = np.empty((len(seqs), max_blocks), dtype=np.int32)
        lens = np.empty(len(seqs), dtype=np.int32)
        check(lib().pa_bm_fill_tables(self._h, seqs.ctypes.data, len(seqs), max_blocks,
                                      tables.ctypes.data, lens.ctypes.data), "pa_bm_fill_tables")
        return tables
