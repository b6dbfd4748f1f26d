"""CPU oracle for paged decode attention and its block bookkeeping.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this package. The GPU library
(paged_kv_cache_410_amd) never imports it and shares no code with it; the
oracle never imports the library.

Contents
  decode(...)        fp64 paged attention, C (pa_oracle.c -> liboracle.so)
  multi_query(...)   fp64 causal attention of several new tokens per sequence
  cache_ops          slot mapping, cache write, block copy (numpy bit moves)
  blockmgr           free list / block tables / refcounts / copy-on-write
  dense              textbook contiguous attention (pins the C decode)

Parity pins for every function are in tests/test_oracle_*.py.
"""

import ctypes
import os
import subprocess

import numpy as np

from . import blockmgr, cache_ops, dense  # noqa: F401
from .blockmgr import BlockManager, OutOfBlocks  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1


def build(force=False):
    """Compile liboracle.so with gcc (plain C, -O2, no fast-math, OpenMP)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC",
           "-std=c11", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        lib.oracle_decode.restype = ctypes.c_int
        lib.oracle_decode.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_float, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_int32]
        lib.oracle_multi_query.restype = ctypes.c_int
        lib.oracle_multi_query.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_float, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32]
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads():
    return _load().oracle_max_threads()


def _dtype_code(arr):
    if arr.dtype == np.uint16:
        return BF16
    if arr.dtype in (np.float32, np.uint32):
        return F32
    raise TypeError(f"unsupported element type {arr.dtype} (uint16 = bf16 bits, float32)")


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, pairs=None, n_threads=0):
    """fp64 paged decode attention.

    q [B, Hq, D]; k_cache, v_cache [NB, Hkv, bs, D]; element type uint16 (raw
    bf16 bits) or float32, the same for all three. block_tables int32 [B, MB];
    context_lens int32 [B]. scale is rounded to fp32 first (the GPU gets an
    fp32 scale). pairs: optional [(s, h), ...] -> output [n, D]; otherwise
    [B, Hq, D]. Returns float64.
    """
    lib = _load()
    q = np.ascontiguousarray(q)
    k_cache = np.ascontiguousarray(k_cache)
    v_cache = np.ascontiguousarray(v_cache)
    dt = _dtype_code(q)
    if _dtype_code(k_cache) != dt or _dtype_code(v_cache) != dt:
        raise TypeError("q, k_cache and v_cache must share one element type")
    B, Hq, D = q.shape
    NB, Hkv, bs, Dk = k_cache.shape
    if v_cache.shape != k_cache.shape or Dk != D:
        raise ValueError("shape mismatch")
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    if bt.ndim != 2 or bt.shape[0] != B or cl.shape != (B,):
        raise ValueError("block_tables / context_lens shape mismatch")
    MB = bt.shape[1]
    if pairs is not None:
        pr = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
        n = pr.shape[0]
        out = np.empty((n, D), dtype=np.float64)
        pr_ptr = pr.ctypes.data
    else:
        pr = None
        n = 0
        out = np.empty((B, Hq, D), dtype=np.float64)
        pr_ptr = None
    rc = lib.oracle_decode(out.ctypes.data, q.ctypes.data, k_cache.ctypes.data,
                           v_cache.ctypes.data, bt.ctypes.data, cl.ctypes.data,
                           B, Hq, Hkv, D, bs, NB, MB, float(np.float32(scale)), dt,
                           pr_ptr, n, int(n_threads))
    if rc != 0:
        raise ValueError(f"oracle_decode failed ({rc}): bad argument or block id out of range")
    return out


def multi_query(q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
                pairs=None, n_threads=0):
    """fp64 causal attention of several new tokens per sequence.

    q [Tq, Hq, D]; sequence s owns rows query_start[s] .. query_start[s+1]-1,
    the last n_s tokens of its context (row i at position ctx_s - n_s + i,
    attending to positions 0 .. ctx_s - n_s + i). Element types as decode().
    pairs: optional [(row, head), ...] -> output [n, D]. Returns float64
    [Tq, Hq, D] otherwise.
    """
    lib = _load()
    q = np.ascontiguousarray(q)
    k_cache = np.ascontiguousarray(k_cache)
    v_cache = np.ascontiguousarray(v_cache)
    dt = _dtype_code(q)
    if _dtype_code(k_cache) != dt or _dtype_code(v_cache) != dt:
        raise TypeError("q, k_cache and v_cache must share one element type")
    Tq, Hq, D = q.shape
    NB, Hkv, bs, Dk = k_cache.shape
    if v_cache.shape != k_cache.shape or Dk != D:
        raise ValueError("shape mismatch")
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    qs = np.ascontiguousarray(query_start, dtype=np.int32)
    B = cl.shape[0]
    if bt.ndim != 2 or bt.shape[0] != B or qs.shape != (B + 1,):
        raise ValueError("block_tables / query_start shape mismatch")
    if pairs is not None:
        pr = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
        out = np.empty((pr.shape[0], D), dtype=np.float64)
        pr_ptr, n_pr = pr.ctypes.data, pr.shape[0]
    else:
        out = np.empty((Tq, Hq, D), dtype=np.float64)
        pr_ptr, n_pr = None, 0
    rc = lib.oracle_multi_query(out.ctypes.data, q.ctypes.data, k_cache.ctypes.data,
                                v_cache.ctypes.data, bt.ctypes.data, cl.ctypes.data,
                                qs.ctypes.data, B, Tq, Hq, Hkv, D, bs, NB, bt.shape[1],
                                float(np.float32(scale)), dt, pr_ptr, n_pr, int(n_threads))
    if rc != 0:
        raise ValueError(f"oracle_multi_query failed ({rc}): bad argument, a chunk longer "
                         "than its context, or a block id out of range")
    return out
