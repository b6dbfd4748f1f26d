"""ctypes view of libpa.so: the C ABI declared in include/pa.h, nothing more.

The library is loaded on first use. There is no fallback: if libpa.so is not
built, every call raises.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

c_i32, c_f32, c_sz, c_vp = ctypes.c_int32, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
c_u32 = ctypes.c_uint32
c_i32p = ctypes.POINTER(ctypes.c_int32)

# name -> (restype, argtypes), in the order of include/pa.h
SIGNATURES = {
    "pa_status_str": (ctypes.c_char_p, [c_i32]),
    "pa_slot_mapping": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_vp]),
    "pa_write_kv": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32,
                            c_i32, c_vp]),
    "pa_append_kv": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32,
                             c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp]),
    "pa_check_slots": (c_i32, [c_vp, c_i32, c_vp, c_vp]),
    "pa_check_pairs": (c_i32, [c_vp, c_i32, c_i32, c_vp, c_vp]),
    "pa_check_tables": (c_i32, [c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp]),
    "pa_check_groups": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp,
                                c_vp]),
    "pa_copy_blocks": (c_i32, [c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp]),
    "pa_decode_default_partition": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_i32]),
    "pa_decode_workspace_bytes": (c_sz, [c_i32, c_i32, c_i32, c_i32, c_i32]),
    "pa_decode": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32,
                          c_i32, c_i32, c_i32, c_f32, c_i32, c_vp, c_sz, c_u32, c_i32, c_vp]),
    "pa_decode_noalloc": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32,
                                  c_i32, c_i32, c_i32, c_i32, c_i32, c_f32, c_i32, c_u32, c_i32,
                                  c_vp]),
    "pa_decode_shared_workspace_bytes": (c_sz, [c_i32, c_i32, c_i32, c_i32, c_i32]),
    "pa_decode_shared_default_partition": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_i32]),
    "pa_decode_shared": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32,
                                 c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                 c_f32, c_i32, c_vp, c_sz, c_u32, c_i32, c_vp]),
    "pa_shared_groups": (c_i32, [c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_i32p]),
    "pa_multi_query": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32,
                               c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_f32, c_i32,
                               c_vp, c_sz, c_u32, c_i32, c_vp]),
    "pa_bm_create": (c_i32, [ctypes.POINTER(c_vp), c_i32, c_i32, c_vp]),
    "pa_bm_destroy": (None, [c_vp]),
    "pa_bm_add_seq": (c_i32, [c_vp, c_i32p]),
    "pa_bm_fork": (c_i32, [c_vp, c_i32, c_i32p]),
    "pa_bm_append": (c_i32, [c_vp, c_i32, c_i32, c_vp, c_vp, c_i32p]),
    "pa_bm_append_tokens": (c_i32, [c_vp, c_i32, c_vp, c_i32, c_vp, c_vp, c_i32p]),
    "pa_bm_add_seq_cached": (c_i32, [c_vp, c_vp, c_i32, c_i32p, c_i32p]),
    "pa_bm_fork_into": (c_i32, [c_vp, c_i32, c_i32]),
    "pa_bm_free_seq": (c_i32, [c_vp, c_i32]),
    "pa_bm_seq_len": (c_i32, [c_vp, c_i32, c_i32p]),
    "pa_bm_num_free": (c_i32, [c_vp, c_i32p]),
    "pa_bm_num_cached": (c_i32, [c_vp, c_i32p]),
    "pa_bm_refcount": (c_i32, [c_vp, c_i32, c_i32p]),
    "pa_bm_block_table": (c_i32, [c_vp, c_i32, c_vp, c_i32, c_i32p]),
    "pa_bm_fill_tables": (c_i32, [c_vp, c_vp, c_i32, c_i32, c_vp, c_vp]),
}

PA_OK, PA_EINVAL, PA_EUNSUPPORTED, PA_EWORKSPACE, PA_EHIP, PA_ENOBLOCKS = 0, -1, -2, -3, -4, -5
PA_F32, PA_BF16 = 0, 1
PA_KV_SHARED = 1
PA_KV_SHARED_GROUPS = 2
PA_NOALLOC_SCRATCH_BYTES = 64 << 20

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m paged_kv_cache_410_amd.build` "
                "(or __graft_entry__.build()) first")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


class PAError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        text = lib().pa_status_str(status).decode()
        super().__init__(f"{what}: {text} ({status})")


def check(status, what):
    if status != PA_OK:
        raise PAError(status, what)
