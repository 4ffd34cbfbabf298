"""ctypes prototypes for libpagedkv.so (the C ABI declared in include/pagedkv.h).

Loading fails loudly: there is no Python or CPU fallback for any call.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedkv.so")

PKV_OK, PKV_EINVAL, PKV_ENOENT, PKV_EEXIST, PKV_ENOMEM, PKV_ECORRUPT, PKV_EHIP = range(7)
PKV_F32, PKV_BF16, PKV_I8 = 0, 1, 2

c_i32, c_i64, c_int, c_void_p, c_size_t, c_float = (
    ctypes.c_int32, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
    ctypes.c_float)
P_i32 = ctypes.POINTER(c_i32)
P_i64 = ctypes.POINTER(c_i64)


class CowPair(ctypes.Structure):
    _fields_ = [("src", c_i32), ("dst", c_i32)]


class Stats(ctypes.Structure):
    _fields_ = [(name, c_i64) for name in (
        "allocated_blocks", "free_blocks", "physical_capacity_tokens",
        "physical_payload_tokens", "logical_tokens", "internal_waste_tokens",
        "sharing_savings_tokens")]


P_cow = ctypes.POINTER(CowPair)

# name -> (restype, argtypes); every symbol include/pagedkv.h declares.
PROTOTYPES = {
    "paged_kv_last_error": (ctypes.c_char_p, []),
    "paged_kv_pool_create": (c_int, [c_i32, c_i32, P_i32, ctypes.POINTER(c_void_p)]),
    "paged_kv_pool_destroy": (None, [c_void_p]),
    "paged_kv_seq_create": (c_int, [c_void_p, c_i64]),
    "paged_kv_alloc": (c_int, [c_void_p, c_i64, c_i32, P_i32, P_cow, P_i32]),
    "paged_kv_alloc_batch": (c_int, [c_void_p, P_i64, P_i32, c_i32, P_i32, P_cow, P_i32,
                                     P_i32]),
    "paged_kv_fork": (c_int, [c_void_p, c_i64, c_i64, c_i32]),
    "paged_kv_free": (c_int, [c_void_p, c_i64]),
    "paged_kv_truncate": (c_int, [c_void_p, c_i64, c_i32]),
    "paged_kv_seq_length": (c_int, [c_void_p, c_i64, P_i32]),
    "paged_kv_seq_ids": (c_int, [c_void_p, P_i64, c_i32, P_i32]),
    "paged_kv_page_table": (c_int, [c_void_p, c_i64, P_i32, c_i32, P_i32]),
    "paged_kv_free_stack": (c_int, [c_void_p, P_i32, c_i32, P_i32]),
    "paged_kv_block_tables": (c_int, [c_void_p, P_i64, c_i32, c_i32, P_i32, P_i32]),
    "paged_kv_stats": (c_int, [c_void_p, ctypes.POINTER(Stats)]),
    "paged_kv_validate": (c_int, [c_void_p]),
    "paged_kv_check_slots": (c_int, [P_i32, c_i32, c_i64, P_i32]),
    "paged_kv_read_probe": (c_int, [c_void_p, c_size_t, c_void_p, c_i32, c_i32, c_int, c_i32,
                                    c_i32, c_void_p, c_void_p]),
    "paged_cache_write": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_i32,
                                  c_i32, c_i32, c_i32, c_i32, c_int, c_void_p]),
    "paged_kv_copy_blocks": (c_int, [c_void_p, c_void_p, c_void_p, c_i32, c_i32, c_i32,
                                     c_i32, c_i32, c_int, c_void_p]),
    "paged_attention_workspace_size": (c_int, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                               c_i32, c_i32, ctypes.POINTER(c_size_t)]),
    "paged_attention_decode": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                       c_i32, c_void_p, c_i32, c_i32, c_i32, c_i32, c_i32,
                                       c_i32, c_i32, c_float, c_int, c_i32, c_void_p,
                                       c_size_t, c_void_p, c_void_p]),
    "paged_attention_decode_noalloc": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p,
                                               c_void_p, c_i32, c_void_p, c_i32, c_i32, c_i32,
                                               c_i32, c_i32, c_i32, c_i32, c_float, c_int,
                                               c_i32, c_void_p, c_void_p]),
    "paged_cache_write_q8": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_i32, c_i32, c_i32, c_i32, c_i32,
                                     c_int, c_void_p]),
    "paged_attention_decode_q8": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                          c_void_p, c_i32, c_void_p, c_i32, c_i32,
                                          c_i32, c_i32, c_i32, c_i32, c_i32, c_float, c_i32,
                                          c_void_p, c_size_t, c_void_p, c_void_p]),
    "paged_cache_write_q3": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_i32, c_i32, c_i32, c_i32, c_i32,
                                     c_int, c_void_p]),
    "paged_attention_decode_q3": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                          c_void_p, c_i32, c_void_p, c_i32, c_i32,
                                          c_i32, c_i32, c_i32, c_i32, c_i32, c_float, c_i32,
                                          c_void_p, c_size_t, c_void_p, c_void_p]),
    "paged_kv_prefix_groups": (c_int, [P_i32, c_i32, P_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                       P_i32, P_i32, P_i32, P_i32, P_i32, P_i32, P_i32]),
    "paged_attention_shared_workspace_size": (c_int, [c_i32, c_i32, c_i32, c_i32, c_i32,
                                                      c_i32, c_i32, c_i32, c_i32, c_i32,
                                                      c_i32, ctypes.POINTER(c_size_t)]),
    "paged_attention_decode_shared": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p,
                                              c_void_p, c_i32, c_void_p, c_i32, c_i32, c_i32,
                                              c_i32, c_i32, c_i32, c_i32, c_float, c_int,
                                              c_i32, c_void_p, c_void_p, c_void_p, c_void_p,
                                              c_i32, c_i32, c_i32, c_i32, c_void_p, c_size_t,
                                              c_void_p, c_void_p]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load the in-tree library (build it first with paged_kv_cache_202_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_202_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in PROTOTYPES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class PagedKVError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class InvalidArgument(PagedKVError, ValueError):
    pass


class UnknownSequence(PagedKVError, KeyError):
    pass


class SequenceExists(PagedKVError, ValueError):
    pass


class OutOfBlocks(PagedKVError, MemoryError):
    pass


class Corrupt(PagedKVError, AssertionError):
    pass


class HipError(PagedKVError):
    pass


_ERRORS = {PKV_EINVAL: InvalidArgument, PKV_ENOENT: UnknownSequence,
           PKV_EEXIST: SequenceExists, PKV_ENOMEM: OutOfBlocks, PKV_ECORRUPT: Corrupt,
           PKV_EHIP: HipError}


def check(rc: int) -> None:
    if rc != PKV_OK:
        msg = load().paged_kv_last_error().decode(errors="replace")
        raise _ERRORS.get(rc, PagedKVError)(rc, msg)
