"""Paged-KV decode for MI355X: Python binding of libpagedkv.so.

The binding only marshals arguments: every step runs in the C++ allocator or
in the HIP kernels of the shared library (see include/pagedkv.h). Names match
the C ABI. Device buffers are torch tensors on the GPU; PyTorch is used for
device memory and streams only.
"""

from __future__ import annotations

import ctypes
import math

import numpy as np

from . import _lib
from ._lib import (  # noqa: F401
    Corrupt, HipError, InvalidArgument, OutOfBlocks, PagedKVError, SequenceExists,
    UnknownSequence, PKV_BF16, PKV_F32, check, load)

__all__ = [
    "paged_kv_read_probe", "PagedKVPool", "paged_cache_write", "paged_kv_copy_blocks",
    "paged_attention_workspace_size", "paged_attention_decode", "dtype_code",
    "PrefixGroups", "paged_kv_prefix_groups", "paged_attention_shared_workspace_size",
    "paged_attention_decode_shared", "Q8Cache", "paged_cache_write_q8",
    "paged_attention_decode_q8", "Q3Cache", "paged_cache_write_q3", "paged_attention_decode_q3",
    "paged_kv_check_slots", "paged_attention_decode_noalloc",
]


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(_lib.P_i32)


def _i64p(a: np.ndarray):
    return a.ctypes.data_as(_lib.P_i64)


class PagedKVPool:
    """Host block allocator (paged_kv_pool_* / paged_kv_* calls)."""

    def __init__(self, total_blocks: int, block_size: int = 16, initial_free_stack=None):
        lib = load()
        self._lib = lib
        self.total_blocks = int(total_blocks)
        self.block_size = int(block_size)
        handle = ctypes.c_void_p()
        stack = None
        if initial_free_stack is not None:
            stack = np.ascontiguousarray(initial_free_stack, dtype=np.int32)
            if stack.shape != (self.total_blocks,):
                raise InvalidArgument(_lib.PKV_EINVAL, "initial free stack needs N entries")
        check(lib.paged_kv_pool_create(self.total_blocks, self.block_size,
                                       None if stack is None else _i32p(stack),
                                       ctypes.byref(handle)))
        self._h = handle

    def close(self) -> None:
        if getattr(self, "_h", None):
            self._lib.paged_kv_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def seq_create(self, seq_id: int) -> None:
        check(self._lib.paged_kv_seq_create(self._h, seq_id))

    def alloc(self, seq_id: int, n_tokens: int):
        """Returns (slots int32 array, list of (src, dst) copy pairs)."""
        slots = np.empty(max(n_tokens, 1), dtype=np.int32)
        cow = (_lib.CowPair * 1)()
        n_cow = ctypes.c_int32()
        check(self._lib.paged_kv_alloc(self._h, seq_id, n_tokens, _i32p(slots), cow,
                                       ctypes.byref(n_cow)))
        return slots[:n_tokens], [(cow[i].src, cow[i].dst) for i in range(n_cow.value)]

    def alloc_batch(self, seq_ids, n_tokens):
        """Returns (slots, copy pairs [n, 2] int32). All or nothing: on any error the
        pool is unchanged and the error is raised."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        ns = np.ascontiguousarray(n_tokens, dtype=np.int32)
        slots = np.empty(max(int(ns.sum()), 1), dtype=np.int32)
        cow = (_lib.CowPair * max(len(ids), 1))()
        n_cow, n_done = ctypes.c_int32(), ctypes.c_int32()
        rc = self._lib.paged_kv_alloc_batch(self._h, _i64p(ids), _i32p(ns), len(ids),
                                            _i32p(slots), cow, ctypes.byref(n_cow),
                                            ctypes.byref(n_done))
        self.last_batch_done = n_done.value
        check(rc)
        pairs = np.array([(cow[i].src, cow[i].dst) for i in range(n_cow.value)],
                         dtype=np.int32).reshape(-1, 2)
        return slots[:int(ns.sum())], pairs

    def fork(self, parent: int, child: int, prefix_tokens: int) -> None:
        check(self._lib.paged_kv_fork(self._h, parent, child, prefix_tokens))

    def free(self, seq_id: int) -> None:
        check(self._lib.paged_kv_free(self._h, seq_id))

    def truncate(self, seq_id: int, new_length: int) -> None:
        check(self._lib.paged_kv_truncate(self._h, seq_id, new_length))

    def seq_length(self, seq_id: int) -> int:
        n = ctypes.c_int32()
        check(self._lib.paged_kv_seq_length(self._h, seq_id, ctypes.byref(n)))
        return n.value

    def seq_ids(self) -> list[int]:
        n = ctypes.c_int32()
        check(self._lib.paged_kv_seq_ids(self._h, None, 0, ctypes.byref(n)))
        out = np.empty(max(n.value, 1), dtype=np.int64)
        check(self._lib.paged_kv_seq_ids(self._h, _i64p(out), len(out), ctypes.byref(n)))
        return out[:n.value].tolist()

    def page_table(self, seq_id: int) -> tuple[int, ...]:
        n = ctypes.c_int32()
        cap = -(-self.seq_length(seq_id) // self.block_size)
        out = np.empty(max(cap, 1), dtype=np.int32)
        check(self._lib.paged_kv_page_table(self._h, seq_id, _i32p(out), len(out),
                                            ctypes.byref(n)))
        return tuple(out[:n.value].tolist())

    def free_stack(self) -> list[int]:
        n = ctypes.c_int32()
        out = np.empty(self.total_blocks, dtype=np.int32)
        check(self._lib.paged_kv_free_stack(self._h, _i32p(out), len(out), ctypes.byref(n)))
        return out[:n.value].tolist()

    def block_tables(self, seq_ids, max_blocks: int):
        """Returns (tables [n, max_blocks] int32 padded with -1, lens [n] int32)."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        tables = np.empty((len(ids), max_blocks), dtype=np.int32)
        lens = np.empty(len(ids), dtype=np.int32)
        check(self._lib.paged_kv_block_tables(self._h, _i64p(ids), len(ids), max_blocks,
                                               _i32p(tables), _i32p(lens)))
        return tables, lens

    def stats(self) -> dict:
        st = _lib.Stats()
        check(self._lib.paged_kv_stats(self._h, ctypes.byref(st)))
        return {name: getattr(st, name) for name, _ in _lib.Stats._fields_}

    def validate(self) -> None:
        check(self._lib.paged_kv_validate(self._h))


def paged_kv_check_slots(slots, num_slots: int) -> None:
    """Raise InvalidArgument if a host slot mapping names one slot in
    [0, num_slots) twice (paged_kv_check_slots)."""
    a = np.ascontiguousarray(slots, dtype=np.int32)
    dup = ctypes.c_int32()
    check(load().paged_kv_check_slots(_i32p(a), len(a), int(num_slots), ctypes.byref(dup)))


# ---------------------------------------------------------------- device ops

def dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return PKV_F32
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    raise InvalidArgument(_lib.PKV_EINVAL, f"unsupported dtype {t.dtype}")


def _stream(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t):
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise InvalidArgument(_lib.PKV_EINVAL, "device tensors must be contiguous on the GPU")
    return ctypes.c_void_p(t.data_ptr())


def _fail(msg: str):
    raise InvalidArgument(_lib.PKV_EINVAL, msg)


def _expect(t, name: str, dtypes, shape=None) -> None:
    """t has one of `dtypes` (a torch dtype or a tuple of them) and, when
    given, exactly `shape`. The kernels read raw memory, so a wrong element
    type or a short array would be read or written past its end."""
    if t is None:
        _fail(f"{name} is required")
    dtypes = dtypes if isinstance(dtypes, tuple) else (dtypes,)
    if t.dtype not in dtypes:
        _fail(f"{name} must be {' or '.join(str(d) for d in dtypes)}, not {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        _fail(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")


def _one_gpu(call: str, *tensors) -> None:
    """Every tensor given is contiguous and on the same GPU."""
    ts = [t for t in tensors if t is not None]
    for t in ts:
        if not t.is_cuda:
            _fail(f"{call}: tensors must be on the GPU, one is on {t.device}")
        if t.device != ts[0].device:
            _fail(f"{call}: tensors on {ts[0].device} and {t.device}")
        if not t.is_contiguous():
            _fail(f"{call}: tensors must be contiguous")


def _torch():
    import torch

    return torch


def _check_attention_io(call, out, lse, block_tables, context_lens, B, nq, Hq, D) -> int:
    """Output, lse and index arrays of an attention call; returns max_blocks."""
    torch = _torch()
    _expect(out, "out", torch.float32, (B, nq, Hq, D))
    if lse is not None:
        _expect(lse, "lse", torch.float32, (B, nq, Hq))
    _expect(block_tables, "block_tables", torch.int32)
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        _fail(f"{call}: block_tables must be [B, max_blocks] with B = {B}")
    _expect(context_lens, "context_lens", torch.int32, (B,))
    return int(block_tables.shape[1])


def paged_cache_write(k_new, v_new, k_cache, v_cache, slot_mapping, stream=None) -> None:
    """k_new, v_new [T, Hkv, D]; caches [NB, Hkv, bs, D]; slot_mapping int32 [T]."""
    torch = _torch()
    dt = (torch.float32, torch.bfloat16)
    _expect(k_cache, "k_cache", dt)
    if k_cache.dim() != 4:
        _fail("paged_cache_write: caches must be [num_blocks, Hkv, block_size, D]")
    NB, Hkv, bs, D = k_cache.shape
    T = k_new.shape[0]
    _expect(v_cache, "v_cache", k_cache.dtype, k_cache.shape)
    _expect(k_new, "k_new", k_cache.dtype, (T, Hkv, D))
    _expect(v_new, "v_new", k_cache.dtype, (T, Hkv, D))
    _expect(slot_mapping, "slot_mapping", torch.int32, (T,))
    _one_gpu("paged_cache_write", k_new, v_new, k_cache, v_cache, slot_mapping)
    check(load().paged_cache_write(_dev(k_new), _dev(v_new), _dev(k_cache), _dev(v_cache),
                                   _dev(slot_mapping), T, NB, Hkv, D, bs,
                                   dtype_code(k_cache), _stream(stream)))


def paged_kv_copy_blocks(k_cache, v_cache, pairs, stream=None) -> None:
    """pairs: device int32 [n, 2] of (src, dst)."""
    torch = _torch()
    _expect(k_cache, "k_cache", (torch.float32, torch.bfloat16))
    if k_cache.dim() != 4:
        _fail("paged_kv_copy_blocks: caches must be [num_blocks, Hkv, block_size, D]")
    _expect(v_cache, "v_cache", k_cache.dtype, k_cache.shape)
    NB, Hkv, bs, D = k_cache.shape
    n = pairs.shape[0]
    _expect(pairs, "pairs", torch.int32, (n, 2))
    _one_gpu("paged_kv_copy_blocks", k_cache, v_cache, pairs)
    check(load().paged_kv_copy_blocks(_dev(k_cache), _dev(v_cache), _dev(pairs), n, NB, Hkv,
                                      D, bs, dtype_code(k_cache), _stream(stream)))


class _CodeCache:
    """What the 8-bit and 3-bit caches share: one float32 scale array
    [NB, Hkv, 2, bs] holding each (block, KV head)'s K row scales (index 0)
    beside its V row scales (index 1), so that one (block, head) reads one
    contiguous run; k_scales and v_scales are views of it."""

    def _init_scales(self, num_blocks, Hkv, block_size, device):
        import torch

        self.scales = torch.ones((num_blocks, Hkv, 2, block_size), dtype=torch.float32,
                                 device=device)

    @property
    def k_scales(self):
        """K row scales [NB, Hkv, bs] (a view of `scales`)."""
        return self.scales[:, :, 0]

    @property
    def v_scales(self):
        """V row scales [NB, Hkv, bs] (a view of `scales`)."""
        return self.scales[:, :, 1]

    def _copy_blocks(self, name, code_row_bytes, pairs, stream) -> None:
        NB, Hkv, bs, _ = self.shape
        n = pairs.shape[0]
        _expect(pairs, "pairs", _torch().int32, (n, 2))
        _one_gpu(name, self.k_codes, pairs)
        check(load().paged_kv_copy_blocks(_dev(self.k_codes), _dev(self.v_codes), _dev(pairs), n,
                                          NB, Hkv, code_row_bytes, bs, _lib.PKV_I8,
                                          _stream(stream)))
        check(load().paged_kv_copy_blocks(_dev(self.scales), None, _dev(pairs), n, NB, Hkv, 2,
                                          bs, PKV_F32, _stream(stream)))


class Q8Cache(_CodeCache):
    """A paged cache of 8-bit per-row codes: int8 codes [NB, Hkv, bs, D] for
    K and for V, and the float32 scales [NB, Hkv, 2, bs] (device tensors)."""

    def __init__(self, num_blocks, Hkv, block_size, D, device):
        import torch

        shape = (num_blocks, Hkv, block_size, D)
        self.k_codes = torch.zeros(shape, dtype=torch.int8, device=device)
        self.v_codes = torch.zeros(shape, dtype=torch.int8, device=device)
        self._init_scales(num_blocks, Hkv, block_size, device)

    @property
    def shape(self):
        return tuple(self.k_codes.shape)

    def copy_blocks(self, pairs, stream=None) -> None:
        """Copy-on-write of whole blocks: codes and scales."""
        self._copy_blocks("Q8Cache.copy_blocks", self.shape[3], pairs, stream)


def paged_cache_write_q8(k_new, v_new, cache: "Q8Cache", slot_mapping, stream=None) -> None:
    """Quantize k_new, v_new [T, Hkv, D] (f32 or bf16) to 8-bit codes with one
    scale per row and scatter them to their slots."""
    torch = _torch()
    NB, Hkv, bs, D = cache.shape
    T = k_new.shape[0]
    _expect(k_new, "k_new", (torch.float32, torch.bfloat16), (T, Hkv, D))
    _expect(v_new, "v_new", k_new.dtype, (T, Hkv, D))
    _expect(slot_mapping, "slot_mapping", torch.int32, (T,))
    _one_gpu("paged_cache_write_q8", k_new, v_new, cache.k_codes, cache.v_codes,
             cache.scales, slot_mapping)
    check(load().paged_cache_write_q8(
        _dev(k_new), _dev(v_new), _dev(cache.k_codes), _dev(cache.v_codes), _dev(cache.scales),
        _dev(slot_mapping), T, NB, Hkv, D, bs, dtype_code(k_new), _stream(stream)))


def paged_attention_decode_q8(out, q, cache: "Q8Cache", block_tables, context_lens, scale,
                              partition_tokens=0, workspace=None, lse=None,
                              stream=None) -> None:
    """paged_attention_decode over a cache of 8-bit codes; q bf16 [B, nq, Hq, D]."""
    torch = _torch()
    _expect(q, "q", torch.bfloat16)
    if q.dim() != 4:
        _fail("paged_attention_decode_q8: q must be [B, nq, Hq, D]")
    B, nq, Hq, D = q.shape
    NB, Hkv, bs, Dk = cache.shape
    if Dk != D:
        _fail(f"paged_attention_decode_q8: head dim {D} of q, {Dk} of the cache")
    max_blocks = _check_attention_io("paged_attention_decode_q8", out, lse, block_tables,
                                     context_lens, B, nq, Hq, D)
    _one_gpu("paged_attention_decode_q8", out, q, cache.k_codes, cache.v_codes,
             cache.scales, block_tables, context_lens, workspace, lse)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(load().paged_attention_decode_q8(
        _dev(out), _dev(q), _dev(cache.k_codes), _dev(cache.v_codes), _dev(cache.scales),
        _dev(block_tables), max_blocks, _dev(context_lens), B, nq, Hq, Hkv, D, bs, NB,
        float(scale), int(partition_tokens), _dev(workspace), ws_bytes, _dev(lse),
        _stream(stream)))


class Q3Cache(_CodeCache):
    """A paged cache of 3-bit per-row codes, two per byte as 4-bit float e2m1
    bits (even dim in the low nibble): codes uint8 [NB, Hkv, bs, D / 2] for K
    and for V, and the float32 scales [NB, Hkv, 2, bs] (device tensors)."""

    def __init__(self, num_blocks, Hkv, block_size, D, device):
        import torch

        shape = (num_blocks, Hkv, block_size, D // 2)
        self.D = D
        self.k_codes = torch.zeros(shape, dtype=torch.uint8, device=device)
        self.v_codes = torch.zeros(shape, dtype=torch.uint8, device=device)
        self._init_scales(num_blocks, Hkv, block_size, device)

    @property
    def shape(self):
        """(num_blocks, Hkv, block_size, D): the logical shape."""
        return tuple(self.k_codes.shape[:3]) + (self.D,)

    def copy_blocks(self, pairs, stream=None) -> None:
        """Copy-on-write of whole blocks: codes and scales."""
        self._copy_blocks("Q3Cache.copy_blocks", self.D // 2, pairs, stream)


def paged_cache_write_q3(k_new, v_new, cache: "Q3Cache", slot_mapping, stream=None) -> None:
    """Quantize k_new, v_new [T, Hkv, D] (f32 or bf16) to 3-bit codes with one
    scale per row and scatter them to their slots."""
    torch = _torch()
    NB, Hkv, bs, D = cache.shape
    T = k_new.shape[0]
    _expect(k_new, "k_new", (torch.float32, torch.bfloat16), (T, Hkv, D))
    _expect(v_new, "v_new", k_new.dtype, (T, Hkv, D))
    _expect(slot_mapping, "slot_mapping", torch.int32, (T,))
    _one_gpu("paged_cache_write_q3", k_new, v_new, cache.k_codes, cache.v_codes,
             cache.scales, slot_mapping)
    check(load().paged_cache_write_q3(
        _dev(k_new), _dev(v_new), _dev(cache.k_codes), _dev(cache.v_codes), _dev(cache.scales),
        _dev(slot_mapping), T, NB, Hkv, D, bs, dtype_code(k_new), _stream(stream)))


def paged_attention_decode_q3(out, q, cache: "Q3Cache", block_tables, context_lens, scale,
                              partition_tokens=0, workspace=None, lse=None,
                              stream=None) -> None:
    """paged_attention_decode over a cache of 3-bit codes; q bf16 [B, nq, Hq, D]."""
    torch = _torch()
    _expect(q, "q", torch.bfloat16)
    if q.dim() != 4:
        _fail("paged_attention_decode_q3: q must be [B, nq, Hq, D]")
    B, nq, Hq, D = q.shape
    NB, Hkv, bs, Dk = cache.shape
    if Dk != D:
        _fail(f"paged_attention_decode_q3: head dim {D} of q, {Dk} of the cache")
    max_blocks = _check_attention_io("paged_attention_decode_q3", out, lse, block_tables,
                                     context_lens, B, nq, Hq, D)
    _one_gpu("paged_attention_decode_q3", out, q, cache.k_codes, cache.v_codes,
             cache.scales, block_tables, context_lens, workspace, lse)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(load().paged_attention_decode_q3(
        _dev(out), _dev(q), _dev(cache.k_codes), _dev(cache.v_codes), _dev(cache.scales),
        _dev(block_tables), max_blocks, _dev(context_lens), B, nq, Hq, Hkv, D, bs, NB,
        float(scale), int(partition_tokens), _dev(workspace), ws_bytes, _dev(lse),
        _stream(stream)))


def paged_attention_workspace_size(B, nq, Hq, Hkv, D, max_blocks, block_size,
                                   partition_tokens=0) -> int:
    out = ctypes.c_size_t()
    check(load().paged_attention_workspace_size(B, nq, Hq, Hkv, D, max_blocks, block_size,
                                                partition_tokens, ctypes.byref(out)))
    return out.value


def _check_decode_args(call, out, q, k_cache, v_cache, block_tables, context_lens, lse) -> int:
    torch = _torch()
    _expect(k_cache, "k_cache", (torch.float32, torch.bfloat16))
    if k_cache.dim() != 4 or q.dim() != 4:
        _fail(f"{call}: caches [num_blocks, Hkv, block_size, D] and q [B, nq, Hq, D] expected")
    _expect(v_cache, "v_cache", k_cache.dtype, k_cache.shape)
    _expect(q, "q", k_cache.dtype)
    B, nq, Hq, D = q.shape
    if k_cache.shape[3] != D:
        _fail(f"{call}: head dim {D} of q, {k_cache.shape[3]} of the caches")
    return _check_attention_io(call, out, lse, block_tables, context_lens, B, nq, Hq, D)


def paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                           partition_tokens=0, workspace=None, lse=None, stream=None) -> None:
    """out fp32 [B, nq, Hq, D]; q [B, nq, Hq, D]; tables int32 [B, max_blocks]."""
    max_blocks = _check_decode_args("paged_attention_decode", out, q, k_cache, v_cache,
                                    block_tables, context_lens, lse)
    B, nq, Hq, D = q.shape
    NB, Hkv, bs, _ = k_cache.shape
    _one_gpu("paged_attention_decode", out, q, k_cache, v_cache, block_tables, context_lens,
             workspace, lse)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(load().paged_attention_decode(
        _dev(out), _dev(q), _dev(k_cache), _dev(v_cache), _dev(block_tables), max_blocks,
        _dev(context_lens), B, nq, Hq, Hkv, D, bs, NB, float(scale), dtype_code(k_cache),
        int(partition_tokens), _dev(workspace), ws_bytes, _dev(lse), _stream(stream)))


def paged_attention_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                                   partition_tokens=0, lse=None, stream=None) -> None:
    """paged_attention_decode without a workspace: partials in the library's
    own per-GPU scratch array (calls on one GPU must not overlap)."""
    max_blocks = _check_decode_args("paged_attention_decode_noalloc", out, q, k_cache, v_cache,
                                    block_tables, context_lens, lse)
    B, nq, Hq, D = q.shape
    NB, Hkv, bs, _ = k_cache.shape
    _one_gpu("paged_attention_decode_noalloc", out, q, k_cache, v_cache, block_tables,
             context_lens, lse)
    check(load().paged_attention_decode_noalloc(
        _dev(out), _dev(q), _dev(k_cache), _dev(v_cache), _dev(block_tables), max_blocks,
        _dev(context_lens), B, nq, Hq, Hkv, D, bs, NB, float(scale), dtype_code(k_cache),
        int(partition_tokens), _dev(lse), _stream(stream)))


# ---------------------------------------------------------------- shared prefixes

class PrefixGroups:
    """Host outputs of paged_kv_prefix_groups (numpy int32 arrays and ints)."""

    def __init__(self, seq_prefix, group_start, members, group_tokens, n_groups, max_members,
                 max_prefix):
        self.seq_prefix, self.group_start = seq_prefix, group_start
        self.members, self.group_tokens = members, group_tokens
        self.n_groups, self.max_members, self.max_prefix = n_groups, max_members, max_prefix
        self.n_members = int(group_start[n_groups])

    def to_device(self, device):
        """The four arrays as device int32 tensors (for paged_attention_decode_shared)."""
        import torch

        def dev(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)

        return (dev(self.seq_prefix), dev(self.group_start[:self.n_groups + 1]),
                dev(self.members[:max(self.n_members, 1)]),
                dev(self.group_tokens[:max(self.n_groups, 1)]))


def paged_kv_prefix_groups(block_tables, context_lens, nq, block_size, min_members=2,
                           min_tokens=256) -> PrefixGroups:
    """Groups that share leading blocks, from host tables [B, max_blocks] and lengths [B]."""
    tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    B, max_blocks = tables.shape
    if lens.shape != (B,):
        raise InvalidArgument(_lib.PKV_EINVAL, "paged_kv_prefix_groups: shape mismatch")
    seq_prefix = np.zeros(B, dtype=np.int32)
    group_start = np.zeros(B + 1, dtype=np.int32)
    members = np.zeros(B, dtype=np.int32)
    group_tokens = np.zeros(B, dtype=np.int32)
    ng, mm, mp = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    check(load().paged_kv_prefix_groups(
        _i32p(tables), max_blocks, _i32p(lens), B, int(nq), int(block_size), int(min_members),
        int(min_tokens), _i32p(seq_prefix), _i32p(group_start), _i32p(members),
        _i32p(group_tokens), ctypes.byref(ng), ctypes.byref(mm), ctypes.byref(mp)))
    return PrefixGroups(seq_prefix, group_start, members, group_tokens, ng.value, mm.value,
                        mp.value)


def paged_attention_shared_workspace_size(B, nq, Hq, Hkv, D, max_blocks, block_size,
                                          groups: PrefixGroups, partition_tokens=0) -> int:
    out = ctypes.c_size_t()
    check(load().paged_attention_shared_workspace_size(
        B, nq, Hq, Hkv, D, max_blocks, block_size, partition_tokens, groups.n_groups,
        groups.max_members, groups.max_prefix, ctypes.byref(out)))
    return out.value


def paged_attention_decode_shared(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                                  groups: PrefixGroups, device_groups, partition_tokens=0,
                                  workspace=None, lse=None, stream=None) -> None:
    """paged_attention_decode with shared prefixes read once per group and KV head.

    device_groups: groups.to_device(...) (seq_prefix, group_start, members,
    group_tokens as device int32 tensors)."""
    max_blocks = _check_decode_args("paged_attention_decode_shared", out, q, k_cache, v_cache,
                                    block_tables, context_lens, lse)
    B, nq, Hq, D = q.shape
    NB, Hkv, bs, _ = k_cache.shape
    seq_prefix, group_start, members, group_tokens = device_groups
    i32 = _torch().int32
    _expect(seq_prefix, "seq_prefix", i32, (B,))
    _expect(group_start, "group_start", i32, (groups.n_groups + 1,))
    _expect(members, "members", i32, (max(groups.n_members, 1),))
    _expect(group_tokens, "group_tokens", i32, (max(groups.n_groups, 1),))
    _one_gpu("paged_attention_decode_shared", out, q, k_cache, v_cache, block_tables,
             context_lens, seq_prefix, group_start, members, group_tokens, workspace, lse)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(load().paged_attention_decode_shared(
        _dev(out), _dev(q), _dev(k_cache), _dev(v_cache), _dev(block_tables), max_blocks,
        _dev(context_lens), B, nq, Hq, Hkv, D, bs, NB, float(scale), dtype_code(k_cache),
        int(partition_tokens), _dev(seq_prefix), _dev(group_start), _dev(members),
        _dev(group_tokens), groups.n_groups, groups.n_members, groups.max_members,
        groups.max_prefix, _dev(workspace), ws_bytes, _dev(lse), _stream(stream)))


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def paged_kv_read_probe(buf, order, sink, chunk_bytes: int = 4096, mode: int = 2,
                        ring_bytes: int = 16384, stream=None) -> None:
    """Measurement aid (paged_kv_read_probe): read chunks of `buf` (a uint8
    device tensor) in the order of `order` (int32 chunk indices) with the
    decode kernels' load pattern; `sink` (uint32 or int32, one per
    workgroup) receives each workgroup's XOR of the words it read. In LDS
    mode (2) each wavefront keeps `ring_bytes` (4, 8 or 16 KiB) in flight."""
    torch = _torch()
    _expect(buf, "buf", torch.uint8)
    _expect(order, "order", torch.int32)
    _expect(sink, "sink", (torch.int32, torch.uint32) if hasattr(torch, "uint32") else torch.int32)
    _one_gpu("paged_kv_read_probe", buf, order, sink)
    check(load().paged_kv_read_probe(
        ctypes.c_void_p(buf.data_ptr()), buf.numel(), ctypes.c_void_p(order.data_ptr()),
        order.numel(), int(chunk_bytes), int(mode), int(ring_bytes), sink.numel(),
        ctypes.c_void_p(sink.data_ptr()), _stream(stream)))
