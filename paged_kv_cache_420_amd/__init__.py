"""paged_kv_cache_420_amd -- paged KV-cache attention for AMD MI355X (gfx950).

Thin Python binding over libpkv.so (C ABI declared in include/pkv.h).  Each
function here has the name of a C entry point without its "pkv_" prefix and
only marshals arguments: shapes and dtypes are read from torch tensors,
pointers and the current HIP stream are passed down, and status codes become
exceptions.  Every step of the computation runs in the library's HIP
kernels; torch provides device memory and streams, nothing else.  There is
no fallback: importing this package fails if libpkv.so has not been built
(python paged_kv_cache_420_amd/_build.py).

Cache layout (K and V alike): [num_blocks, num_kv_heads, block_size, head_dim],
a tensor of the cache dtype (float32, float16 or bfloat16) on the GPU, or of
8-bit E4M3 codes (uint8 or float8_e4m3fn) for the *_fp8 calls.
"""

import ctypes
import os

import numpy as np
import torch

__all__ = [
    "PkvError", "InvalidArgument", "OutOfBlocks", "NoSuchSequence",
    "SequenceExists", "BufferTooSmall", "HipError", "Unsupported",
    "BlockAllocator", "Scheduler", "StepPlan", "DecodeLauncher", "paged_kv_append", "copy_blocks",
    "paged_attention_decode_workspace_size", "paged_attention_decode_partition_size",
    "paged_attention_decode", "paged_attention_decode_append",
    "paged_attention_decode_append_partials", "paged_attention_decode_step",
    "paged_attention_decode_step_mapped",
    "paged_attention_decode_partials", "paged_attention_decode_merge",
    "paged_attention_prefill", "paged_attention_prefill_fp8", "paged_kv_append_fp8",
    "paged_attention_decode_fp8",
    "paged_attention_decode_fp8_partials", "paged_attention_decode_fp8_step",
    "paged_attention_decode_shared_prefix",
    "paged_attention_decode_shared_prefix_step",
    "paged_attention_decode_shared_prefix_workspace_size",
    "paged_attention_decode_grouped_prefix", "paged_attention_decode_grouped_prefix_step",
    "paged_attention_decode_grouped_prefix_workspace_size", "paged_attention_decode_noalloc",
    "stream_read", "matrix_loop", "swap_blocks", "library_path", "version",
]

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")


class PkvError(RuntimeError):
    """Base class of errors reported by libpkv."""


class InvalidArgument(PkvError, ValueError):
    pass


class OutOfBlocks(PkvError):
    """The block pool is exhausted; the allocator state is unchanged."""


class NoSuchSequence(PkvError, KeyError):
    pass


class SequenceExists(PkvError, ValueError):
    pass


class BufferTooSmall(PkvError, ValueError):
    pass


class HipError(PkvError):
    pass


class Unsupported(PkvError, NotImplementedError):
    pass


_ERRORS = {1: InvalidArgument, 2: OutOfBlocks, 3: NoSuchSequence,
           4: SequenceExists, 5: BufferTooSmall, 6: HipError, 7: Unsupported}

_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_P = ctypes.c_void_p
_PI32 = ctypes.POINTER(ctypes.c_int32)
_PI64 = ctypes.POINTER(ctypes.c_int64)

_SIGNATURES = {
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_version": (ctypes.c_char_p, []),
    "pkv_allocator_create": (_I32, [_I32, _I32, _P, ctypes.POINTER(_P)]),
    "pkv_allocator_destroy": (None, [_P]),
    "pkv_seq_add": (_I32, [_P, _I64]),
    "pkv_seq_free": (_I32, [_P, _I64]),
    "pkv_seq_fork": (_I32, [_P, _I64, _I64]),
    "pkv_seq_append": (_I32, [_P, _I64, _I32, _P, _P, _P, _P]),
    "pkv_append_batch": (_I32, [_P, _P, _P, _I32, _P, _I64, _P, _P, _I32, _P]),
    "pkv_append_batch_tables": (_I32, [_P, _P, _P, _I32, _P, _I64, _P, _P, _I32, _P,
                                       _I32, _P, _P]),
    "pkv_append_batch_changes": (_I32, [_P, _P, _P, _I32, _P, _I64, _P, _P, _I32, _P, _P, _P, _I32,
                                        _P]),
    "pkv_paged_attention_decode_step": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32,
                                               _I32, _I32, _I32, _I32, _I32, ctypes.c_float, _I32,
                                               _P, _P, ctypes.c_size_t, _I32, _P]),
    "pkv_paged_attention_decode_step_mapped": (
        _I32, [_P, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32,
               _I32, _I32, _I32, ctypes.c_float, _I32, _P, _P, ctypes.c_size_t, _I32, _P]),
    "pkv_paged_attention_decode_step_partials": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32,
                                                        _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                                        ctypes.c_float, _I32, _P, _P,
                                                        ctypes.c_size_t, _I32, _P]),
    "pkv_paged_attention_decode_step_merge": (_I32, [_P, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                                     _I32, _P, _P, ctypes.c_size_t, _P]),
    "pkv_seq_len": (_I32, [_P, _I64, _P]),
    "pkv_seq_block_table": (_I32, [_P, _I64, _P, _I32, _P]),
    "pkv_num_free_blocks": (_I32, [_P, _P]),
    "pkv_num_blocks": (_I32, [_P, _P]),
    "pkv_block_size": (_I32, [_P, _P]),
    "pkv_block_refcount": (_I32, [_P, _I32, _P]),
    "pkv_allocator_snapshot": (_I32, [_P, _P, _P, _P]),
    "pkv_allocator_set_host_pool": (_I32, [_P, _I32]),
    "pkv_num_free_host_blocks": (_I32, [_P, _P]),
    "pkv_seq_is_swapped": (_I32, [_P, _I64, _P]),
    "pkv_seq_swap_out": (_I32, [_P, _I64, _P, _P, _I32, _P]),
    "pkv_seq_swap_in": (_I32, [_P, _I64, _P, _P, _I32, _P]),
    "pkv_allocator_host_snapshot": (_I32, [_P, _P, _P]),
    "pkv_swap_blocks": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I64, _P]),
    "pkv_build_block_tables": (_I32, [_P, _P, _I32, _I32, _P, _P]),
    "pkv_paged_kv_append": (_I32, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _P]),
    "pkv_copy_blocks": (_I32, [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _P]),
    "pkv_paged_attention_decode_partition_size": (_I32, [_I32, _I32, _I32, _I32, _I32, _P]),
    "pkv_paged_attention_decode_workspace_size": (_I32, [_I32, _I32, _I32, _I32, _I32, _I32,
                                                         ctypes.POINTER(ctypes.c_size_t)]),
    "pkv_paged_attention_decode": (_I32, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                          ctypes.c_float, _I32, _P, _P, ctypes.c_size_t, _I32, _P]),
    "pkv_paged_attention_decode_append": (_I32, [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                                 _I32, _I32, _I32, ctypes.c_float, _I32, _P, _P,
                                                 ctypes.c_size_t, _I32, _P]),
    "pkv_paged_attention_decode_append_partials": (_I32, [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32,
                                                          _I32, _I32, _I32, _I32, _I32, ctypes.c_float,
                                                          _I32, _P, _P, ctypes.c_size_t, _I32, _P]),
    "pkv_paged_attention_decode_partials": (_I32, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                                   _I32, ctypes.c_float, _I32, _P, _P, ctypes.c_size_t, _I32, _P]),
    "pkv_paged_attention_decode_merge": (_I32, [_P, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P,
                                                ctypes.c_size_t, _P]),
    "pkv_stream_read": (_I32, [_P, _I64, _I32, _P, _P]),
    "pkv_matrix_loop": (_I32, [_I32, _I32, _P, _P]),
    "pkv_paged_attention_decode_noalloc": (_I32, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                                  _I32, _I32, _I32, ctypes.c_float, _I32, _P, _I32,
                                                  _P]),
    "pkv_paged_kv_append_fp8": (_I32, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                       ctypes.c_float, ctypes.c_float, _I32, _P]),
    "pkv_paged_attention_decode_fp8": (_I32, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                              _I32, _I32, ctypes.c_float, ctypes.c_float,
                                              ctypes.c_float, _I32, _P, _P, ctypes.c_size_t, _I32,
                                              _P]),
    "pkv_paged_attention_decode_fp8_partials": (_I32, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32,
                                                       _I32, _I32, _I32, _I32, ctypes.c_float,
                                                       ctypes.c_float, ctypes.c_float, _I32, _P,
                                                       _P, ctypes.c_size_t, _I32, _P]),
    "pkv_paged_attention_decode_fp8_step": (
        _I32, [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
               _I32, ctypes.c_float, ctypes.c_float, ctypes.c_float, _I32, _P, _P,
               ctypes.c_size_t, _I32, _P]),
    "pkv_paged_attention_decode_shared_prefix_workspace_size": (
        _I32, [_I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32, ctypes.POINTER(ctypes.c_size_t)]),
    "pkv_paged_attention_decode_shared_prefix": (_I32, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32,
                                                        _I32, _I32, _I32, _I32, _I32,
                                                        ctypes.c_float, _I32, _P, _P,
                                                        ctypes.c_size_t, _I32, _P]),
    "pkv_paged_attention_decode_shared_prefix_step": (
        _I32, [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
               _I32, _I32, ctypes.c_float, _I32, _P, _P, ctypes.c_size_t, _I32, _P]),
    "pkv_paged_attention_decode_grouped_prefix_workspace_size": (
        _I32, [_I32, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _I32,
               ctypes.POINTER(ctypes.c_size_t)]),
    "pkv_paged_attention_decode_grouped_prefix": (
        _I32, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P,
               ctypes.c_float, _I32, _P, _P, ctypes.c_size_t, _I32, _P]),
    "pkv_paged_attention_decode_grouped_prefix_step": (
        _I32, [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
               _I32, _I32, _P, _P, ctypes.c_float, _I32, _P, _P, ctypes.c_size_t, _I32, _P]),
    "pkv_scheduler_create": (_I32, [_I32, _I32, _P, _I32, _I32, _I32, _I32, _I32,
                                    ctypes.POINTER(_P)]),
    "pkv_scheduler_last_swaps": (_I32, [_P, _P, _P, _I32, _P, _P, _P, _I32, _P]),
    "pkv_scheduler_destroy": (None, [_P]),
    "pkv_scheduler_add_request": (_I32, [_P, _I64, _I32, _I32]),
    "pkv_scheduler_max_blocks": (_I32, [_P, _P]),
    "pkv_scheduler_step": (_I32, [_P, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P]),
    "pkv_scheduler_last_events": (_I32, [_P, _P, _I32, _P, _P, _I32, _P]),
    "pkv_scheduler_stats": (_I32, [_P, _P]),
    "pkv_paged_attention_prefill": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                           _I32, ctypes.c_float, _P, _I32, _P]),
    "pkv_paged_attention_prefill_fp8": (
        _I32, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
               ctypes.c_float, ctypes.c_float, ctypes.c_float, _P, _I32, _P]),
}


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is not built; run `python paged_kv_cache_420_amd/_build.py` "
            "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(_LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def library_path():
    return _LIB_PATH


def version():
    return _lib.pkv_version().decode()


def _check(status):
    if status != 0:
        msg = _lib.pkv_last_error().decode()
        raise _ERRORS.get(status, PkvError)(msg or f"libpkv status {status}")


def _i32p(arr):
    return arr.ctypes.data


# ---------------------------------------------------------------------------
# Host block allocator
# ---------------------------------------------------------------------------

class BlockAllocator:
    """Handle on a pkv_allocator (free stack, refcounts, block tables).

    Semantics are those of include/pkv.h: blocks on demand, LIFO free stack
    seeded by ``init_free_order``, refcounted fork, copy-on-write pair
    reported by append, release in logical order, all-or-nothing failure.
    """

    def __init__(self, num_blocks, block_size, init_free_order=None):
        handle = _P()
        order = None
        if init_free_order is not None:
            order = np.ascontiguousarray(np.asarray(init_free_order, dtype=np.int32))
            if order.shape != (num_blocks,):
                raise InvalidArgument("init_free_order must hold num_blocks entries")
        _check(_lib.pkv_allocator_create(num_blocks, block_size,
                                         _i32p(order) if order is not None else None,
                                         ctypes.byref(handle)))
        self._h = handle
        self._cow = None
        self.num_blocks = num_blocks
        self.block_size = block_size

    def close(self):
        # at interpreter shutdown the module globals may already be gone
        if getattr(self, "_h", None) and _lib is not None:
            _lib.pkv_allocator_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def add(self, seq):
        _check(_lib.pkv_seq_add(self._h, seq))

    def free(self, seq):
        _check(_lib.pkv_seq_free(self._h, seq))

    def fork(self, parent, child):
        _check(_lib.pkv_seq_fork(self._h, parent, child))

    def append(self, seq, n):
        """Returns (slots: int32 array [n], cow: list of (src, dst))."""
        slots = np.empty(max(n, 1), dtype=np.int32)
        src, dst, cnt = _I32(), _I32(), _I32()
        _check(_lib.pkv_seq_append(self._h, seq, n, _i32p(slots), ctypes.byref(src),
                                   ctypes.byref(dst), ctypes.byref(cnt)))
        return slots[:n], ([(src.value, dst.value)] if cnt.value else [])

    def append_batch(self, seqs, counts, slots_out=None):
        """All-or-nothing append; returns (slots int32 [sum counts], cow pairs).
        ``slots_out``: optional contiguous int32 array to write the slots into
        (a view of it is returned)."""
        seqs = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        counts = np.ascontiguousarray(np.asarray(counts, dtype=np.int32))
        if seqs.shape != counts.shape:
            raise InvalidArgument("seqs and counts differ in length")
        total = int(counts.astype(np.int64).sum())
        if slots_out is None:
            slots = np.empty(max(total, 1), dtype=np.int32)
        else:
            slots = slots_out
            if (slots.dtype != np.int32 or slots.ndim != 1 or not slots.flags.c_contiguous
                    or slots.shape[0] < total):
                raise InvalidArgument("slots_out must be a contiguous int32 array of sum(counts)")
        cap = max(len(seqs), 1)
        src = np.empty(cap, dtype=np.int32)
        dst = np.empty(cap, dtype=np.int32)
        cnt = _I32()
        _check(_lib.pkv_append_batch(self._h, seqs.ctypes.data, _i32p(counts), len(seqs),
                                     _i32p(slots), total, _i32p(src), _i32p(dst), len(seqs),
                                     ctypes.byref(cnt)))
        return slots[:total], list(zip(src[:cnt.value].tolist(), dst[:cnt.value].tolist()))

    def append_batch_tables(self, seqs, counts, max_blocks, slots_out=None, tables_out=None,
                            lens_out=None):
        """append_batch, then the batch's updated tables [B, max_blocks] and
        lengths [B] (pkv_append_batch_tables): all in one call, all or
        nothing.  Outputs may be given as contiguous int32 arrays (e.g. views
        of a pinned staging buffer).  Returns (slots, cow pairs, tables, lens)."""
        seqs = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        counts = np.ascontiguousarray(np.asarray(counts, dtype=np.int32))
        b = len(seqs)
        if counts.shape != seqs.shape:
            raise InvalidArgument("seqs and counts differ in length")
        total = int(counts.sum(dtype=np.int64))

        def out(arr, shape):
            if arr is None:
                return np.empty(shape, dtype=np.int32)
            if arr.dtype != np.int32 or arr.shape != shape or not arr.flags.c_contiguous:
                raise InvalidArgument(f"output must be a contiguous int32 array of shape {shape}")
            return arr

        slots = out(slots_out, (total,))
        tables = out(tables_out, (b, max_blocks))
        lens = out(lens_out, (b,))
        cap = max(b, 1)
        if self._cow is None or len(self._cow[0]) < cap:
            self._cow = (np.empty(cap, dtype=np.int32), np.empty(cap, dtype=np.int32))
        src, dst = self._cow
        cnt = _I32()
        _check(_lib.pkv_append_batch_tables(
            self._h, seqs.ctypes.data, counts.ctypes.data, b,
            slots.ctypes.data, total, src.ctypes.data,
            dst.ctypes.data, b, ctypes.byref(cnt), max_blocks,
            tables.ctypes.data, lens.ctypes.data))
        pairs = list(zip(src[:cnt.value].tolist(), dst[:cnt.value].tolist()))
        return slots, pairs, tables, lens

    def prepared_append_tables(self, seqs, counts, max_blocks, slots_out, tables_out, lens_out):
        """append_batch_tables with every argument marshalled once, for a
        loop that appends the same counts to the same sequences into the
        same (e.g. pinned staging) arrays each step.  Returns a function
        that makes the call and returns the copy-on-write pairs."""
        seqs = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        counts = np.ascontiguousarray(np.asarray(counts, dtype=np.int32))
        b = len(seqs)
        total = int(counts.sum(dtype=np.int64))
        for arr, shape in ((slots_out, (total,)), (tables_out, (b, max_blocks)), (lens_out, (b,))):
            if arr.dtype != np.int32 or arr.shape != shape or not arr.flags.c_contiguous:
                raise InvalidArgument(f"output must be a contiguous int32 array of shape {shape}")
        src = np.empty(max(b, 1), dtype=np.int32)
        dst = np.empty(max(b, 1), dtype=np.int32)
        cnt = _I32()
        keep = (seqs, counts, slots_out, tables_out, lens_out, src, dst, cnt)
        args = (self._h, seqs.ctypes.data, counts.ctypes.data, b, slots_out.ctypes.data, total,
                src.ctypes.data, dst.ctypes.data, b, ctypes.byref(cnt), max_blocks,
                tables_out.ctypes.data, lens_out.ctypes.data)
        fn = _lib.pkv_append_batch_tables

        def call(_keep=keep):
            _check(fn(*args))
            k = cnt.value
            return list(zip(src[:k].tolist(), dst[:k].tolist())) if k else []
        return call

    def append_batch_changes(self, seqs, counts):
        """append_batch, reporting the table entries it set and the lengths
        (pkv_append_batch_changes).  Returns (slots, cow pairs, lens [B],
        changes [n, 3] int32 rows of (batch row, logical block, block))."""
        seqs = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        counts = np.ascontiguousarray(np.asarray(counts, dtype=np.int32))
        b = len(seqs)
        if counts.shape != seqs.shape:
            raise InvalidArgument("seqs and counts differ in length")
        total = int(counts.sum(dtype=np.int64))
        cap = int(np.sum(-(-counts.astype(np.int64) // self.block_size))) + b + 1
        slots = np.empty(max(total, 1), dtype=np.int32)
        lens = np.empty(max(b, 1), dtype=np.int32)
        changes = np.empty((cap, 3), dtype=np.int32)
        src = np.empty(max(b, 1), dtype=np.int32)
        dst = np.empty(max(b, 1), dtype=np.int32)
        ncow, nch = _I32(), _I32()
        _check(_lib.pkv_append_batch_changes(
            self._h, seqs.ctypes.data, counts.ctypes.data, b, slots.ctypes.data, total,
            src.ctypes.data, dst.ctypes.data, b, ctypes.byref(ncow), lens.ctypes.data,
            changes.ctypes.data, cap, ctypes.byref(nch)))
        pairs = list(zip(src[:ncow.value].tolist(), dst[:ncow.value].tolist()))
        return slots[:total], pairs, lens[:b], changes[:nch.value]

    def prepared_append_changes(self, seqs, counts, slots_out, lens_out, changes_out):
        """append_batch_changes with every argument marshalled once, into
        the given contiguous int32 arrays (changes_out [cap, 3]).  Returns a
        function that makes the call and returns (cow pairs, number of
        changes)."""
        seqs = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        counts = np.ascontiguousarray(np.asarray(counts, dtype=np.int32))
        b = len(seqs)
        total = int(counts.sum(dtype=np.int64))
        for arr, nd in ((slots_out, 1), (lens_out, 1), (changes_out, 2)):
            if arr.dtype != np.int32 or arr.ndim != nd or not arr.flags.c_contiguous:
                raise InvalidArgument("outputs must be contiguous int32 arrays")
        if slots_out.shape[0] < total or lens_out.shape[0] < b or changes_out.shape[1] != 3:
            raise InvalidArgument("output arrays too small")
        src = np.empty(max(b, 1), dtype=np.int32)
        dst = np.empty(max(b, 1), dtype=np.int32)
        ncow, nch = _I32(), _I32()
        keep = (seqs, counts, slots_out, lens_out, changes_out, src, dst, ncow, nch)
        args = (self._h, seqs.ctypes.data, counts.ctypes.data, b, slots_out.ctypes.data, total,
                src.ctypes.data, dst.ctypes.data, b, ctypes.byref(ncow), lens_out.ctypes.data,
                changes_out.ctypes.data, changes_out.shape[0], ctypes.byref(nch))
        fn = _lib.pkv_append_batch_changes

        def call(_keep=keep):
            _check(fn(*args))
            k = ncow.value
            pairs = list(zip(src[:k].tolist(), dst[:k].tolist())) if k else []
            return pairs, nch.value
        return call

    def seq_len(self, seq):
        out = _I32()
        _check(_lib.pkv_seq_len(self._h, seq, ctypes.byref(out)))
        return out.value

    def block_table(self, seq):
        n = _I32()
        st = _lib.pkv_seq_block_table(self._h, seq, None, 0, ctypes.byref(n))
        if st not in (0, 5):
            _check(st)
        buf = np.empty(max(n.value, 1), dtype=np.int32)
        _check(_lib.pkv_seq_block_table(self._h, seq, _i32p(buf), n.value, ctypes.byref(n)))
        return buf[:n.value].tolist()

    def num_free(self):
        out = _I32()
        _check(_lib.pkv_num_free_blocks(self._h, ctypes.byref(out)))
        return out.value

    def refcount(self, block):
        out = _I32()
        _check(_lib.pkv_block_refcount(self._h, block, ctypes.byref(out)))
        return out.value

    def snapshot(self):
        """(free stack top first, refcounts) as lists."""
        free = np.empty(self.num_blocks, dtype=np.int32)
        ref = np.empty(self.num_blocks, dtype=np.int32)
        nf = _I32()
        _check(_lib.pkv_allocator_snapshot(self._h, _i32p(free), ctypes.byref(nf), _i32p(ref)))
        return free[:nf.value].tolist(), ref.tolist()

    # -- swap space (pkv_allocator_set_host_pool, pkv_seq_swap_out/in) -----
    def set_host_pool(self, num_host_blocks):
        _check(_lib.pkv_allocator_set_host_pool(self._h, int(num_host_blocks)))
        self.num_host_blocks = int(num_host_blocks)

    def num_free_host(self):
        out = _I32()
        _check(_lib.pkv_num_free_host_blocks(self._h, ctypes.byref(out)))
        return out.value

    def is_swapped(self, seq):
        out = _I32()
        _check(_lib.pkv_seq_is_swapped(self._h, int(seq), ctypes.byref(out)))
        return bool(out.value)

    def _swap(self, fn, seq):
        cap = max(1, self.num_blocks, getattr(self, "num_host_blocks", 0))
        a = np.empty(cap, dtype=np.int32)
        b = np.empty(cap, dtype=np.int32)
        n = _I32()
        _check(fn(self._h, int(seq), _i32p(a), _i32p(b), cap, ctypes.byref(n)))
        return np.stack([a[:n.value], b[:n.value]], axis=1)

    def swap_out(self, seq):
        """Move seq to the host tier; returns int32 pairs [n, 2] (device, host)."""
        return self._swap(_lib.pkv_seq_swap_out, seq)

    def swap_in(self, seq):
        """Back to device blocks; returns int32 pairs [n, 2] (host, device)."""
        return self._swap(_lib.pkv_seq_swap_in, seq)

    def host_snapshot(self):
        """Free host blocks, top of the stack first."""
        out = np.empty(max(1, getattr(self, "num_host_blocks", 0)), dtype=np.int32)
        n = _I32()
        _check(_lib.pkv_allocator_host_snapshot(self._h, _i32p(out), ctypes.byref(n)))
        return out[:n.value].tolist()

    def build_block_tables(self, seqs, max_blocks, tables_out=None, lens_out=None):
        """Host int32 arrays (block_tables [B, max_blocks] -1 padded, context_lens [B]).
        ``tables_out``/``lens_out``: optional contiguous int32 arrays of those
        shapes to fill instead (e.g. views of a pinned staging buffer)."""
        seqs = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        b = len(seqs)
        if tables_out is None or lens_out is None:
            tables = np.empty((max(b, 1), max(max_blocks, 1)), dtype=np.int32)
            lens = np.empty(max(b, 1), dtype=np.int32)
        else:
            tables, lens = tables_out, lens_out
            if (tables.dtype != np.int32 or tables.shape != (b, max_blocks)
                    or not tables.flags.c_contiguous or lens.dtype != np.int32
                    or lens.shape != (b,) or not lens.flags.c_contiguous):
                raise InvalidArgument("tables_out/lens_out must be contiguous int32 "
                                      "[B, max_blocks] and [B]")
        _check(_lib.pkv_build_block_tables(self._h, seqs.ctypes.data, b, max_blocks,
                                           _i32p(tables), _i32p(lens)))
        return tables[:b, :max_blocks], lens[:b]


class StepPlan:
    """One scheduler step: rows [0, num_decode) are decode rows, the rest
    prefill chunks.  Arrays are views of the scheduler's buffers, valid until
    its next step."""

    def __init__(self, seq_ids, query_lens, context_lens, slots, block_tables, num_decode,
                 finished, preempted, swap_in=None, swap_out=None):
        self.seq_ids = seq_ids
        self.query_lens = query_lens
        self.context_lens = context_lens
        self.slots = slots
        self.block_tables = block_tables
        self.num_decode = num_decode
        self.finished = finished
        self.preempted = preempted
        # int32 [n, 2]: (host, device) block pairs to copy in, (device, host) out
        self.swap_in = np.zeros((0, 2), np.int32) if swap_in is None else swap_in
        self.swap_out = np.zeros((0, 2), np.int32) if swap_out is None else swap_out

    @property
    def num_rows(self):
        return len(self.seq_ids)

    @property
    def num_prefill(self):
        return self.num_rows - self.num_decode

    @property
    def num_tokens(self):
        return len(self.slots)


_STAT_NAMES = ("steps", "running", "waiting", "finished", "preemptions", "cached_tokens",
               "allocated_slots", "reserved_slots", "free_blocks", "swapped_out", "swapped_in")


class Scheduler:
    """Continuous-batching step scheduler (pkv_scheduler_*; policy in pkv.h)."""

    def __init__(self, num_blocks, block_size, max_num_seqs, max_num_batched_tokens, chunk_size,
                 reserve_tokens=0, init_free_order=None, host_blocks=0):
        self._h = _P()
        order = None
        if init_free_order is not None:
            order = np.ascontiguousarray(init_free_order, dtype=np.int32)
            if order.shape != (num_blocks,):
                raise InvalidArgument("init_free_order must hold num_blocks entries")
        _check(_lib.pkv_scheduler_create(num_blocks, block_size,
                                         None if order is None else order.ctypes.data,
                                         max_num_seqs, max_num_batched_tokens, chunk_size,
                                         reserve_tokens, host_blocks, ctypes.byref(self._h)))
        self.num_blocks, self.host_blocks = num_blocks, host_blocks
        cap = max(1, num_blocks, host_blocks)
        self._swaps = [np.empty(cap, dtype=np.int32) for _ in range(4)]
        self.max_num_seqs = max_num_seqs
        self.max_num_batched_tokens = max_num_batched_tokens
        self._ids = np.empty(max_num_seqs, dtype=np.int64)
        self._qlen = np.empty(max_num_seqs, dtype=np.int32)
        self._ctx = np.empty(max_num_seqs, dtype=np.int32)
        self._slots = np.empty(max_num_batched_tokens, dtype=np.int32)
        self._fin = np.empty(max_num_seqs, dtype=np.int64)
        self._pre = np.empty(max_num_seqs, dtype=np.int64)
        self._tables = np.empty(0, dtype=np.int32)
        self._counts = np.empty(3, dtype=np.int32)
        self._stats = np.empty(11, dtype=np.int64)

    def close(self):
        if getattr(self, "_h", None) and _lib is not None:
            _lib.pkv_scheduler_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def add_request(self, rid, prompt_len, output_len):
        _check(_lib.pkv_scheduler_add_request(self._h, int(rid), int(prompt_len),
                                              int(output_len)))

    def max_blocks(self):
        out = _I32()
        _check(_lib.pkv_scheduler_max_blocks(self._h, ctypes.byref(out)))
        return out.value

    def step(self, max_blocks=None):
        """Run one step; returns a StepPlan (block_tables [rows, max_blocks])."""
        mb = self.max_blocks() if max_blocks is None else int(max_blocks)
        if self._tables.size < self.max_num_seqs * mb:
            self._tables = np.empty(self.max_num_seqs * mb, dtype=np.int32)
        c = self._counts
        _check(_lib.pkv_scheduler_step(self._h, self.max_num_seqs, self.max_num_batched_tokens, mb,
                                       self._ids.ctypes.data, self._qlen.ctypes.data,
                                       self._ctx.ctypes.data, self._slots.ctypes.data,
                                       self._tables.ctypes.data, c[0:].ctypes.data,
                                       c[1:].ctypes.data, c[2:].ctypes.data))
        nd, nr, nt = int(c[0]), int(c[1]), int(c[2])
        nf, npre = _I32(), _I32()
        _check(_lib.pkv_scheduler_last_events(self._h, self._fin.ctypes.data, len(self._fin),
                                              ctypes.byref(nf), self._pre.ctypes.data,
                                              len(self._pre), ctypes.byref(npre)))
        tables = self._tables[:self.max_num_seqs * mb].reshape(self.max_num_seqs, mb)[:nr]
        ih, idv, od, oh = self._swaps
        ni, no = _I32(), _I32()
        _check(_lib.pkv_scheduler_last_swaps(self._h, ih.ctypes.data, idv.ctypes.data, len(ih),
                                             ctypes.byref(ni), od.ctypes.data, oh.ctypes.data,
                                             len(od), ctypes.byref(no)))
        swap_in = np.stack([ih[:ni.value], idv[:ni.value]], axis=1)
        swap_out = np.stack([od[:no.value], oh[:no.value]], axis=1)
        return StepPlan(self._ids[:nr], self._qlen[:nr], self._ctx[:nr], self._slots[:nt], tables,
                        nd, self._fin[:nf.value].tolist(), self._pre[:npre.value].tolist(),
                        swap_in, swap_out)

    def stats(self):
        _check(_lib.pkv_scheduler_stats(self._h, self._stats.ctypes.data))
        return dict(zip(_STAT_NAMES, (int(x) for x in self._stats)))


# ---------------------------------------------------------------------------
# Device calls
# ---------------------------------------------------------------------------

_DTYPES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
# 8-bit caches hold E4M3 codes; a uint8 tensor or torch's float8_e4m3fn
# (the same bytes) is accepted.
_FP8_CODE = 3
_FP8_TYPES = (torch.uint8, torch.float8_e4m3fn)


# pkv.h PKV_DECODE_SHARED_BLOCKS: OR'd into a decode call's dtype when
# blocks are shared by several sequences of the batch (cached K/V loads
# instead of streaming ones; results are unchanged)
DECODE_SHARED_BLOCKS = 0x100


def _decode_code(t, shared_blocks):
    return _dtype_code(t) | (DECODE_SHARED_BLOCKS if shared_blocks else 0)


def _dtype_code(t):
    if t.dtype in _FP8_TYPES:
        return _FP8_CODE
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise InvalidArgument(f"unsupported dtype {t.dtype}") from None


def _dev(t, name, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise InvalidArgument(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise InvalidArgument(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise InvalidArgument(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise InvalidArgument(f"{name} must have {ndim} dimensions")
    return t.data_ptr()


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _cache_dims(key_cache, value_cache):
    _dev(key_cache, "key_cache", ndim=4)
    _dev(value_cache, "value_cache", dtype=key_cache.dtype, ndim=4)
    if key_cache.shape != value_cache.shape:
        raise InvalidArgument("key_cache and value_cache differ in shape")
    return tuple(key_cache.shape)  # (num_blocks, num_kv_heads, block_size, head_dim)


def paged_kv_append(key, value, key_cache, value_cache, slot_mapping):
    """Scatter key/value [T, Hkv, D] into the caches at int32 slot_mapping [T]
    (negative slot = skip).  pkv_paged_kv_append."""
    nb, hkv, bs, d = _cache_dims(key_cache, value_cache)
    _dev(key, "key", dtype=key_cache.dtype, ndim=3)
    _dev(value, "value", dtype=key_cache.dtype, ndim=3)
    _dev(slot_mapping, "slot_mapping", dtype=torch.int32, ndim=1)
    t = key.shape[0]
    if key.shape != (t, hkv, d) or value.shape != key.shape or slot_mapping.shape[0] != t:
        raise InvalidArgument("key/value must be [T, num_kv_heads, head_dim] with T slots")
    _check(_lib.pkv_paged_kv_append(key.data_ptr(), value.data_ptr(), key_cache.data_ptr(),
                                    value_cache.data_ptr(), slot_mapping.data_ptr(), t, hkv, d, bs,
                                    nb, _dtype_code(key_cache), _stream(key_cache)))


def copy_blocks(key_cache, value_cache, src, dst):
    """Block dst[i] := block src[i] in both caches (int32 GPU tensors).
    pkv_copy_blocks."""
    nb, hkv, bs, d = _cache_dims(key_cache, value_cache)
    _dev(src, "src", dtype=torch.int32, ndim=1)
    _dev(dst, "dst", dtype=torch.int32, ndim=1)
    if src.shape != dst.shape:
        raise InvalidArgument("src and dst differ in length")
    _check(_lib.pkv_copy_blocks(key_cache.data_ptr(), value_cache.data_ptr(), src.data_ptr(),
                                dst.data_ptr(), src.shape[0], nb, hkv, bs, d,
                                _dtype_code(key_cache), _stream(key_cache)))


def swap_blocks(src_key_cache, src_value_cache, dst_key_cache, dst_value_cache, src_blocks,
                dst_blocks):
    """Block dst_blocks[i] of the destination caches := block src_blocks[i]
    of the source caches (pkv_swap_blocks).  Caches of one shape per side
    ([blocks, Hkv, block_size, D], same dtype), each on the GPU or in pinned
    host memory; block ids are host arrays.  Enqueued on the current
    stream of the GPU side."""
    for t, name in ((src_key_cache, "src_key_cache"), (src_value_cache, "src_value_cache"),
                    (dst_key_cache, "dst_key_cache"), (dst_value_cache, "dst_value_cache")):
        if not isinstance(t, torch.Tensor) or t.dim() != 4 or not t.is_contiguous():
            raise InvalidArgument(f"{name} must be a contiguous 4-d tensor")
        if not t.is_cuda and not t.is_pinned():
            raise InvalidArgument(f"{name} must be on the GPU or in pinned host memory")
    if src_key_cache.shape[1:] != dst_key_cache.shape[1:] or \
            src_key_cache.dtype != dst_key_cache.dtype or \
            src_value_cache.shape != src_key_cache.shape or \
            dst_value_cache.shape != dst_key_cache.shape:
        raise InvalidArgument("source and destination pools differ in block layout")
    src = np.ascontiguousarray(src_blocks, dtype=np.int32).reshape(-1)
    dst = np.ascontiguousarray(dst_blocks, dtype=np.int32).reshape(-1)
    if src.shape != dst.shape:
        raise InvalidArgument("src_blocks and dst_blocks differ in length")
    gpu = dst_key_cache if dst_key_cache.is_cuda else src_key_cache
    block_bytes = src_key_cache[0].numel() * src_key_cache.element_size()
    _check(_lib.pkv_swap_blocks(src_key_cache.data_ptr(), src_value_cache.data_ptr(),
                                dst_key_cache.data_ptr(), dst_value_cache.data_ptr(), _i32p(src),
                                _i32p(dst), len(src), src_key_cache.shape[0],
                                dst_key_cache.shape[0], block_bytes, _stream(gpu)))


def paged_attention_decode_partition_size(num_seqs, num_kv_heads, block_size, max_context_len,
                                          partition_size=0):
    """Split-K partition (tokens) the decode call uses for these sizes."""
    out = _I32()
    _check(_lib.pkv_paged_attention_decode_partition_size(num_seqs, num_kv_heads, block_size,
                                                          max_context_len, partition_size,
                                                          ctypes.byref(out)))
    return out.value


def paged_attention_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim,
                                          max_context_len, partition_size=0):
    """Bytes of workspace pkv_paged_attention_decode needs for these sizes."""
    out = ctypes.c_size_t()
    _check(_lib.pkv_paged_attention_decode_workspace_size(num_seqs, num_heads, num_kv_heads,
                                                          head_dim, max_context_len,
                                                          partition_size, ctypes.byref(out)))
    return out.value


def _decode_args(query, key_cache, value_cache, block_tables, context_lens, max_context_len,
                 partition_size, out, workspace, fp8=False, mapped=False):
    nb, hkv, bs, d = _cache_dims(key_cache, value_cache)
    if fp8:
        if key_cache.dtype not in _FP8_TYPES:
            raise InvalidArgument("an 8-bit cache must be uint8 or float8_e4m3fn")
        _dev(query, "query", ndim=3)
        if query.dtype not in (torch.bfloat16, torch.float16):
            raise InvalidArgument("the query of an 8-bit cache must be bfloat16 or float16")
    else:
        _dev(query, "query", dtype=key_cache.dtype, ndim=3)
    _dev(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    b, hq, dq = query.shape
    if context_lens is not None:  # None: host lengths, checked by the caller
        _dev(context_lens, "context_lens", dtype=torch.int32, ndim=1)
        if context_lens.shape[0] != b:
            raise InvalidArgument("query and context_lens disagree on shape")
    if dq != d or (block_tables.shape[0] != b and not mapped):
        raise InvalidArgument("query and block_tables disagree on shape")
    if out is None:
        out = torch.empty((b, hq, d), dtype=torch.float32, device=query.device)
    _dev(out, "out", dtype=torch.float32, ndim=3)
    if tuple(out.shape) != (b, hq, d):
        raise InvalidArgument("out must be [B, Hq, D]")
    need = paged_attention_decode_workspace_size(b, hq, hkv, d, int(max_context_len),
                                                 partition_size)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=query.device)
    ws_ptr, ws_bytes = (None, 0)
    if workspace is not None:
        _dev(workspace, "workspace")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    return (nb, hkv, bs, d, b, hq), out, workspace, ws_ptr, ws_bytes


def paged_attention_decode(query, key_cache, value_cache, block_tables, context_lens, scale,
                           max_context_len, partition_size=0, out=None, workspace=None,
                           shared_blocks=False):
    """Decode attention (pkv_paged_attention_decode).

    query [B, Hq, D] (cache dtype); block_tables [B, max_blocks] int32;
    context_lens [B] int32; returns out [B, Hq, D] float32.
    ``max_context_len`` is a host-side bound on context_lens (sizes the grid).
    ``shared_blocks``: some blocks are shared by several sequences of the
    batch (PKV_DECODE_SHARED_BLOCKS; same result, cached loads).
    """
    (nb, hkv, bs, d, b, hq), out, workspace, ws_ptr, ws_bytes = _decode_args(
        query, key_cache, value_cache, block_tables, context_lens, max_context_len,
        partition_size, out, workspace)
    _check(_lib.pkv_paged_attention_decode(
        query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(), block_tables.data_ptr(),
        context_lens.data_ptr(), b, hq, hkv, d, bs, block_tables.shape[1], nb,
        int(max_context_len), float(scale), int(partition_size), out.data_ptr(), ws_ptr, ws_bytes,
        _decode_code(key_cache, shared_blocks), _stream(query)))
    return out


def _decode_append(fn, query, key, value, key_cache, value_cache, block_tables, context_lens,
                   scale, max_context_len, partition_size, out, workspace):
    (nb, hkv, bs, d, b, hq), out, workspace, ws_ptr, ws_bytes = _decode_args(
        query, key_cache, value_cache, block_tables, context_lens, max_context_len,
        partition_size, out, workspace)
    _dev(key, "key", dtype=key_cache.dtype, ndim=3)
    _dev(value, "value", dtype=key_cache.dtype, ndim=3)
    if tuple(key.shape) != (b, hkv, d) or value.shape != key.shape:
        raise InvalidArgument("key/value must be [B, num_kv_heads, head_dim]")
    _check(fn(query.data_ptr(), key.data_ptr(), value.data_ptr(), key_cache.data_ptr(),
              value_cache.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(), b, hq,
              hkv, d, bs, block_tables.shape[1], nb, int(max_context_len), float(scale),
              int(partition_size), out.data_ptr(), ws_ptr, ws_bytes, _dtype_code(key_cache),
              _stream(query)))
    return out


def stream_read(buffer, workgroups, sink):
    """Read every byte of the device tensor ``buffer`` once (pkv_stream_read,
    a measurement aid: the achievable HBM read rate); ``sink`` is a device
    tensor of at least 4 bytes the kernel may write."""
    _dev(buffer, "buffer")
    _dev(sink, "sink")
    if sink.numel() * sink.element_size() < 4:
        raise InvalidArgument("sink must hold at least 4 bytes")
    _check(_lib.pkv_stream_read(buffer.data_ptr(), buffer.numel() * buffer.element_size(),
                                int(workgroups), sink.data_ptr(), _stream(buffer)))


def matrix_loop(iters, workgroups, sink):
    """Run ``iters`` iterations of four independent bf16 16x16x32 matrix
    products per wavefront over ``workgroups`` workgroups of 256 threads
    (pkv_matrix_loop, a measurement aid: the matrix-core rate this GPU
    sustains); ``sink`` is a float32 device tensor the kernel may write.
    Returns the floating-point operations one launch performs."""
    _dev(sink, "sink", dtype=torch.float32)
    _check(_lib.pkv_matrix_loop(int(iters), int(workgroups), sink.data_ptr(), _stream(sink)))
    return int(workgroups) * 4 * int(iters) * 4 * 16384


def paged_attention_decode_noalloc(query, key_cache, value_cache, block_tables, context_lens,
                                   scale, max_context_len, out, partition_size=0,
                                   shared_blocks=False):
    """paged_attention_decode with its split-K partials in the library's
    fixed device array instead of a workspace (pkv_paged_attention_decode_noalloc):
    the call allocates nothing, so ``out`` [B, Hq, D] float32 is required.
    Calls on one GPU share the array and must not overlap."""
    nb, hkv, bs, d = _cache_dims(key_cache, value_cache)
    _dev(query, "query", dtype=key_cache.dtype, ndim=3)
    _dev(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _dev(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    b, hq, dq = query.shape
    if dq != d or block_tables.shape[0] != b or context_lens.shape[0] != b:
        raise InvalidArgument("query [B, Hq, D], block_tables [B, max_blocks], context_lens [B]")
    _dev(out, "out", dtype=torch.float32, ndim=3)
    if tuple(out.shape) != (b, hq, d):
        raise InvalidArgument("out must be [B, Hq, D]")
    _check(_lib.pkv_paged_attention_decode_noalloc(
        query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(), block_tables.data_ptr(),
        context_lens.data_ptr(), b, hq, hkv, d, bs, block_tables.shape[1], nb,
        int(max_context_len), float(scale), int(partition_size), out.data_ptr(),
        _decode_code(key_cache, shared_blocks), _stream(query)))
    return out


def paged_attention_decode_append(query, key, value, key_cache, value_cache, block_tables,
                                  context_lens, scale, max_context_len, partition_size=0,
                                  out=None, workspace=None):
    """One decode step with the append fused into the decode kernel
    (pkv_paged_attention_decode_append): store key/value [B, Hkv, D] at each
    sequence's newest position (context_lens[b] - 1, counted in
    context_lens), then decode.  Returns out [B, Hq, D] float32."""
    return _decode_append(_lib.pkv_paged_attention_decode_append, query, key, value, key_cache,
                          value_cache, block_tables, context_lens, scale, max_context_len,
                          partition_size, out, workspace)


def paged_attention_decode_append_partials(query, key, value, key_cache, value_cache,
                                           block_tables, context_lens, scale, max_context_len,
                                           partition_size, out, workspace):
    """First stage of paged_attention_decode_append
    (pkv_paged_attention_decode_append_partials); pass the same ``out`` and
    ``workspace`` to paged_attention_decode_merge."""
    return _decode_append(_lib.pkv_paged_attention_decode_append_partials, query, key, value,
                          key_cache, value_cache, block_tables, context_lens, scale,
                          max_context_len, partition_size, out, workspace)


class DecodeLauncher:
    """Paged decode launches with the fixed arguments marshalled once: a
    serving loop's hot path costs one ctypes call per launch.

    The caches, output, workspace and sizes are checked when the launcher
    is made; each launch checks only the shapes and dtypes of the per-step
    tensors (query, new K/V rows, tables, lengths) and that its
    max_context_len is within the bound the workspace was sized for.  The
    library checks everything else, as for the plain functions.
    ``partials`` (with ``key``/``value``: the append fused in) and ``merge``
    are the two stages of paged_attention_decode(_append).  ``shared_blocks``
    sets PKV_DECODE_SHARED_BLOCKS on every launch."""

    def __init__(self, key_cache, value_cache, num_heads, num_seqs, max_blocks,
                 max_context_len, partition_size, out, workspace, stream=None,
                 shared_blocks=False):
        nb, hkv, bs, d = _cache_dims(key_cache, value_cache)
        _dev(out, "out", dtype=torch.float32, ndim=3)
        if tuple(out.shape) != (num_seqs, num_heads, d):
            raise InvalidArgument("out must be [num_seqs, num_heads, head_dim]")
        need = paged_attention_decode_workspace_size(num_seqs, num_heads, hkv, d,
                                                     int(max_context_len), partition_size)
        ws_ptr, ws_bytes = None, 0
        if workspace is not None:
            _dev(workspace, "workspace")
            ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
        if ws_bytes < need:
            raise BufferTooSmall(f"workspace needs {need} bytes")
        self.part = paged_attention_decode_partition_size(num_seqs, hkv, bs, int(max_context_len),
                                                          partition_size)
        self._keep = (key_cache, value_cache, out, workspace)
        self._dtype = key_cache.dtype
        self._q_shape = (num_seqs, num_heads, d)
        self._kv_shape = (num_seqs, hkv, d)
        self._t_shape = (num_seqs, max_blocks)
        self._max_ctx = int(max_context_len)
        self._stream = ctypes.c_void_p((torch.cuda.current_stream(key_cache.device)
                                        if stream is None else stream).cuda_stream)
        self._dims = (num_seqs, num_heads, hkv, d, bs, max_blocks, nb)
        self._kc, self._vc, self._out = key_cache.data_ptr(), value_cache.data_ptr(), out.data_ptr()
        self._ws = (ws_ptr, ws_bytes)
        self._code = _decode_code(key_cache, shared_blocks)

    def _check_step(self, t, shape, dtype, name):
        if t.shape != shape or t.dtype != dtype or not t.is_contiguous():
            raise InvalidArgument(f"{name} must be a contiguous {dtype} tensor of shape {shape}")
        return t.data_ptr()

    def _host_lens(self, lens):
        b = self._dims[0]
        if not (isinstance(lens, np.ndarray) and lens.dtype == np.int32 and lens.shape == (b,)
                and lens.flags.c_contiguous):
            raise InvalidArgument(f"lens must be a contiguous int32 numpy array of shape ({b},)")
        return lens.ctypes.data

    @staticmethod
    def _host_changes(changes, num_changes):
        if not (isinstance(changes, np.ndarray) and changes.dtype == np.int32 and
                changes.ndim == 2 and changes.shape[1] == 3 and changes.flags.c_contiguous):
            raise InvalidArgument("changes must be a contiguous int32 numpy array of shape (n, 3)")
        if not 0 <= int(num_changes) <= changes.shape[0]:
            raise InvalidArgument("num_changes outside the changes array")
        return changes.ctypes.data

    def partials(self, query, block_tables, context_lens, max_context_len, scale, key=None,
                 value=None):
        if max_context_len > self._max_ctx:
            raise InvalidArgument("max_context_len above the launcher's bound")
        q = self._check_step(query, self._q_shape, self._dtype, "query")
        t = self._check_step(block_tables, self._t_shape, torch.int32, "block_tables")
        l_ = self._check_step(context_lens, self._t_shape[:1], torch.int32, "context_lens")
        b, hq, hkv, d, bs, mb, nb = self._dims
        if key is None:
            _check(_lib.pkv_paged_attention_decode_partials(
                q, self._kc, self._vc, t, l_, b, hq, hkv, d, bs, mb, nb, int(max_context_len),
                float(scale), self.part, self._out, self._ws[0], self._ws[1], self._code,
                self._stream))
        else:
            k = self._check_step(key, self._kv_shape, self._dtype, "key")
            v = self._check_step(value, self._kv_shape, self._dtype, "value")
            _check(_lib.pkv_paged_attention_decode_append_partials(
                q, k, v, self._kc, self._vc, t, l_, b, hq, hkv, d, bs, mb, nb,
                int(max_context_len), float(scale), self.part, self._out, self._ws[0],
                self._ws[1], self._code, self._stream))

    def step_partials(self, query, block_tables, lens, changes, num_changes, max_context_len,
                      scale, key=None, value=None):
        """First stage of pkv_paged_attention_decode_step: host lengths
        ``lens`` and table changes ``changes[:num_changes]`` (contiguous
        int32 numpy arrays) go by value in the kernel arguments."""
        if max_context_len > self._max_ctx:
            raise InvalidArgument("max_context_len above the launcher's bound")
        q = self._check_step(query, self._q_shape, self._dtype, "query")
        t = self._check_step(block_tables, self._t_shape, torch.int32, "block_tables")
        b, hq, hkv, d, bs, mb, nb = self._dims
        k = v = None
        if key is not None:
            k = self._check_step(key, self._kv_shape, self._dtype, "key")
            v = self._check_step(value, self._kv_shape, self._dtype, "value")
        lp = self._host_lens(lens)
        cp = self._host_changes(changes, num_changes)
        _check(_lib.pkv_paged_attention_decode_step_partials(
            q, k, v, self._kc, self._vc, t, lp, cp,
            int(num_changes), b, hq, hkv, d, bs, mb, nb, int(max_context_len), float(scale),
            self.part, self._out, self._ws[0], self._ws[1], self._code, self._stream))

    def step_merge(self, lens, max_context_len):
        """Second stage of pkv_paged_attention_decode_step (host lengths)."""
        if max_context_len > self._max_ctx:
            raise InvalidArgument("max_context_len above the launcher's bound")
        b, hq, hkv, d, bs, mb, nb = self._dims
        _check(_lib.pkv_paged_attention_decode_step_merge(
            self._host_lens(lens), b, hq, hkv, d, bs, mb, int(max_context_len), self.part,
            self._out, self._ws[0], self._ws[1], self._stream))

    def merge(self, context_lens, max_context_len):
        if max_context_len > self._max_ctx:
            raise InvalidArgument("max_context_len above the launcher's bound")
        l_ = self._check_step(context_lens, self._t_shape[:1], torch.int32, "context_lens")
        b, hq, hkv, d, bs, mb, nb = self._dims
        _check(_lib.pkv_paged_attention_decode_merge(
            l_, b, hq, hkv, d, bs, mb, int(max_context_len), self.part, self._out, self._ws[0],
            self._ws[1], self._stream))


def paged_attention_decode_step(query, key, value, key_cache, value_cache, block_tables,
                                context_lens, changes, scale, max_context_len, partition_size=0,
                                out=None, workspace=None, shared_blocks=False):
    """Decode step with host metadata by value (pkv_paged_attention_decode_step).

    block_tables: device int32 [B, max_blocks], updated in place with
    ``changes``; context_lens: host int32 [B] (numpy); changes: host int32
    [n, 3] (batch row, logical block, block), e.g. from
    BlockAllocator.append_batch_changes; key/value: new rows [B, Hkv, D] or
    None.  Returns out [B, Hq, D] float32."""
    (nb, hkv, bs, d, b, hq), out, workspace, ws_ptr, ws_bytes = _decode_args(
        query, key_cache, value_cache, block_tables, None, max_context_len, partition_size, out,
        workspace)
    lens = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    changes = np.ascontiguousarray(np.asarray(changes, dtype=np.int32).reshape(-1, 3))
    if lens.shape != (b,):
        raise InvalidArgument("context_lens must hold one length per sequence")
    kp = vp = None
    if key is not None or value is not None:
        _dev(key, "key", dtype=key_cache.dtype, ndim=3)
        _dev(value, "value", dtype=key_cache.dtype, ndim=3)
        if tuple(key.shape) != (b, hkv, d) or value.shape != key.shape:
            raise InvalidArgument("key/value must be [B, num_kv_heads, head_dim]")
        kp, vp = key.data_ptr(), value.data_ptr()
    _check(_lib.pkv_paged_attention_decode_step(
        query.data_ptr(), kp, vp, key_cache.data_ptr(), value_cache.data_ptr(),
        block_tables.data_ptr(), lens.ctypes.data, changes.ctypes.data, changes.shape[0], b, hq,
        hkv, d, bs, block_tables.shape[1], nb, int(max_context_len), float(scale),
        int(partition_size), out.data_ptr(), ws_ptr, ws_bytes,
        _decode_code(key_cache, shared_blocks), _stream(query)))
    return out


def paged_attention_decode_step_mapped(query, key, value, key_cache, value_cache, block_tables,
                                       table_rows, context_lens, changes, scale,
                                       max_context_len, partition_size=0, out=None,
                                       workspace=None, shared_blocks=False):
    """paged_attention_decode_step with the block tables in rows of the
    caller's choosing (pkv_paged_attention_decode_step_mapped): batch row b
    reads and updates row table_rows[b] (host int32 [B], distinct) of
    block_tables (device int32 [rows, max_blocks]); changes name batch
    rows."""
    (nb, hkv, bs, d, b, hq), out, workspace, ws_ptr, ws_bytes = _decode_args(
        query, key_cache, value_cache, block_tables, None, max_context_len, partition_size, out,
        workspace, mapped=True)
    lens = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    rows = np.ascontiguousarray(np.asarray(table_rows, dtype=np.int32))
    changes = np.ascontiguousarray(np.asarray(changes, dtype=np.int32).reshape(-1, 3))
    if lens.shape != (b,) or rows.shape != (b,):
        raise InvalidArgument("context_lens and table_rows must hold one entry per sequence")
    kp = vp = None
    if key is not None or value is not None:
        _dev(key, "key", dtype=key_cache.dtype, ndim=3)
        _dev(value, "value", dtype=key_cache.dtype, ndim=3)
        if tuple(key.shape) != (b, hkv, d) or value.shape != key.shape:
            raise InvalidArgument("key/value must be [B, num_kv_heads, head_dim]")
        kp, vp = key.data_ptr(), value.data_ptr()
    _check(_lib.pkv_paged_attention_decode_step_mapped(
        query.data_ptr(), kp, vp, key_cache.data_ptr(), value_cache.data_ptr(),
        block_tables.data_ptr(), block_tables.shape[0], rows.ctypes.data, lens.ctypes.data,
        changes.ctypes.data, changes.shape[0], b, hq, hkv, d, bs, block_tables.shape[1], nb,
        int(max_context_len), float(scale), int(partition_size), out.data_ptr(), ws_ptr, ws_bytes,
        _decode_code(key_cache, shared_blocks), _stream(query)))
    return out


def paged_attention_decode_partials(query, key_cache, value_cache, block_tables, context_lens,
                                    scale, max_context_len, partition_size, out, workspace):
    """First stage of decode (pkv_paged_attention_decode_partials); pass the
    same ``out``/``workspace`` to paged_attention_decode_merge."""
    (nb, hkv, bs, d, b, hq), out, workspace, ws_ptr, ws_bytes = _decode_args(
        query, key_cache, value_cache, block_tables, context_lens, max_context_len,
        partition_size, out, workspace)
    _check(_lib.pkv_paged_attention_decode_partials(
        query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(), block_tables.data_ptr(),
        context_lens.data_ptr(), b, hq, hkv, d, bs, block_tables.shape[1], nb,
        int(max_context_len), float(scale), int(partition_size), out.data_ptr(), ws_ptr, ws_bytes,
        _dtype_code(key_cache), _stream(query)))
    return out


def paged_kv_append_fp8(key, value, key_cache, value_cache, slot_mapping, k_scale, v_scale):
    """Quantising scatter of key/value [T, Hkv, D] (float32/float16/bfloat16)
    into 8-bit E4M3 caches (uint8 or float8_e4m3fn) at slot_mapping [T]:
    code = nearest E4M3 to x / scale.  pkv_paged_kv_append_fp8."""
    nb, hkv, bs, d = _cache_dims(key_cache, value_cache)
    if key_cache.dtype not in _FP8_TYPES:
        raise InvalidArgument("the caches must be uint8 or float8_e4m3fn")
    _dev(key, "key", ndim=3)
    _dev(value, "value", dtype=key.dtype, ndim=3)
    _dev(slot_mapping, "slot_mapping", dtype=torch.int32, ndim=1)
    t = key.shape[0]
    if key.shape != (t, hkv, d) or value.shape != key.shape or slot_mapping.shape[0] != t:
        raise InvalidArgument("key/value must be [T, num_kv_heads, head_dim] with T slots")
    _check(_lib.pkv_paged_kv_append_fp8(key.data_ptr(), value.data_ptr(), key_cache.data_ptr(),
                                        value_cache.data_ptr(), slot_mapping.data_ptr(), t, hkv,
                                        d, bs, nb, float(k_scale), float(v_scale),
                                        _dtype_code(key), _stream(key_cache)))


def _decode_fp8(fn, query, key_cache, value_cache, block_tables, context_lens, scale, k_scale,
                v_scale, max_context_len, partition_size, out, workspace, shared_blocks=False):
    (nb, hkv, bs, d, b, hq), out, workspace, ws_ptr, ws_bytes = _decode_args(
        query, key_cache, value_cache, block_tables, context_lens, max_context_len,
        partition_size, out, workspace, fp8=True)
    _check(fn(query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
              block_tables.data_ptr(), context_lens.data_ptr(), b, hq, hkv, d, bs,
              block_tables.shape[1], nb, int(max_context_len), float(scale), float(k_scale),
              float(v_scale), int(partition_size), out.data_ptr(), ws_ptr, ws_bytes,
              _decode_code(query, shared_blocks), _stream(query)))
    return out


def paged_attention_decode_fp8(query, key_cache, value_cache, block_tables, context_lens, scale,
                               k_scale, v_scale, max_context_len, partition_size=0, out=None,
                               workspace=None, shared_blocks=False):
    """Decode over 8-bit E4M3 caches (pkv_paged_attention_decode_fp8): as
    paged_attention_decode with K = code value * k_scale, V = code value *
    v_scale; query bfloat16 or float16; returns out [B, Hq, D] float32."""
    return _decode_fp8(_lib.pkv_paged_attention_decode_fp8, query, key_cache, value_cache,
                       block_tables, context_lens, scale, k_scale, v_scale, max_context_len,
                       partition_size, out, workspace, shared_blocks)


def paged_attention_decode_fp8_step(query, key, value, key_cache, value_cache, block_tables,
                                    context_lens, changes, scale, k_scale, v_scale,
                                    max_context_len, partition_size=0, out=None, workspace=None,
                                    shared_blocks=False):
    """Step form of paged_attention_decode_fp8 (pkv_paged_attention_decode_fp8_step):
    block_tables is the device table kept across steps (updated in place
    with ``changes``); context_lens host int32 [B]; changes host int32 [n, 3];
    key/value the step's new rows [B, Hkv, D] in the query's dtype, quantised
    with k_scale / v_scale as paged_kv_append_fp8 does, or None."""
    (nb, hkv, bs, d, b, hq), out, workspace, ws_ptr, ws_bytes = _decode_args(
        query, key_cache, value_cache, block_tables, None, max_context_len, partition_size, out,
        workspace, fp8=True)
    lens = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    changes = np.ascontiguousarray(np.asarray(changes, dtype=np.int32).reshape(-1, 3))
    if lens.shape != (b,):
        raise InvalidArgument("context_lens must hold one length per sequence")
    kp = vp = None
    if key is not None or value is not None:
        _dev(key, "key", dtype=query.dtype, ndim=3)
        _dev(value, "value", dtype=query.dtype, ndim=3)
        if tuple(key.shape) != (b, hkv, d) or value.shape != key.shape:
            raise InvalidArgument("key/value must be [B, num_kv_heads, head_dim]")
        kp, vp = key.data_ptr(), value.data_ptr()
    _check(_lib.pkv_paged_attention_decode_fp8_step(
        query.data_ptr(), kp, vp, key_cache.data_ptr(), value_cache.data_ptr(),
        block_tables.data_ptr(), lens.ctypes.data, changes.ctypes.data, changes.shape[0], b, hq,
        hkv, d, bs, block_tables.shape[1], nb, int(max_context_len), float(scale),
        float(k_scale), float(v_scale), int(partition_size), out.data_ptr(), ws_ptr, ws_bytes,
        _decode_code(query, shared_blocks), _stream(query)))
    return out


def paged_attention_decode_fp8_partials(query, key_cache, value_cache, block_tables,
                                        context_lens, scale, k_scale, v_scale, max_context_len,
                                        partition_size, out, workspace):
    """First stage of paged_attention_decode_fp8; paged_attention_decode_merge
    with the same ``out``/``workspace`` completes it."""
    return _decode_fp8(_lib.pkv_paged_attention_decode_fp8_partials, query, key_cache,
                       value_cache, block_tables, context_lens, scale, k_scale, v_scale,
                       max_context_len, partition_size, out, workspace)


def paged_attention_decode_shared_prefix_workspace_size(num_seqs, num_heads, num_kv_heads,
                                                        head_dim, block_size, max_context_len,
                                                        prefix_len, partition_size=0):
    """Workspace bytes of paged_attention_decode_shared_prefix
    (pkv_paged_attention_decode_shared_prefix_workspace_size)."""
    out = ctypes.c_size_t()
    _check(_lib.pkv_paged_attention_decode_shared_prefix_workspace_size(
        int(num_seqs), int(num_heads), int(num_kv_heads), int(head_dim), int(block_size),
        int(max_context_len), int(prefix_len), int(partition_size), ctypes.byref(out)))
    return out.value


def paged_attention_decode_shared_prefix(query, key_cache, value_cache, block_tables,
                                         context_lens, prefix_len, scale, max_context_len,
                                         partition_size=0, out=None, workspace=None,
                                         shared_blocks=False):
    """Decode for a batch whose sequences share their first ``prefix_len``
    tokens (pkv_paged_attention_decode_shared_prefix): the prefix part as
    one matrix-core contraction per head, the private suffixes by the split-K
    decode kernel, then the merge.  Same arguments and result as
    paged_attention_decode, plus ``prefix_len`` (a multiple of the block
    size; the prefix is read through row 0 of ``block_tables``).
    ``shared_blocks`` applies the load hint to the suffix reads."""
    nb, hkv, bs, d = _cache_dims(key_cache, value_cache)
    _dev(query, "query", dtype=key_cache.dtype, ndim=3)
    _dev(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _dev(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    b, hq, _ = query.shape
    if query.shape[2] != d or block_tables.shape[0] != b or context_lens.shape[0] != b:
        raise InvalidArgument("query [B, Hq, D], block_tables [B, max_blocks], context_lens [B]")
    if out is None:
        out = torch.empty((b, hq, d), dtype=torch.float32, device=query.device)
    _dev(out, "out", dtype=torch.float32, ndim=3)
    if tuple(out.shape) != (b, hq, d):
        raise InvalidArgument("out must be [B, Hq, D]")
    need = paged_attention_decode_shared_prefix_workspace_size(
        b, hq, hkv, d, bs, int(max_context_len), int(prefix_len), partition_size)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=query.device)
    _dev(workspace, "workspace")
    _check(_lib.pkv_paged_attention_decode_shared_prefix(
        query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(), block_tables.data_ptr(),
        context_lens.data_ptr(), b, hq, hkv, d, bs, block_tables.shape[1], nb,
        int(max_context_len), int(prefix_len), float(scale), int(partition_size),
        out.data_ptr(), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _decode_code(key_cache, shared_blocks), _stream(query)))
    return out


def paged_attention_decode_shared_prefix_step(query, key, value, key_cache, value_cache,
                                              block_tables, context_lens, changes, prefix_len,
                                              scale, max_context_len, partition_size=0, out=None,
                                              workspace=None, shared_blocks=False):
    """Step form of paged_attention_decode_shared_prefix
    (pkv_paged_attention_decode_shared_prefix_step): block_tables is the
    device table kept across steps (updated in place with ``changes``);
    context_lens host int32 [B] and changes host int32 [n, 3] as for
    paged_attention_decode_step; key/value the step's new rows or None."""
    nb, hkv, bs, d = _cache_dims(key_cache, value_cache)
    _dev(query, "query", dtype=key_cache.dtype, ndim=3)
    _dev(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    b, hq, _ = query.shape
    lens = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    changes = np.ascontiguousarray(np.asarray(changes, dtype=np.int32).reshape(-1, 3))
    if lens.shape != (b,) or query.shape[2] != d or block_tables.shape[0] != b:
        raise InvalidArgument("query [B, Hq, D], block_tables [B, max_blocks], context_lens [B]")
    kp = vp = None
    if key is not None or value is not None:
        _dev(key, "key", dtype=key_cache.dtype, ndim=3)
        _dev(value, "value", dtype=key_cache.dtype, ndim=3)
        if tuple(key.shape) != (b, hkv, d) or value.shape != key.shape:
            raise InvalidArgument("key/value must be [B, num_kv_heads, head_dim]")
        kp, vp = key.data_ptr(), value.data_ptr()
    if out is None:
        out = torch.empty((b, hq, d), dtype=torch.float32, device=query.device)
    _dev(out, "out", dtype=torch.float32, ndim=3)
    if tuple(out.shape) != (b, hq, d):
        raise InvalidArgument("out must be [B, Hq, D]")
    need = paged_attention_decode_shared_prefix_workspace_size(
        b, hq, hkv, d, bs, int(max_context_len), int(prefix_len), partition_size)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=query.device)
    _dev(workspace, "workspace")
    _check(_lib.pkv_paged_attention_decode_shared_prefix_step(
        query.data_ptr(), kp, vp, key_cache.data_ptr(), value_cache.data_ptr(),
        block_tables.data_ptr(), lens.ctypes.data, changes.ctypes.data, changes.shape[0], b, hq,
        hkv, d, bs, block_tables.shape[1], nb, int(max_context_len), int(prefix_len), float(scale),
        int(partition_size), out.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _decode_code(key_cache, shared_blocks),
        _stream(query)))
    return out


def _prefix_groups(group_starts, prefix_lens):
    """Host int32 copies of a grouped-prefix call's group arrays."""
    starts = np.ascontiguousarray(np.asarray(group_starts, dtype=np.int32).reshape(-1))
    lens = np.ascontiguousarray(np.asarray(prefix_lens, dtype=np.int32).reshape(-1))
    if starts.shape[0] != lens.shape[0] + 1 or lens.shape[0] == 0:
        raise InvalidArgument("group_starts must have one entry more than prefix_lens (>= 1)")
    return starts, lens


def paged_attention_decode_grouped_prefix_workspace_size(num_seqs, num_heads, num_kv_heads,
                                                         head_dim, block_size, max_context_len,
                                                         group_starts, prefix_lens,
                                                         partition_size=0):
    """Workspace bytes of paged_attention_decode_grouped_prefix
    (pkv_paged_attention_decode_grouped_prefix_workspace_size)."""
    starts, lens = _prefix_groups(group_starts, prefix_lens)
    out = ctypes.c_size_t()
    _check(_lib.pkv_paged_attention_decode_grouped_prefix_workspace_size(
        int(num_seqs), int(num_heads), int(num_kv_heads), int(head_dim), int(block_size),
        int(max_context_len), lens.shape[0], starts.ctypes.data, lens.ctypes.data,
        int(partition_size), ctypes.byref(out)))
    return out.value


def _grouped_args(query, key_cache, value_cache, block_tables, group_starts, prefix_lens,
                  max_context_len, partition_size, out, workspace):
    nb, hkv, bs, d = _cache_dims(key_cache, value_cache)
    _dev(query, "query", dtype=key_cache.dtype, ndim=3)
    _dev(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    b, hq, _ = query.shape
    if query.shape[2] != d or block_tables.shape[0] != b:
        raise InvalidArgument("query [B, Hq, D], block_tables [B, max_blocks]")
    starts, lens = _prefix_groups(group_starts, prefix_lens)
    if out is None:
        out = torch.empty((b, hq, d), dtype=torch.float32, device=query.device)
    _dev(out, "out", dtype=torch.float32, ndim=3)
    if tuple(out.shape) != (b, hq, d):
        raise InvalidArgument("out must be [B, Hq, D]")
    need = paged_attention_decode_grouped_prefix_workspace_size(
        b, hq, hkv, d, bs, int(max_context_len), starts, lens, partition_size)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=query.device)
    _dev(workspace, "workspace")
    return nb, hkv, bs, d, b, hq, starts, lens, out, workspace


def paged_attention_decode_grouped_prefix(query, key_cache, value_cache, block_tables,
                                          context_lens, group_starts, prefix_lens, scale,
                                          max_context_len, partition_size=0, out=None,
                                          workspace=None, shared_blocks=False):
    """Decode for a batch of prefix groups
    (pkv_paged_attention_decode_grouped_prefix): rows group_starts[g] ..
    group_starts[g + 1] - 1 share their first prefix_lens[g] tokens (0: no
    sharing), read through the table of the group's first row.  Same result
    as paged_attention_decode on the same tables."""
    nb, hkv, bs, d, b, hq, starts, lens, out, workspace = _grouped_args(
        query, key_cache, value_cache, block_tables, group_starts, prefix_lens,
        max_context_len, partition_size, out, workspace)
    _dev(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    if context_lens.shape[0] != b:
        raise InvalidArgument("context_lens must be [B]")
    _check(_lib.pkv_paged_attention_decode_grouped_prefix(
        query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(), block_tables.data_ptr(),
        context_lens.data_ptr(), b, hq, hkv, d, bs, block_tables.shape[1], nb,
        int(max_context_len), lens.shape[0], starts.ctypes.data, lens.ctypes.data, float(scale),
        int(partition_size), out.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _decode_code(key_cache, shared_blocks),
        _stream(query)))
    return out


def paged_attention_decode_grouped_prefix_step(query, key, value, key_cache, value_cache,
                                               block_tables, context_lens, changes, group_starts,
                                               prefix_lens, scale, max_context_len,
                                               partition_size=0, out=None, workspace=None,
                                               shared_blocks=False):
    """Step form of paged_attention_decode_grouped_prefix
    (pkv_paged_attention_decode_grouped_prefix_step): block_tables is the
    device table kept across steps (updated in place with ``changes``);
    context_lens host int32 [B] and changes host int32 [n, 3] as for
    paged_attention_decode_step; key/value the step's new rows or None."""
    nb, hkv, bs, d, b, hq, starts, glens, out, workspace = _grouped_args(
        query, key_cache, value_cache, block_tables, group_starts, prefix_lens,
        max_context_len, partition_size, out, workspace)
    lens = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    changes = np.ascontiguousarray(np.asarray(changes, dtype=np.int32).reshape(-1, 3))
    if lens.shape != (b,):
        raise InvalidArgument("context_lens must be host int32 [B]")
    kp = vp = None
    if key is not None or value is not None:
        _dev(key, "key", dtype=key_cache.dtype, ndim=3)
        _dev(value, "value", dtype=key_cache.dtype, ndim=3)
        if tuple(key.shape) != (b, hkv, d) or value.shape != key.shape:
            raise InvalidArgument("key/value must be [B, num_kv_heads, head_dim]")
        kp, vp = key.data_ptr(), value.data_ptr()
    _check(_lib.pkv_paged_attention_decode_grouped_prefix_step(
        query.data_ptr(), kp, vp, key_cache.data_ptr(), value_cache.data_ptr(),
        block_tables.data_ptr(), lens.ctypes.data, changes.ctypes.data, changes.shape[0], b, hq,
        hkv, d, bs, block_tables.shape[1], nb, int(max_context_len), glens.shape[0],
        starts.ctypes.data, glens.ctypes.data, float(scale), int(partition_size), out.data_ptr(),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _decode_code(key_cache, shared_blocks), _stream(query)))
    return out


def paged_attention_decode_merge(context_lens, num_kv_heads, block_size, max_blocks_per_seq,
                                 max_context_len, partition_size, out, workspace):
    """Second stage of decode (pkv_paged_attention_decode_merge)."""
    _dev(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    _dev(out, "out", dtype=torch.float32, ndim=3)
    b, hq, d = out.shape
    ws_ptr, ws_bytes = (None, 0)
    if workspace is not None:
        _dev(workspace, "workspace")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check(_lib.pkv_paged_attention_decode_merge(
        context_lens.data_ptr(), b, hq, num_kv_heads, d, block_size, max_blocks_per_seq,
        int(max_context_len), int(partition_size), out.data_ptr(), ws_ptr, ws_bytes,
        _stream(out)))
    return out


def paged_attention_prefill(query, key_cache, value_cache, block_tables, context_lens,
                            cu_query_lens, scale, max_query_len, out=None):
    """Causal chunked prefill (pkv_paged_attention_prefill).

    query [sum c_b, Hq, D] (cache dtype); cu_query_lens [B+1] int32;
    context_lens [B] int32 counting the chunk; returns out float32.
    """
    return _prefill(query, key_cache, value_cache, block_tables, context_lens, cu_query_lens,
                    scale, max_query_len, out)


def paged_attention_prefill_fp8(query, key_cache, value_cache, block_tables, context_lens,
                                cu_query_lens, scale, k_scale, v_scale, max_query_len, out=None):
    """Causal chunked prefill over 8-bit E4M3 caches
    (pkv_paged_attention_prefill_fp8): as paged_attention_prefill with
    K = code value * k_scale, V = code value * v_scale; query bfloat16 or
    float16."""
    return _prefill(query, key_cache, value_cache, block_tables, context_lens, cu_query_lens,
                    scale, max_query_len, out, fp8=(k_scale, v_scale))


def _prefill(query, key_cache, value_cache, block_tables, context_lens, cu_query_lens, scale,
             max_query_len, out, fp8=None):
    nb, hkv, bs, d = _cache_dims(key_cache, value_cache)
    if fp8 is None:
        _dev(query, "query", dtype=key_cache.dtype, ndim=3)
    else:
        if key_cache.dtype not in _FP8_TYPES:
            raise InvalidArgument("an 8-bit cache must be uint8 or float8_e4m3fn")
        _dev(query, "query", ndim=3)
        if query.dtype not in (torch.bfloat16, torch.float16):
            raise InvalidArgument("the query of an 8-bit cache must be bfloat16 or float16")
    _dev(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _dev(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    _dev(cu_query_lens, "cu_query_lens", dtype=torch.int32, ndim=1)
    b = context_lens.shape[0]
    total, hq, dq = query.shape
    if dq != d or block_tables.shape[0] != b or cu_query_lens.shape[0] != b + 1:
        raise InvalidArgument("query, block_tables, context_lens and cu_query_lens disagree")
    if out is None:
        out = torch.empty((total, hq, d), dtype=torch.float32, device=query.device)
    _dev(out, "out", dtype=torch.float32, ndim=3)
    if tuple(out.shape) != (total, hq, d):
        raise InvalidArgument("out must be [sum c_b, Hq, D]")
    args = (query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
            block_tables.data_ptr(), context_lens.data_ptr(), cu_query_lens.data_ptr(), b, hq,
            hkv, d, bs, block_tables.shape[1], nb, total, int(max_query_len), float(scale))
    if fp8 is None:
        _check(_lib.pkv_paged_attention_prefill(*args, out.data_ptr(), _dtype_code(key_cache),
                                                _stream(query)))
    else:
        _check(_lib.pkv_paged_attention_prefill_fp8(*args, float(fp8[0]), float(fp8[1]),
                                                    out.data_ptr(), _dtype_code(query),
                                                    _stream(query)))
    return out
