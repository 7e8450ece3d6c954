"""C ABI checks that need no GPU: the library loads, exports every function
include/pkv.h declares, rejects bad arguments before touching the device,
and its allocator reproduces the reference allocator bit for bit."""

import ctypes
import json
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from conftest import GOLDEN, ROOT

import paged_kv_cache_420_amd as pkv
from oracle import OutOfBlocks as RefOutOfBlocks, RefAllocator


def _declared():
    text = open(os.path.join(ROOT, "include", "pkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 20
    lib = ctypes.CDLL(pkv.library_path())
    missing = [n for n in names if not hasattr(lib, n)]
    assert missing == []


def test_library_is_the_in_tree_build():
    assert os.path.dirname(pkv.library_path()) == os.path.join(ROOT, "paged_kv_cache_420_amd")
    assert pkv.version().count(".") == 2


def test_device_calls_reject_bad_arguments_before_launch():
    lib = pkv._lib
    null = None
    # unknown dtype
    assert lib.pkv_paged_kv_append(null, null, null, null, null, 1, 1, 64, 16, 4, 9, null) == 1
    # head_dim * elem not a multiple of 16 bytes
    assert lib.pkv_copy_blocks(null, null, null, null, 1, 4, 1, 16, 3, 2, null) == 1
    # decode: GQA ratio not supported
    ws = ctypes.c_size_t()
    assert lib.pkv_paged_attention_decode(null, null, null, null, null, 2, 6, 2, 128, 16, 8, 64,
                                          100, 1.0, 0, null, null, 0, 2, null) == 7
    # decode: partition size not a multiple of 64
    assert lib.pkv_paged_attention_decode_workspace_size(2, 4, 4, 128, 100, 100,
                                                         ctypes.byref(ws)) == 1
    assert lib.pkv_paged_attention_decode_workspace_size(2, 4, 4, 128, 100, 0,
                                                         ctypes.byref(ws)) == 0
    assert ws.value == 0                     # one partition: no workspace
    assert lib.pkv_paged_attention_decode_workspace_size(2, 4, 4, 128, 1000, 512,
                                                         ctypes.byref(ws)) == 0
    assert ws.value == 2 * 4 * 2 * (128 + 2) * 4
    # automatic partition: small grids get shorter partitions (more of them)
    assert lib.pkv_paged_attention_decode_workspace_size(1, 8, 8, 128, 4096, 0,
                                                         ctypes.byref(ws)) == 0
    assert ws.value == 1 * 8 * (4096 // 128) * (128 + 2) * 4
    assert lib.pkv_paged_attention_decode_workspace_size(64, 32, 32, 128, 2000, 0,
                                                         ctypes.byref(ws)) == 0
    assert ws.value == 0                     # one 2048-token partition
    assert lib.pkv_paged_attention_decode_workspace_size(64, 32, 32, 128, 4000, 0,
                                                         ctypes.byref(ws)) == 0
    assert ws.value == 64 * 32 * 2 * (128 + 2) * 4
    # GQA: partials per query head
    assert lib.pkv_paged_attention_decode_workspace_size(256, 64, 8, 128, 8192, 512,
                                                         ctypes.byref(ws)) == 0
    assert ws.value == 256 * 64 * 16 * (128 + 2) * 4
    # decode: NULL pointers with otherwise valid sizes
    assert lib.pkv_paged_attention_decode(null, null, null, null, null, 2, 4, 4, 128, 16, 8, 64,
                                          100, 1.0, 0, null, null, 0, 2, null) == 1
    assert b"NULL" in lib.pkv_last_error()
    # fused decode + append: NULL new rows with a non-empty batch
    assert lib.pkv_paged_attention_decode_append(null, null, null, null, null, null, null, 2, 4, 4,
                                                 128, 16, 8, 64, 100, 1.0, 0, null, null, 0, 2,
                                                 null) == 1
    # 8-bit caches: only through the *_fp8 calls, with a 16-bit query and
    # positive finite scales
    assert lib.pkv_paged_attention_decode(null, null, null, null, null, 2, 4, 4, 128, 16, 8, 64,
                                          100, 1.0, 0, null, null, 0, 3, null) == 1
    assert b"fp8" in lib.pkv_last_error()
    assert lib.pkv_paged_attention_decode_fp8(null, null, null, null, null, 2, 4, 4, 128, 16, 8,
                                              64, 100, 1.0, 0.5, 0.5, 0, null, null, 0, 0,
                                              null) == 1
    assert lib.pkv_paged_attention_decode_fp8(null, null, null, null, null, 2, 4, 4, 128, 16, 8,
                                              64, 100, 1.0, 0.0, 0.5, 0, null, null, 0, 2,
                                              null) == 1
    assert lib.pkv_paged_attention_decode_fp8_partials(null, null, null, null, null, 2, 6, 2,
                                                       128, 16, 8, 64, 100, 1.0, 0.5, 0.5, 0,
                                                       null, null, 0, 2, null) == 7
    # head_dim 64 codes in 8-token blocks: tiles under 1 KiB
    assert lib.pkv_paged_attention_decode_fp8(null, null, null, null, null, 2, 4, 4, 64, 8, 8,
                                              64, 100, 1.0, 0.5, 0.5, 0, null, null, 0, 2,
                                              null) == 7
    assert lib.pkv_paged_kv_append_fp8(null, null, null, null, null, 1, 1, 64, 16, 4, 1.0, 1.0,
                                       3, null) == 1
    assert lib.pkv_paged_kv_append_fp8(null, null, null, null, null, 1, 1, 64, 16, 4, -1.0, 1.0,
                                       2, null) == 1
    assert lib.pkv_paged_kv_append_fp8(null, null, null, null, null, 1, 1, 24, 16, 4, 1.0, 1.0,
                                       2, null) == 1          # 24 codes: not 16-byte rows
    assert lib.pkv_paged_attention_prefill(null, null, null, null, null, null, 1, 4, 4, 128, 16,
                                           8, 64, 1, 1, 1.0, null, 3, null) == 7
    # empty batches are no-ops
    assert lib.pkv_paged_kv_append_fp8(null, null, null, null, null, 0, 1, 64, 16, 4, 1.0, 1.0,
                                       2, null) == 0
    assert lib.pkv_paged_kv_append(null, null, null, null, null, 0, 1, 64, 16, 4, 2, null) == 0
    assert lib.pkv_paged_attention_decode(null, null, null, null, null, 0, 4, 4, 128, 16, 8, 64,
                                          100, 1.0, 0, null, null, 0, 2, null) == 0
    # measurement aids: sizes and the sink are checked before any launch
    assert lib.pkv_stream_read(null, 24, 64, null, null) == 1      # not a multiple of 16
    assert lib.pkv_stream_read(null, 64, 0, null, null) == 1       # no workgroups
    assert lib.pkv_stream_read(null, 0, 64, null, null) == 0       # nothing to read
    assert lib.pkv_matrix_loop(-1, 64, null, null) == 1
    assert lib.pkv_matrix_loop(10, 0, null, null) == 1
    assert lib.pkv_matrix_loop(10, (1 << 20) + 1, null, null) == 1
    assert lib.pkv_matrix_loop(10, 64, null, null) == 1            # NULL sink
    assert b"NULL" in lib.pkv_last_error()


def test_shared_blocks_hint_is_checked_like_the_dtype_it_rides_on():
    """PKV_DECODE_SHARED_BLOCKS (0x100) is taken off a decode call's dtype
    before the dtype and everything else are checked; calls that move bytes
    (append, block copies) do not take it."""
    lib = pkv._lib
    null = None
    hint = pkv.DECODE_SHARED_BLOCKS
    assert hint == 0x100
    # a valid dtype with the hint: the remaining checks still run
    assert lib.pkv_paged_attention_decode(null, null, null, null, null, 2, 4, 4, 128, 16, 8, 64,
                                          100, 1.0, 0, null, null, 0, 2 | hint, null) == 1
    assert b"NULL" in lib.pkv_last_error()
    assert lib.pkv_paged_attention_decode(null, null, null, null, null, 2, 6, 2, 128, 16, 8, 64,
                                          100, 1.0, 0, null, null, 0, 2 | hint, null) == 7
    assert lib.pkv_paged_attention_decode(null, null, null, null, null, 0, 4, 4, 128, 16, 8, 64,
                                          100, 1.0, 0, null, null, 0, 2 | hint, null) == 0
    # an unknown dtype stays unknown with the hint
    assert lib.pkv_paged_attention_decode(null, null, null, null, null, 2, 4, 4, 128, 16, 8, 64,
                                          100, 1.0, 0, null, null, 0, 9 | hint, null) == 1
    assert b"dtype" in lib.pkv_last_error()
    # 8-bit decode: the hint rides on the query dtype
    assert lib.pkv_paged_attention_decode_fp8(null, null, null, null, null, 2, 4, 4, 128, 16, 8,
                                              64, 100, 1.0, 0.5, 0.5, 0, null, null, 0,
                                              0 | hint, null) == 1
    assert lib.pkv_paged_attention_decode_fp8(null, null, null, null, null, 2, 4, 4, 128, 16, 8,
                                              64, 100, 1.0, 0.5, 0.5, 0, null, null, 0,
                                              2 | hint, null) == 1
    assert b"NULL" in lib.pkv_last_error()
    # the byte-moving calls reject it as an unknown dtype
    assert lib.pkv_paged_kv_append(null, null, null, null, null, 1, 1, 64, 16, 4, 2 | hint,
                                   null) == 1


def test_allocator_reports_errors():
    with pytest.raises(pkv.InvalidArgument):
        pkv.BlockAllocator(4, 2, [0, 1, 1, 2])
    with pytest.raises(pkv.InvalidArgument):
        pkv.BlockAllocator(1 << 27, 16)
    a = pkv.BlockAllocator(4, 2)
    a.add(5)
    with pytest.raises(pkv.SequenceExists):
        a.add(5)
    with pytest.raises(pkv.NoSuchSequence):
        a.free(6)
    with pytest.raises(pkv.NoSuchSequence):
        a.append(6, 1)
    with pytest.raises(pkv.InvalidArgument):
        a.append(5, -1)
    with pytest.raises(pkv.OutOfBlocks):
        a.append(5, 9)
    with pytest.raises(pkv.InvalidArgument):
        a.append_batch([5, 5], [1, 1])
    with pytest.raises(pkv.BufferTooSmall):
        a.build_block_tables([5], 0) if a.append(5, 1) else None


def _live(a):
    """Sequence ids the native allocator holds (ids 0..5 in the op tests)."""
    out = set()
    for q in range(6):
        try:
            a.seq_len(q)
            out.add(q)
        except pkv.NoSuchSequence:
            pass
    return out


def _state(a, seqs):
    if isinstance(a, RefAllocator):
        free, ref, tables = a.snapshot()
        return (free, ref, {s: tables[s] for s in seqs if s in tables},
                sorted(q for q in a.swapped if q in seqs), a.host_free_stack())
    free, ref = a.snapshot()
    tables, swapped = {}, []
    for s in seqs:
        try:
            tables[s] = (a.block_table(s), a.seq_len(s))
            if a.is_swapped(s):
                swapped.append(s)
        except pkv.NoSuchSequence:
            pass
    return free, ref, tables, swapped, a.host_snapshot()


def test_hand_worked_trace_through_the_c_abi():
    fx = json.load(open(os.path.join(GOLDEN, "allocator_trace.json")))
    a = pkv.BlockAllocator(fx["num_blocks"], fx["block_size"], fx["init_order"])
    ids = {"A": 1, "B": 2, "C": 3, "D": 4}
    for step in fx["steps"]:
        op = step["op"]
        if op == "add":
            a.add(ids[step["seq"]])
        elif op == "fork":
            a.fork(ids[step["parent"]], ids[step["child"]])
        elif op == "free":
            a.free(ids[step["seq"]])
        elif step.get("expect_error"):
            with pytest.raises(pkv.OutOfBlocks):
                a.append(ids[step["seq"]], step["n"])
        else:
            slots, cow = a.append(ids[step["seq"]], step["n"])
            assert slots.tolist() == step["slots"]
            assert [list(p) for p in cow] == step["cow"]
        free, ref = a.snapshot()
        assert free == step["free"] and ref == step["ref"], step
        for name, (table, n) in step["tables"].items():
            assert a.block_table(ids[name]) == table
            assert a.seq_len(ids[name]) == n


ops = st.lists(
    st.tuples(st.sampled_from(["add", "append", "fork", "free", "batch", "batch_tables",
                               "batch_changes", "swap_out", "swap_in"]),
              st.integers(0, 5), st.integers(0, 5), st.integers(0, 23)),
    min_size=1, max_size=80)


@settings(max_examples=300, deadline=None)
@given(ops, st.integers(1, 8), st.integers(1, 24), st.integers(0, 16),
       st.randoms(use_true_random=False))
def test_native_allocator_matches_reference_bit_for_bit(seq_ops, block_size, num_blocks,
                                                        host_blocks, rnd):
    order = list(range(num_blocks))
    rnd.shuffle(order)
    ref = RefAllocator(num_blocks, block_size, order)
    nat = pkv.BlockAllocator(num_blocks, block_size, order)
    ref.set_host_pool(host_blocks)
    nat.set_host_pool(host_blocks)
    ids = range(6)
    for op, s, t, n in seq_ops:
        def apply(a, is_ref):
            try:
                if op == "add":
                    a.add(s)
                elif op == "free":
                    a.free(s)
                elif op == "fork":
                    a.fork(s, t)
                elif op == "append":
                    slots, pairs = a.append(s, n)
                    return ("ok", list(slots), [tuple(p) for p in pairs])
                elif op in ("swap_out", "swap_in"):
                    pairs = getattr(a, op)(s)
                    return ("ok", [tuple(int(x) for x in p) for p in pairs])
                elif op == "batch_changes":
                    # the reported entries turn the old tables into the new ones
                    batch = sorted({s, t, (s + 3) % 6})
                    counts = [(n + 2 * i) % 8 for i in range(len(batch))]
                    if is_ref:
                        slots, pairs = a.append_batch(batch, counts)
                        lens = [a.length(q) for q in batch]
                        tables = [a.table(q) for q in batch]
                    else:
                        before = [a.block_table(q) if q in _live(a) else None for q in batch]
                        slots, pairs, lens, changes = a.append_batch_changes(batch, counts)
                        tables = [list(tb) for tb in before]
                        for row, idx, blk in changes.tolist():
                            if idx == len(tables[row]):
                                tables[row].append(blk)
                            else:
                                tables[row][idx] = blk
                        assert tables == [a.block_table(q) for q in batch]
                    return ("ok", list(slots), [tuple(p) for p in pairs], [int(x) for x in lens],
                            [list(tb) for tb in tables])
                elif op == "batch_tables":
                    # append + the batch's tables in one call; max_blocks is
                    # small enough to overflow now and then (all or nothing)
                    batch = sorted({s, t})
                    counts = [(n + 5 * i) % 9 for i in range(len(batch))]
                    mb = 1 + n % 6
                    if is_ref:
                        for q in batch:  # each sequence in batch order:
                            a.length(q)  # KeyError for an unknown one,
                            if q in a.swapped:  # then swapped out
                                raise ValueError("swapped out")
                        if any(-(-(a.length(q) + c) // block_size) > mb
                               for q, c in zip(batch, counts)):
                            return ("too_small",)
                        slots, pairs = a.append_batch(batch, counts)
                        tables, lens = a.build_tables(batch, mb)
                    else:
                        slots, pairs, tables, lens = a.append_batch_tables(batch, counts, mb)
                    return ("ok", list(slots), [tuple(p) for p in pairs],
                            np.asarray(tables, dtype=np.int32).reshape(len(batch), mb).tolist(),
                            [int(x) for x in lens])
                else:
                    batch = sorted({s, t, (s + 2) % 6})
                    counts = [(n + 3 * i) % 7 for i in range(len(batch))]
                    slots, pairs = a.append_batch(batch, counts)
                    return ("ok", list(slots), [tuple(p) for p in pairs])
                return ("ok",)
            except (RefOutOfBlocks, pkv.OutOfBlocks):
                return ("out_of_blocks",)
            except pkv.BufferTooSmall:
                return ("too_small",)
            except (KeyError, pkv.NoSuchSequence):
                return ("no_such_seq",)
            except (ValueError, pkv.SequenceExists, pkv.InvalidArgument):
                return ("invalid",)
        r1 = apply(ref, True)
        r2 = apply(nat, False)
        assert r1 == r2, (op, s, t, n)
        assert _state(ref, ids) == _state(nat, ids)
    live = [i for i in ids if i in ref.tables and i not in ref.swapped]
    tables_r, lens_r = ref.build_tables(live, 30)
    tables_n, lens_n = nat.build_block_tables(live, 30)
    assert np.array_equal(np.array(tables_r, dtype=np.int32).reshape(tables_n.shape), tables_n)
    assert list(lens_r) == lens_n.tolist()
    nat.close()


def test_shared_prefix_workload_builds_identically():
    import workloads
    w = workloads.scaled(workloads.get("shared_prefix_bf16"), num_seqs=16)
    p = workloads.plan(w)
    ref = RefAllocator(p.num_blocks, w.block_size, p.free_order)
    nat = pkv.BlockAllocator(p.num_blocks, w.block_size, p.free_order)
    log_r, log_n = [], []
    workloads.run_schedule(p.ops, ref, on_append=lambda i, s, n, sl: log_r.append(list(sl)))
    workloads.run_schedule(p.ops, nat, on_append=lambda i, s, n, sl: log_n.append(sl.tolist()))
    assert log_r == log_n
    assert _state(ref, p.seqs) == _state(nat, p.seqs)
    # chunk growth as one all-or-nothing batch per step
    s_r, c_r = ref.append_batch(p.seqs, [w.chunk] * len(p.seqs))
    s_n, c_n = nat.append_batch(p.seqs, [w.chunk] * len(p.seqs))
    assert list(s_r) == s_n.tolist() and c_r == c_n


def test_prepared_append_tables_repeats_the_call():
    """The marshalled-once variant used by serving loops writes the same
    slots, tables and lengths as the plain call, step after step, into the
    arrays it was given."""
    order = list(range(40))[::-1]
    a = pkv.BlockAllocator(40, 4, order)
    b = pkv.BlockAllocator(40, 4, order)
    for x in (a, b):
        for q in (7, 8):
            x.add(q)
        x.append(7, 5)
        x.fork(7, 9)  # shares 7's partly filled last block: copy-on-write below
    seqs, counts, mb = [7, 8, 9], [1, 2, 1], 8
    slots = np.empty(4, dtype=np.int32)
    tables = np.empty((3, mb), dtype=np.int32)
    lens = np.empty(3, dtype=np.int32)
    step = a.prepared_append_tables(seqs, counts, mb, slots, tables, lens)
    for _ in range(6):
        pairs = step()
        s2, p2, t2, l2 = b.append_batch_tables(seqs, counts, mb)
        assert pairs == p2
        assert slots.tolist() == s2.tolist()
        assert np.array_equal(tables, t2) and lens.tolist() == l2.tolist()
    assert a.snapshot() == b.snapshot()
    # a table would outgrow max_blocks: the failing call changes nothing
    while True:
        before = (a.snapshot(), [a.block_table(q) for q in seqs], [a.seq_len(q) for q in seqs])
        try:
            step()
        except pkv.BufferTooSmall:
            break
    assert before == (a.snapshot(), [a.block_table(q) for q in seqs],
                      [a.seq_len(q) for q in seqs])


def test_swap_walkthrough_through_the_c_abi():
    """The hand-worked swap walkthrough of the oracle tests, natively."""
    from test_oracle_allocator import _swap_walkthrough
    a = pkv.BlockAllocator(4, 2)
    ids = {"A": 1, "B": 2}

    class Named:  # the walkthrough names sequences by letter
        def __getattr__(self, name):
            f = getattr(a, name)
            return lambda *args: f(*[ids.get(x, x) if isinstance(x, str) else x for x in args])

        def set_host_pool(self, n):
            a.set_host_pool(n)

    _swap_walkthrough(Named())
    free, ref = a.snapshot()
    assert free == [1, 0] and ref == [0, 0, 1, 1]
    assert a.block_table(1) == [2, 3] and a.seq_len(1) == 3
    assert a.host_snapshot() == [1, 0, 2]
    assert not a.is_swapped(1)
    a.close()


def test_shared_prefix_decode_checks_its_arguments_before_launch():
    lib = pkv._lib
    null = None
    ws = ctypes.c_size_t()
    # shared-prefix batch geometry: 256 sequences, 32 heads, prefix 1024 in
    # blocks of 16, contexts up to 3000: 8 prefix ranges of 128 keys (a
    # workgroup per CU) + one 2048-token suffix partition; up to 3100, two
    # (the workspace starts with a 16-byte record per sequence)
    assert lib.pkv_paged_attention_decode_shared_prefix_workspace_size(
        256, 32, 32, 128, 16, 3000, 1024, 0, ctypes.byref(ws)) == 0
    assert ws.value == 256 * 16 + 256 * 32 * (8 + 1) * (128 + 2) * 4
    assert lib.pkv_paged_attention_decode_shared_prefix_workspace_size(
        256, 32, 32, 128, 16, 3100, 1024, 0, ctypes.byref(ws)) == 0
    assert ws.value == 256 * 16 + 256 * 32 * (8 + 2) * (128 + 2) * 4
    # one 64-key range when the prefix is one tile
    assert lib.pkv_paged_attention_decode_shared_prefix_workspace_size(
        4, 4, 4, 128, 16, 300, 64, 64, ctypes.byref(ws)) == 0
    assert ws.value == 4 * 16 + 4 * 4 * (1 + 4) * (128 + 2) * 4
    # prefix not a multiple of the block size, longer than the contexts
    assert lib.pkv_paged_attention_decode_shared_prefix_workspace_size(
        4, 4, 4, 128, 16, 300, 72, 0, ctypes.byref(ws)) == 1
    assert lib.pkv_paged_attention_decode_shared_prefix_workspace_size(
        4, 4, 4, 128, 16, 300, 320, 0, ctypes.byref(ws)) == 1
    args = (null, null, null, null, null)
    # float32 caches and head_dim 64 are not served by the matrix-core part
    assert lib.pkv_paged_attention_decode_shared_prefix(*args, 4, 4, 4, 128, 16, 32, 64, 300,
                                                        64, 1.0, 0, null, null, 0, 0,
                                                        null) == 7
    assert lib.pkv_paged_attention_decode_shared_prefix(*args, 4, 4, 4, 64, 16, 32, 64, 300,
                                                        64, 1.0, 0, null, null, 0, 2,
                                                        null) == 7
    # the hint is taken off the dtype; then the NULL pointers are caught
    assert lib.pkv_paged_attention_decode_shared_prefix(*args, 4, 4, 4, 128, 16, 32, 64, 300,
                                                        64, 1.0, 0, null, null, 0,
                                                        2 | pkv.DECODE_SHARED_BLOCKS,
                                                        null) == 1
    assert b"NULL" in lib.pkv_last_error()
    # empty batch: nothing to do
    assert lib.pkv_paged_attention_decode_shared_prefix(*args, 0, 4, 4, 128, 16, 32, 64, 300,
                                                        64, 1.0, 0, null, null, 0, 2,
                                                        null) == 0


def test_grouped_prefix_decode_checks_its_arguments_before_launch():
    lib = pkv._lib
    null = None
    ws = ctypes.c_size_t()

    def arr(xs):
        return (ctypes.c_int32 * len(xs))(*xs)

    # four groups of 64 of 256 sequences, prefixes 1024/512/1536/768,
    # contexts up to 3600: four row tiles x 32 heads = 128 (head, tile)
    # pairs, so 2 key ranges for the longest prefix (24 tiles of 64 keys ->
    # ranges of 768 keys; every prefix needs at most 2); suffixes up to
    # 3600 - 512 = 3088 tokens in 2048-token partitions: 2 + 2 slots
    starts, plens = arr([0, 64, 128, 192, 256]), arr([1024, 512, 1536, 768])
    assert lib.pkv_paged_attention_decode_grouped_prefix_workspace_size(
        256, 32, 32, 128, 16, 3600, 4, starts, plens, 0, ctypes.byref(ws)) == 0
    assert ws.value == 256 * 16 + 256 * 32 * (2 + 2) * (128 + 2) * 4
    # no prefix anywhere: no prefix slot, suffixes from token 0
    assert lib.pkv_paged_attention_decode_grouped_prefix_workspace_size(
        8, 4, 4, 128, 16, 300, 2, arr([0, 3, 8]), arr([0, 0]), 64, ctypes.byref(ws)) == 0
    assert ws.value == 8 * 16 + 8 * 4 * 5 * (128 + 2) * 4
    # bad groups: no group, too many, not starting at 0, not ending at
    # num_seqs, decreasing, a prefix off the block grid or past the contexts
    assert lib.pkv_paged_attention_decode_grouped_prefix_workspace_size(
        8, 4, 4, 128, 16, 300, 0, arr([0]), arr([0]), 0, ctypes.byref(ws)) == 1
    assert lib.pkv_paged_attention_decode_grouped_prefix_workspace_size(
        8, 4, 4, 128, 16, 300, 129, arr([0] * 129 + [8]), arr([0] * 129), 0,
        ctypes.byref(ws)) == 7
    for s_, p_ in (([1, 3, 8], [16, 32]), ([0, 3, 7], [16, 32]), ([0, 5, 3, 8], [16, 32, 0]),
                   ([0, 3, 8], [24, 32]), ([0, 3, 8], [16, 320]), ([0, 3, 8], [-16, 32])):
        assert lib.pkv_paged_attention_decode_grouped_prefix_workspace_size(
            8, 4, 4, 128, 16, 300, len(p_), arr(s_), arr(p_), 0, ctypes.byref(ws)) == 1, (s_, p_)
    assert lib.pkv_paged_attention_decode_grouped_prefix_workspace_size(
        8, 4, 4, 128, 16, 300, 2, null, arr([0, 0]), 0, ctypes.byref(ws)) == 1
    # block size 8 is not served by the matrix-core part
    assert lib.pkv_paged_attention_decode_grouped_prefix_workspace_size(
        8, 4, 4, 128, 8, 300, 2, arr([0, 3, 8]), arr([16, 32]), 0, ctypes.byref(ws)) == 7
    args = (null, null, null, null, null)
    g = (2, arr([0, 3, 8]), arr([16, 32]))
    # float32 caches are not served; NULL pointers are caught; an empty
    # batch does nothing
    assert lib.pkv_paged_attention_decode_grouped_prefix(*args, 8, 4, 4, 128, 16, 32, 64, 300,
                                                         *g, 1.0, 0, null, null, 0, 0,
                                                         null) == 7
    assert lib.pkv_paged_attention_decode_grouped_prefix(*args, 8, 4, 4, 128, 16, 32, 64, 300,
                                                         *g, 1.0, 0, null, null, 0, 2,
                                                         null) == 1
    assert lib.pkv_paged_attention_decode_grouped_prefix(*args, 0, 4, 4, 128, 16, 32, 64, 300,
                                                         1, arr([0, 0]), arr([16]), 1.0, 0, null,
                                                         null, 0, 2, null) == 0
    # step form: a new row inside a group's prefix, a change to a prefix
    # entry, both rejected before any launch (NULL device pointers here)
    lens = arr([20, 30, 40, 50, 60, 70, 80, 90])
    kv = ctypes.c_void_p(16)   # never dereferenced: the host checks fail first
    assert lib.pkv_paged_attention_decode_grouped_prefix_step(
        null, kv, kv, null, null, null, arr([16] + [20] * 7), null, 0, 8, 4, 4, 128, 16, 32, 64,
        300, *g, 1.0, 0, null, null, 0, 2, null) == 1
    assert b"no suffix position" in lib.pkv_last_error()
    assert lib.pkv_paged_attention_decode_grouped_prefix_step(
        null, null, null, null, null, null, lens, arr([4, 1, 7]), 1, 8, 4, 4, 128, 16, 32, 64,
        300, *g, 1.0, 0, null, null, 0, 2, null) == 1
    assert b"shared prefix" in lib.pkv_last_error()
