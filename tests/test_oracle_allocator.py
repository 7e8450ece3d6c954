"""Pins for the reference allocator (CPU only): the hand-worked trace in
tests/golden/allocator_trace.json, a closed-form block count for shared
prefixes, and invariants under random operation sequences."""

import json
import os

import pytest
from hypothesis import given, settings, strategies as st

from conftest import GOLDEN
from oracle import OutOfBlocks, RefAllocator


def _cdiv(a, b):
    return -(-a // b)


def check_invariants(a):
    """Counting invariants that any correct block allocator must keep."""
    held = {}
    for seq, table in a.tables.items():
        assert len(table) == _cdiv(a.lens[seq], a.block_size)
        assert len(set(table)) == len(table)
        for b in table:
            held[b] = held.get(b, 0) + 1
    for b in range(a.num_blocks):
        assert a.ref[b] == held.get(b, 0)
    free = a.free_stack()
    assert len(set(free)) == len(free)
    assert set(free) == {b for b in range(a.num_blocks) if a.ref[b] == 0}
    assert len(free) + sum(1 for r in a.ref if r > 0) == a.num_blocks


def test_hand_worked_trace():
    fx = json.load(open(os.path.join(GOLDEN, "allocator_trace.json")))
    a = RefAllocator(fx["num_blocks"], fx["block_size"], fx["init_order"])
    for step in fx["steps"]:
        op = step["op"]
        if op == "add":
            a.add(step["seq"])
        elif op == "fork":
            a.fork(step["parent"], step["child"])
        elif op == "free":
            a.free(step["seq"])
        elif op == "append":
            if step.get("expect_error") == "out_of_blocks":
                with pytest.raises(OutOfBlocks):
                    a.append(step["seq"], step["n"])
            else:
                slots, pairs = a.append(step["seq"], step["n"])
                assert slots == step["slots"]
                assert [list(p) for p in pairs] == step["cow"]
        assert a.free_stack() == step["free"], step
        assert a.ref == step["ref"], step
        want = {s: (t, n) for s, (t, n) in step["tables"].items()}
        assert {s: (a.table(s), a.length(s)) for s in a.tables} == want, step
        check_invariants(a)


def test_shared_prefix_block_count_closed_form():
    # 1024-token prefix (block aligned) shared by 256 forks, each then grows
    # a private suffix: blocks in use = 1024/16 + sum ceil(s/16), against
    # 256 * 64 + sum ceil(s/16) if every sequence stored its own prefix.
    import numpy as np
    bs = 16
    suffix = np.random.default_rng(11).integers(10, 2000, endpoint=True, size=256)
    need = 64 + int(sum(_cdiv(int(s), bs) for s in suffix))
    a = RefAllocator(need + 5, bs)
    a.add("prefix")
    a.append("prefix", 1024)
    for i in range(256):
        a.fork("prefix", i)
    a.free("prefix")
    for i, s in enumerate(suffix):
        _, pairs = a.append(i, int(s))
        assert pairs == []  # the prefix ends on a block boundary: no copy
    assert a.num_blocks - a.num_free() == need
    prefix_blocks = a.table(0)[:64]
    for i in range(256):
        assert a.table(i)[:64] == prefix_blocks
    for b in prefix_blocks:
        assert a.ref[b] == 256
    check_invariants(a)


def test_out_of_blocks_changes_nothing():
    a = RefAllocator(4, 4, [2, 0, 3, 1])
    a.add(0)
    a.append(0, 9)
    before = a.snapshot()
    with pytest.raises(OutOfBlocks):
        a.append(0, 8)
    assert a.snapshot() == before
    a.add(1)
    before = a.snapshot()
    with pytest.raises(OutOfBlocks):
        a.append_batch([1, 0], [3, 4])  # 1 fits, then 0 needs 1 more: 2 > 1
    assert a.snapshot() == before


def test_cow_only_when_shared_and_partial():
    a = RefAllocator(10, 4)
    a.add(0)
    a.append(0, 8)           # exactly two full blocks
    a.fork(0, 1)
    _, pairs = a.append(1, 1)
    assert pairs == []        # aligned: the new token starts a fresh block
    a.add(2)
    a.append(2, 5)
    a.fork(2, 3)
    a.fork(2, 4)
    _, p3 = a.append(3, 2)
    _, p4 = a.append(4, 1)
    _, p2 = a.append(2, 1)
    assert len(p3) == 1 and len(p4) == 1 and p2 == []  # last holder writes in place
    check_invariants(a)


def test_released_blocks_are_reused_at_once():
    # explainer: a finished request's blocks return to the pool and any free
    # block can serve any request
    a = RefAllocator(3, 2, [0, 1, 2])
    a.add("x")
    a.append("x", 6)
    assert a.num_free() == 0
    a.free("x")
    a.add("y")
    slots, _ = a.append("y", 6)
    assert sorted(s // 2 for s in slots[::2]) == [0, 1, 2]


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        RefAllocator(3, 2, [0, 0, 1])
    a = RefAllocator(3, 2)
    a.add(1)
    with pytest.raises(ValueError):
        a.add(1)
    with pytest.raises(KeyError):
        a.append(2, 1)
    with pytest.raises(KeyError):
        a.free(2)
    with pytest.raises(ValueError):
        a.fork(1, 1)
    with pytest.raises(ValueError):
        a.append_batch([1, 1], [1, 1])


# --- random operation sequences ------------------------------------------------

ops = st.lists(
    st.tuples(st.sampled_from(["add", "append", "fork", "free"]),
              st.integers(0, 5), st.integers(0, 5), st.integers(0, 23)),
    min_size=1, max_size=60)


@settings(max_examples=300, deadline=None)
@given(ops, st.integers(1, 8), st.integers(1, 24), st.randoms(use_true_random=False))
def test_random_ops_keep_invariants(seq_ops, block_size, num_blocks, rnd):
    order = list(range(num_blocks))
    rnd.shuffle(order)
    a = RefAllocator(num_blocks, block_size, order)
    for op, s, t, n in seq_ops:
        before = a.snapshot()
        try:
            if op == "add":
                a.add(s)
            elif op == "fork":
                a.fork(s, t)
            elif op == "free":
                a.free(s)
            else:
                old_table = a.table(s) if s in a.tables else None
                slots, pairs = a.append(s, n)
                start = a.length(s) - n
                # every written slot lies in a block this sequence owns alone
                for i, slot in enumerate(slots):
                    blk = slot // block_size
                    assert a.ref[blk] == 1
                    assert slot % block_size == (start + i) % block_size
                    assert a.table(s)[(start + i) // block_size] == blk
                # earlier positions keep their blocks, except a copied last one
                for j, b in enumerate(old_table):
                    if pairs and j == len(old_table) - 1:
                        assert pairs == [(b, a.table(s)[j])]
                    else:
                        assert a.table(s)[j] == b
        except (OutOfBlocks, KeyError, ValueError):
            assert a.snapshot() == before
        check_invariants(a)


def _swap_walkthrough(a):
    """Worked by hand (device pool 4 blocks, block 0 first; block size 2;
    host pool 3 blocks, host block 0 first): a sequence shared by a fork is
    swapped out and back while its sibling grows."""
    a.set_host_pool(3)
    a.add("A")
    slots, _ = a.append("A", 3)
    assert list(slots) == [0, 1, 2]                      # blocks 0, 1
    a.fork("A", "B")                                     # both hold [0, 1]
    assert [tuple(int(x) for x in p) for p in a.swap_out("A")] == [(0, 0), (1, 1)]
    # A's host blocks 0, 1; device blocks stay with B (counts back to 1)
    slots, pairs = a.append("B", 1)
    assert list(slots) == [3] and len(pairs) == 0         # no longer shared: no copy
    assert [tuple(int(x) for x in p) for p in a.swap_in("A")] == [(0, 2), (1, 3)]
    a.free("B")                                          # pushes 0 then 1


def test_swap_walkthrough_worked_by_hand():
    a = RefAllocator(4, 2)
    _swap_walkthrough(a)
    free, ref, tables = a.snapshot()
    assert free == [1, 0] and ref == [0, 0, 1, 1]
    assert tables == {"A": ([2, 3], 3)}
    assert a.host_free_stack() == [1, 0, 2]


def test_swapped_sequence_is_frozen_and_frees_host_blocks():
    a = RefAllocator(6, 2)
    a.set_host_pool(2)
    a.add(1)
    a.append(1, 4)                                       # blocks 0, 1
    a.add(3)
    a.append(3, 5)                                       # blocks 2, 3, 4
    before = a.snapshot()
    with pytest.raises(OutOfBlocks):
        a.swap_out(3)                                    # 3 blocks, host pool of 2
    assert a.snapshot() == before and a.host_free_stack() == [0, 1]
    a.swap_out(1)
    assert a.free_stack() == [1, 0, 5]
    for bad in (lambda: a.append(1, 1), lambda: a.fork(1, 9), lambda: a.build_tables([1], 4),
                lambda: a.append_batch([1], [1]), lambda: a.swap_out(1)):
        with pytest.raises(ValueError):
            bad()
    a.free(1)
    assert a.host_free_stack() == [1, 0] and 1 not in a.tables
