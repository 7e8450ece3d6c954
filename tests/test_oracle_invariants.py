"""Paging and sharing invariants of the oracle, plus its append/copy
helpers, checked on the CPU.

* Physical placement must not matter: moving blocks around the pool (data
  and table together) leaves every output bitwise unchanged -- paging does
  not change the model's output (explainer, closing section; tutorial §1.4).
* Sharing must not matter: a fork that points at the parent's blocks gives
  the parent's output bit for bit, and a fork that then diverges matches an
  unshared copy (explainer, "内存共享" section).
"""

import numpy as np
import pytest

from oracle import (RefAllocator, copy_blocks, kv_append, paged_decode,
                    paged_prefill)


def _build(lens, hkv, d, bs, rng, spare=4):
    """Fill a pool through the reference allocator and oracle append."""
    pool = sum(-(-n // bs) for n in lens) + spare
    alloc = RefAllocator(pool, bs, rng.permutation(pool))
    kc = np.full((pool, hkv, bs, d), np.nan)
    vc = np.full((pool, hkv, bs, d), np.nan)
    for b, n in enumerate(lens):
        alloc.add(b)
        slots, pairs = alloc.append(b, n)
        assert pairs == []
        kv_append(kc, vc, rng.normal(size=(n, hkv, d)), rng.normal(size=(n, hkv, d)), slots, bs)
    maxb = max(-(-n // bs) for n in lens)
    tables, ls = alloc.build_tables(range(len(lens)), maxb)
    return kc, vc, np.array(tables), np.array(ls), alloc


def test_block_permutation_is_bitwise_invisible():
    rng = np.random.default_rng(21)
    lens, hq, hkv, d, bs = [17, 33, 64, 100], 4, 2, 16, 16
    kc, vc, tables, ls, _ = _build(lens, hkv, d, bs, rng)
    q = rng.normal(size=(len(lens), hq, d))
    base = paged_decode(q, kc, vc, tables, ls, 0.125, bs)
    perm = rng.permutation(kc.shape[0])          # new home of each block
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    tables2 = np.where(tables >= 0, perm[np.maximum(tables, 0)], -1)
    again = paged_decode(q, kc2, vc2, tables2, ls, 0.125, bs)
    assert np.array_equal(base, again)


def test_fork_at_equal_length_is_bitwise_identical():
    rng = np.random.default_rng(22)
    hkv, d, bs = 2, 8, 4
    kc, vc, tables, ls, alloc = _build([23], hkv, d, bs, rng, spare=6)
    alloc.fork(0, 1)
    t, l = alloc.build_tables([0, 1], tables.shape[1])
    q = np.repeat(rng.normal(size=(1, hkv, d)), 2, axis=0)
    out = paged_decode(q, kc, vc, np.array(t), l, 0.3, bs)
    assert np.array_equal(out[0], out[1])


def test_fork_then_diverge_matches_unshared_copy():
    rng = np.random.default_rng(23)
    hkv, d, bs, n0, extra = 2, 8, 4, 10, 7  # fork mid-block: copy-on-write
    pool = 20
    alloc = RefAllocator(pool, bs, rng.permutation(pool))
    kc = np.full((pool, hkv, bs, d), np.nan)
    vc = np.full((pool, hkv, bs, d), np.nan)
    k0, v0 = rng.normal(size=(n0, hkv, d)), rng.normal(size=(n0, hkv, d))
    k1, v1 = rng.normal(size=(extra, hkv, d)), rng.normal(size=(extra, hkv, d))
    alloc.add(0)
    s, _ = alloc.append(0, n0)
    kv_append(kc, vc, k0, v0, s, bs)
    alloc.fork(0, 1)
    s, pairs = alloc.append(1, extra)
    assert len(pairs) == 1
    copy_blocks(kc, vc, [p[0] for p in pairs], [p[1] for p in pairs])
    kv_append(kc, vc, k1, v1, s, bs)
    # the unshared twin: one sequence holding prefix + suffix by itself
    alloc.add(2)
    s, _ = alloc.append(2, n0 + extra)
    kv_append(kc, vc, np.concatenate([k0, k1]), np.concatenate([v0, v1]), s, bs)
    t, l = alloc.build_tables([0, 1, 2], 6)
    q = np.stack([rng.normal(size=(hkv, d))] * 3)
    out = paged_decode(q, kc, vc, np.array(t), l, 0.3, bs)
    assert np.array_equal(out[1], out[2])
    # the parent still sees only its own prefix
    assert l[0] == n0


def test_prefill_block_permutation_is_bitwise_invisible():
    rng = np.random.default_rng(24)
    lens, hq, hkv, d, bs = [9, 30], 2, 1, 8, 4
    kc, vc, tables, ls, _ = _build(lens, hkv, d, bs, rng)
    cu = [0, 5, 5 + 30]
    q = rng.normal(size=(35, hq, d))
    base = paged_prefill(q, kc, vc, tables, ls, cu, 0.5, bs)
    perm = rng.permutation(kc.shape[0])
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc
    tables2 = np.where(tables >= 0, perm[np.maximum(tables, 0)], -1)
    assert np.array_equal(base, paged_prefill(q, kc2, vc2, tables2, ls, cu, 0.5, bs))


def test_kv_append_places_rows_by_hand():
    kc = np.zeros((3, 1, 2, 1))
    vc = np.zeros((3, 1, 2, 1))
    k_new = np.array([[[1.0]], [[2.0]], [[3.0]]])
    kv_append(kc, vc, k_new, -k_new, [5, -1, 0], 2)
    assert kc[2, 0, 1, 0] == 1.0 and vc[2, 0, 1, 0] == -1.0   # slot 5 = block 2 row 1
    assert kc[0, 0, 0, 0] == 3.0                               # slot 0
    assert np.count_nonzero(kc) == 2                           # slot -1 skipped
    with pytest.raises(ValueError):
        kv_append(kc, vc, k_new[:2], k_new[:2], [1, 1], 2)
    with pytest.raises(ValueError):
        kv_append(kc, vc, k_new[:1], k_new[:1], [6], 2)


def test_copy_blocks_by_hand():
    kc = np.arange(12.0).reshape(3, 1, 2, 2)
    vc = -kc
    copy_blocks(kc, vc, [0], [2])
    assert np.array_equal(kc[2], kc[0]) and np.array_equal(vc[2], vc[0])
    assert kc[1, 0, 0, 0] == 4.0
    with pytest.raises(ValueError):
        copy_blocks(kc, vc, [0, 1], [2, 2])
    with pytest.raises(ValueError):
        copy_blocks(kc, vc, [0, 2], [2, 1])
