"""Pins for the float64 attention oracle (CPU only).

Each test checks the oracle against something other than itself: a
hand-worked fixture, a closed form, torch's own scaled_dot_product_attention
in float64 (an independent library routine), or an invariant that a wrong
index, sign or dropped term would break.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from conftest import GOLDEN
from oracle import dense_attention, gather_kv, paged_decode, paged_prefill, slot_of


def _rng(seed):
    return np.random.default_rng(seed)


def _paged_from_contiguous(k, v, block_size, rng, spare=3):
    """Scatter contiguous [n, Hkv, D] K/V into a shuffled pool by hand
    (no oracle code), returning caches and the block table."""
    n, hkv, d = k.shape
    nblk = -(-n // block_size)
    pool = nblk + spare
    perm = rng.permutation(pool)
    table = perm[:nblk]
    kc = np.full((pool, hkv, block_size, d), np.nan)
    vc = np.full((pool, hkv, block_size, d), np.nan)
    for t in range(n):
        kc[table[t // block_size], :, t % block_size, :] = k[t]
        vc[table[t // block_size], :, t % block_size, :] = v[t]
    return kc, vc, table


def _sdpa(q, k, v, scale, causal=False, attn_mask=None):
    """torch SDPA, float64 CPU.  q [Lq, Hq, D], k/v [n, Hkv, D]."""
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None]
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None]
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=attn_mask, is_causal=causal,
                                       scale=scale, enable_gqa=True)
    return o[0].numpy().transpose(1, 0, 2)


# --- hand-worked fixtures -------------------------------------------------

def test_figure_page_table_fixture():
    fx = json.load(open(os.path.join(GOLDEN, "figure_page_table.json")))
    bs, table = fx["block_size"], fx["block_table"]
    for p, phys, row, slot in zip(fx["positions"], fx["expected_physical"],
                                  fx["expected_row"], fx["expected_slot"]):
        assert slot_of(table, p, bs) == slot
        assert slot == phys * bs + row
    # gather returns exactly the cache rows the figure names, in order
    nb, d = fx["num_blocks"], 2
    cache = np.zeros((nb, 1, bs, d))
    for b in range(nb):
        for r in range(bs):
            cache[b, 0, r] = [b, r]
    got = gather_kv(cache, table, fx["context_len"], bs)
    for p, phys, row in zip(fx["positions"], fx["expected_physical"], fx["expected_row"]):
        assert got[p, 0].tolist() == [phys, row]
    assert got.shape == (fx["context_len"], 1, d)


def test_two_key_softmax_fixture():
    fx = json.load(open(os.path.join(GOLDEN, "softmax_two_keys.json")))
    q = np.array(fx["q"])[None, None]
    k = np.array(fx["k"])[:, None]
    v = np.array(fx["v"])[:, None]
    out = dense_attention(q, k, v, fx["scale"])[0, 0]
    np.testing.assert_allclose(out, fx["expected_out"], rtol=0, atol=1e-14)


# --- closed forms -----------------------------------------------------------

def test_single_token_returns_its_value():
    rng = _rng(1)
    q = rng.normal(size=(1, 3, 8))
    k = rng.normal(size=(1, 3, 8))
    v = rng.normal(size=(1, 3, 8))
    assert np.array_equal(dense_attention(q, k, v, 0.7)[0], v[0])


@pytest.mark.parametrize("case", ["zero_q", "zero_scale", "equal_keys"])
def test_uniform_weights_give_mean_value(case):
    rng = _rng(2)
    n, h, d = 37, 2, 16
    q = rng.normal(size=(1, h, d))
    k = rng.normal(size=(n, h, d))
    v = rng.normal(size=(n, h, d))
    scale = 0.3
    if case == "zero_q":
        q[:] = 0
    elif case == "zero_scale":
        scale = 0.0
    else:
        k[:] = k[0]
    out = dense_attention(q, k, v, scale)[0]
    np.testing.assert_allclose(out, v.mean(axis=0), rtol=0, atol=1e-13)


def test_constant_values_are_reproduced():
    # weights sum to one: a missing or wrong normaliser breaks this
    rng = _rng(3)
    q = rng.normal(size=(4, 2, 8))
    k = rng.normal(size=(20, 2, 8)) * 3
    v = np.full((20, 2, 8), 2.5)
    np.testing.assert_allclose(dense_attention(q, k, v, 1.0), 2.5, rtol=0, atol=1e-13)


def test_sharp_softmax_selects_argmax():
    rng = _rng(4)
    n, d = 50, 8
    q = rng.normal(size=(1, 1, d))
    k = rng.normal(size=(n, 1, d))
    v = rng.normal(size=(n, 1, d))
    s = (k[:, 0] @ q[0, 0])
    out = dense_attention(q, k, v, 1e6)[0, 0]
    np.testing.assert_allclose(out, v[np.argmax(s), 0], rtol=0, atol=1e-12)


def test_sign_of_scores_matters():
    # the larger q.k must get the larger weight: flipping the sign of the
    # scores (or of the max shift) moves the output towards the other value
    q = np.array([[[1.0]]])
    k = np.array([[[2.0]], [[0.0]]])
    v = np.array([[[1.0]], [[0.0]]])
    out = dense_attention(q, k, v, 1.0)[0, 0, 0]
    assert out == pytest.approx(math.exp(2) / (math.exp(2) + 1), abs=1e-15)


def test_zero_length_context_outputs_zero():
    q = np.ones((1, 2, 4))
    k = np.zeros((0, 2, 4))
    assert np.array_equal(dense_attention(q, k, k, 1.0), np.zeros((1, 2, 4)))


# --- library routine: torch SDPA in float64 -------------------------------

@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2), (6, 1)])
@pytest.mark.parametrize("n", [1, 5, 16, 33, 100])
def test_decode_matches_torch_sdpa(hq, hkv, n):
    rng = _rng(100 + n + hq)
    d, bs = 16, 8
    q = rng.normal(size=(1, hq, d))
    k = rng.normal(size=(n, hkv, d))
    v = rng.normal(size=(n, hkv, d))
    scale = 1 / math.sqrt(d)
    kc, vc, table = _paged_from_contiguous(k, v, bs, rng)
    got = paged_decode(q, kc, vc, table[None], [n], scale, bs)[0]
    want = _sdpa(q, k, v, scale)[0]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (4, 2)])
@pytest.mark.parametrize("n", [1, 7, 40])
def test_prefill_from_empty_cache_matches_causal_sdpa(hq, hkv, n):
    rng = _rng(200 + n + hq)
    d, bs = 8, 4
    q = rng.normal(size=(n, hq, d))
    k = rng.normal(size=(n, hkv, d))
    v = rng.normal(size=(n, hkv, d))
    kc, vc, table = _paged_from_contiguous(k, v, bs, rng)
    got = paged_prefill(q, kc, vc, table[None], [n], [0, n], 0.4, bs)
    want = _sdpa(q, k, v, 0.4, causal=True)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_prefill_rows_independent_of_chunking():
    # a chunk [a, b) computed with the cache holding b tokens equals rows
    # a..b-1 of the whole prompt from an empty cache (pinned above by SDPA):
    # an off-by-one in the chunk's first position breaks this
    rng = _rng(5)
    n, h, d, bs = 29, 2, 8, 4
    q = rng.normal(size=(n, h, d))
    k = rng.normal(size=(n, h, d))
    v = rng.normal(size=(n, h, d))
    kc, vc, table = _paged_from_contiguous(k, v, bs, rng)
    full = _sdpa(q, k, v, 0.5, causal=True)
    for a, b in [(0, 1), (0, 12), (12, 13), (12, 29), (5, 20)]:
        got = paged_prefill(q[a:b], kc, vc, table[None], [b], [0, b - a], 0.5, bs)
        np.testing.assert_allclose(got, full[a:b], rtol=0, atol=1e-12)


def test_prefill_chunk_of_one_is_decode():
    rng = _rng(6)
    n, h, d, bs = 21, 3, 8, 4
    q = rng.normal(size=(1, h, d))
    k = rng.normal(size=(n, h, d))
    v = rng.normal(size=(n, h, d))
    kc, vc, table = _paged_from_contiguous(k, v, bs, rng)
    a = paged_prefill(q, kc, vc, table[None], [n], [0, 1], 0.3, bs)
    b = paged_decode(q, kc, vc, table[None], [n], 0.3, bs)
    np.testing.assert_array_equal(a, b)


def test_multi_sequence_batch_matches_sdpa_per_sequence():
    rng = _rng(7)
    hq, hkv, d, bs = 4, 2, 16, 16
    lens = [17, 33, 64, 100, 1]
    pool = sum(-(-n // bs) for n in lens) + 4
    perm = rng.permutation(pool)
    kc = np.full((pool, hkv, bs, d), np.nan)
    vc = np.full((pool, hkv, bs, d), np.nan)
    tables = np.full((len(lens), 8), -1)
    q = rng.normal(size=(len(lens), hq, d))
    ks, vs, used = [], [], 0
    for b, n in enumerate(lens):
        k = rng.normal(size=(n, hkv, d))
        v = rng.normal(size=(n, hkv, d))
        nblk = -(-n // bs)
        tables[b, :nblk] = perm[used:used + nblk]
        used += nblk
        for t in range(n):
            kc[tables[b, t // bs], :, t % bs] = k[t]
            vc[tables[b, t // bs], :, t % bs] = v[t]
        ks.append(k)
        vs.append(v)
    got = paged_decode(q, kc, vc, tables, lens, 0.25, bs)
    for b in range(len(lens)):
        want = _sdpa(q[b:b + 1], ks[b], vs[b], 0.25)[0]
        np.testing.assert_allclose(got[b], want, rtol=0, atol=1e-12)


def test_gather_rejects_out_of_pool_entries():
    cache = np.zeros((4, 1, 2, 1))
    with pytest.raises(ValueError):
        gather_kv(cache, [0, 4], 3, 2)
    with pytest.raises(ValueError):
        gather_kv(cache, [-1], 1, 2)
