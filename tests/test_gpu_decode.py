"""GPU parity of paged_attention_decode against the float64 oracle.

Small cases run the whole oracle path (reference allocator, oracle append,
oracle paged decode over a NaN-poisoned pool) and compare every output
element.  Full-size workloads, in the launch configuration bench.py times,
compare sampled sequences against oracle attention over the sequence's
logical K/V drawn again from the generator.  Tolerances: 1e-5 max-abs for
float32 caches, 2e-3 for float16/bfloat16 caches (float32 accumulation).
"""

import math

import numpy as np
import pytest
import torch

import paged_kv_cache_420_amd as pkv
import workloads
from cases import (DEV, TOL, GpuState, OracleState, decode_queries, log, logical_kv,
                   logical_segments, max_abs_err)
from oracle import dense_attention, paged_decode

pytestmark = pytest.mark.gpu


def run_decode(g, w, seqs=None, partition_size=None, max_ctx=None):
    seqs = g.p.seqs if seqs is None else seqs
    tables, lens, _, lens_h = g.tables(seqs)
    q, q64 = decode_queries(w, seqs)
    mc = int(lens_h.max()) if max_ctx is None else max_ctx
    part = w.partition_size if partition_size is None else partition_size
    out = pkv.paged_attention_decode(q.to(DEV), g.kc, g.vc, tables, lens, w.scale, mc,
                                     partition_size=part)
    torch.cuda.synchronize()
    return out.cpu().numpy(), q64


SMALL = {
    "tiny_fp32": workloads.get("tiny_fp32"),
    "tiny_fp32_long": workloads.scaled(workloads.get("tiny_fp32"), num_seqs=5, num_blocks=0,
                                       lens="uniform:1,1300"),
    "llama7b_small": workloads.scaled(workloads.get("llama7b_bf16"), num_seqs=6, num_heads=4,
                                      num_kv_heads=4, lens="uniform:1,1600"),
    "llama13b_small": workloads.scaled(workloads.get("llama13b_fp16"), num_seqs=8, num_heads=3,
                                       num_kv_heads=3, lens="geometric:300,1,2000"),
    "gqa_small": workloads.scaled(workloads.get("gqa_bf16"), num_seqs=4, num_heads=16,
                                  num_kv_heads=2, lens="uniform:1,1500"),
    "gqa4_d64_bs8": workloads.scaled(workloads.get("gqa_bf16"), num_seqs=4, num_heads=8,
                                     num_kv_heads=2, head_dim=64, block_size=8,
                                     lens="uniform:1,900"),
    "gqa2_fp16_bs64": workloads.scaled(workloads.get("llama13b_fp16"), num_seqs=4, num_heads=4,
                                       num_kv_heads=2, block_size=64, lens="uniform:1,1200"),
    "fp32_d128_gqa8": workloads.scaled(workloads.get("tiny_fp32"), num_seqs=3, num_heads=16,
                                       num_kv_heads=2, head_dim=128, num_blocks=0,
                                       lens="uniform:1,700"),
    "bf16_bs256": workloads.scaled(workloads.get("llama7b_bf16"), num_seqs=3, num_heads=2,
                                   num_kv_heads=2, block_size=256, lens="uniform:1,1100"),
    "shared_prefix_small": workloads.scaled(workloads.get("shared_prefix_bf16"), num_seqs=6,
                                            num_heads=2, num_kv_heads=2, prefix=64,
                                            lens="uniform:10,700", chunk=0),
    "shared_prefix_cow": workloads.scaled(workloads.get("shared_prefix_bf16"), num_seqs=5,
                                          num_heads=2, num_kv_heads=2, prefix=40,
                                          lens="uniform:1,90", chunk=0),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_decode_matches_oracle(name):
    w = SMALL[name]
    log("case", name, w)
    p = workloads.plan(w)
    g = GpuState(w, p)
    o = OracleState(w, p)
    got, q64 = run_decode(g, w)
    tables, lens = o.tables()
    want = paged_decode(q64, o.kc, o.vc, tables, lens, w.scale, w.block_size)
    err = max_abs_err(got, want)
    log(name, "max abs err", err)
    assert err <= TOL[w.dtype]


@pytest.mark.parametrize("part", [64, 128, 256, 1024])
def test_partition_size_only_changes_rounding(part):
    w = SMALL["llama7b_small"]
    p = workloads.plan(w)
    g = GpuState(w, p)
    o = OracleState(w, p)
    got, q64 = run_decode(g, w, partition_size=part)
    tables, lens = o.tables()
    want = paged_decode(q64, o.kc, o.vc, tables, lens, w.scale, w.block_size)
    assert max_abs_err(got, want) <= TOL[w.dtype]


def test_block_placement_is_bitwise_invisible():
    # same logical content, different physical blocks (another free order)
    w = SMALL["gqa_small"]
    p1 = workloads.plan(w)
    p2 = workloads.plan(w)
    p2.free_order = np.ascontiguousarray(p2.free_order[::-1])
    a, _ = run_decode(GpuState(w, p1), w)
    b, _ = run_decode(GpuState(w, p2), w)
    assert np.array_equal(a, b)


def test_fork_is_bitwise_identical_to_parent():
    w = workloads.scaled(SMALL["llama7b_small"], num_seqs=1, lens="fixed:777")
    p = workloads.plan(w)
    p.ops = p.ops + [("fork", 0, 1), ("fork", 0, 2)]
    p.seqs = [0, 1, 2]
    g = GpuState(w, p)
    tables, lens, th, _ = g.tables()
    assert (th[1] == th[0]).all() and (th[2] == th[0]).all()
    q, _ = decode_queries(w, [0, 0, 0])
    out = pkv.paged_attention_decode(q.to(DEV), g.kc, g.vc, tables, lens, w.scale, 777)
    out = out.cpu().numpy()
    assert np.array_equal(out[0], out[1]) and np.array_equal(out[0], out[2])


def test_single_token_returns_its_value_exactly():
    w = workloads.scaled(SMALL["llama7b_small"], num_seqs=3, lens="fixed:1")
    p = workloads.plan(w)
    g = GpuState(w, p)
    got, _ = run_decode(g, w)
    segs = logical_segments(p.ops)
    for b in p.seqs:
        _, v = logical_kv(w, segs[b])
        assert np.array_equal(got[b], v[0])  # weight exp(0) = 1, sum 1


def test_zero_length_and_inconsistent_rows():
    w = workloads.scaled(SMALL["llama7b_small"], num_seqs=4, lens="fixed:40")
    p = workloads.plan(w)
    g = GpuState(w, p)
    tables, lens, _, _ = g.tables()
    lens[1] = 0                       # empty context: zeros
    lens[2] = 50                      # longer than max_context_len below: NaN
    bad_tables = tables.clone()
    bad_tables[3, 0] = p.num_blocks   # table entry outside the pool: NaN
    q, _ = decode_queries(w, p.seqs)
    out = pkv.paged_attention_decode(q.to(DEV), g.kc, g.vc, bad_tables, lens, w.scale, 45)
    out = out.cpu().numpy()
    assert np.isfinite(out[0]).all()
    assert (out[1] == 0).all()
    assert np.isnan(out[2]).all()
    assert np.isnan(out[3]).all()


def test_multi_partition_inconsistent_rows_are_nan():
    w = workloads.scaled(SMALL["llama7b_small"], num_seqs=2, lens="fixed:1500")
    p = workloads.plan(w)
    g = GpuState(w, p)
    tables, lens, _, _ = g.tables()
    tables[1, 40] = -7                # a block of the second partition
    q, _ = decode_queries(w, p.seqs)
    out = pkv.paged_attention_decode(q.to(DEV), g.kc, g.vc, tables, lens, w.scale, 1500,
                                     partition_size=512).cpu().numpy()
    assert np.isfinite(out[0]).all() and np.isnan(out[1]).all()


FULL = ["tiny_fp32", "llama7b_bf16", "llama13b_fp16", "gqa_bf16", "shared_prefix_bf16"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_against_oracle(name):
    w = workloads.get(name)
    if w.chunk:
        w = workloads.scaled(w, chunk=0)  # decode state; prefill is its own test
    log("full-size case", name)
    p = workloads.plan(w)
    g = GpuState(w, p)
    tables, lens, th, lh = g.tables()
    # allocator state at full size, bit-exact against the reference
    from oracle import RefAllocator
    ref = RefAllocator(p.num_blocks, w.block_size, p.free_order)
    workloads.run_schedule(p.ops, ref)
    rt, rl = ref.build_tables(p.seqs, th.shape[1])
    assert np.array_equal(np.array(rt, dtype=np.int32), th) and list(rl) == lh.tolist()
    got, q64 = run_decode(g, w)
    segs = logical_segments(p.ops)
    rng = np.random.default_rng(7)
    pick = sorted(set(rng.choice(len(p.seqs), size=min(8, len(p.seqs)), replace=False).tolist())
                  | {int(np.argmax(lh)), int(np.argmin(lh))})
    worst = 0.0
    for b in pick:
        k, v = logical_kv(w, segs[p.seqs[b]])
        want = dense_attention(q64[b][None], k, v, w.scale)[0]
        worst = max(worst, max_abs_err(got[b], want))
    log(name, "sampled max abs err", worst, "over", len(pick), "sequences")
    assert worst <= TOL[w.dtype]
    assert np.isfinite(got).all()
