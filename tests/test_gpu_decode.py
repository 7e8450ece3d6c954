"""GPU parity of paged_attention_decode against the float64 oracle.

Small cases run the whole oracle path (reference allocator, oracle append,
oracle paged decode over a NaN-poisoned pool) and compare every output
element.  Full-size workloads, in the launch configuration bench.py times,
compare every sequence and head against oracle attention over the
sequence's logical K/V drawn again from the generator.  Tolerances: 1e-5 max-abs for
float32 caches, 2e-3 for float16/bfloat16 caches (float32 accumulation).
"""

import math

import numpy as np
import pytest
import torch

import paged_kv_cache_420_amd as pkv
import workloads
from cases import (DEV, TOL, GpuState, LogicalKV, OracleState, decode_queries, log,
                   logical_kv, logical_segments, max_abs_err, parallel_map)
from oracle import dense_attention, paged_decode

pytestmark = pytest.mark.gpu


def run_decode(g, w, seqs=None, partition_size=None, max_ctx=None, shared_blocks=False):
    seqs = g.p.seqs if seqs is None else seqs
    tables, lens, _, lens_h = g.tables(seqs)
    q, q64 = decode_queries(w, seqs)
    mc = int(lens_h.max()) if max_ctx is None else max_ctx
    part = w.partition_size if partition_size is None else partition_size
    out = pkv.paged_attention_decode(q.to(DEV), g.kc, g.vc, tables, lens, w.scale, mc,
                                     partition_size=part, shared_blocks=shared_blocks)
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


# Every (cache type, head_dim, query heads per kv head) the decode kernels
# are compiled for: the score reduction and the combine across a wave's
# token rows change shape with the lanes per row (4 .. 32) and with G, so
# each instantiation meets the oracle at least once.  Partitions of 128
# tokens with lengths up to 400 cover one- and multi-partition rows.
SWEEP = [(dt, d, g) for dt in (torch.bfloat16, torch.float16, torch.float32)
         for d in (64, 128) for g in (1, 2, 4, 8)]


@pytest.mark.parametrize("dt,d,grp", SWEEP,
                         ids=[f"{str(dt)[6:]}-d{d}-g{g}" for dt, d, g in SWEEP])
def test_every_instantiation_matches_oracle(dt, d, grp):
    w = workloads.scaled(workloads.get("llama7b_bf16"), num_seqs=3, num_kv_heads=2,
                         num_heads=2 * grp, head_dim=d, dtype=dt, lens="uniform:1,400",
                         seed=4300 + d + grp)
    log("case", w)
    p = workloads.plan(w)
    g = GpuState(w, p)
    o = OracleState(w, p)
    got, q64 = run_decode(g, w, partition_size=128)
    tables, lens = o.tables()
    want = paged_decode(q64, o.kc, o.vc, tables, lens, w.scale, w.block_size)
    err = max_abs_err(got, want)
    log("max abs err", err)
    assert err <= TOL[w.dtype]
    # the cached-load instantiation (shared-blocks hint): the same bits
    hinted, _ = run_decode(g, w, partition_size=128, shared_blocks=True)
    assert np.array_equal(hinted, got)


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
def test_full_size_every_sequence_against_oracle(name):
    """Each workload at full size over a NaN-poisoned pool: every sequence
    and every head of the plain decode call, and of the second of two
    steps of the step call in the launch configuration bench.py times
    (batch append with table changes, each new K/V row stored by the
    kernel, the library's partition size and the grid order that goes with
    it, the shared-blocks hint when blocks are shared), against oracle
    attention over the sequence's logical K/V drawn again from the
    generator (paging leaves the result unchanged)."""
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

    # the step path, two steps
    seqs = p.seqs
    nb = len(seqs)
    mb = th.shape[1] + 2
    t0, _ = g.alloc.build_block_tables(seqs, mb)
    dev_tables = torch.from_numpy(t0.copy()).to(DEV)
    shared = any(r > 1 for r in g.alloc.snapshot()[1])
    ones = np.ones(nb, dtype=np.int32)
    new_k, new_v = [], []
    for i in range(2):
        k, v = workloads.kv_rows(w, len(p.ops) + i, nb)
        kt, vt = workloads.to_dtype(k, w.dtype), workloads.to_dtype(v, w.dtype)
        new_k.append(workloads.as_f64(kt))
        new_v.append(workloads.as_f64(vt))
        qt = workloads.to_dtype(workloads.normal([w.seed, 11, i], (nb, w.num_heads, w.head_dim),
                                                 w.std), w.dtype)
        _, pairs, step_lens, changes = g.alloc.append_batch_changes(seqs, ones)
        if pairs:
            g._copy(pairs)
        out = pkv.paged_attention_decode_step(qt.to(DEV), kt.to(DEV), vt.to(DEV), g.kc, g.vc,
                                              dev_tables, step_lens, changes, w.scale,
                                              int(step_lens.max()),
                                              partition_size=w.partition_size,
                                              shared_blocks=shared)
    torch.cuda.synchronize()
    got_step = out.cpu().numpy()
    q64_step = workloads.as_f64(qt)

    lkv = LogicalKV(w, p.ops)

    def errors(b):
        k, v = lkv.get(seqs[b])
        plain = dense_attention(q64[b][None], k, v, w.scale)[0]
        k = np.concatenate([k] + [x[b][None] for x in new_k])
        v = np.concatenate([v] + [x[b][None] for x in new_v])
        step = dense_attention(q64_step[b][None], k, v, w.scale)[0]
        return max_abs_err(got[b], plain), max_abs_err(got_step[b], step)

    errs = np.array(parallel_map(errors, range(nb)))
    log(name, "every sequence and head:", nb, "sequences; max abs err plain",
        errs[:, 0].max(), "step", errs[:, 1].max(), "shared hint", shared)
    assert errs[:, 0].max() <= TOL[w.dtype]
    assert errs[:, 1].max() <= TOL[w.dtype]


# ---------------------------------------------------------------------------
# one-call decode vs its two stages; decode with the append fused in
# ---------------------------------------------------------------------------

MULTI = {
    "bf16_part64": (workloads.scaled(workloads.get("llama7b_bf16"), num_seqs=6, num_heads=4,
                                     num_kv_heads=4, lens="uniform:1,900"), 64),
    "gqa8_part128": (workloads.scaled(workloads.get("gqa_bf16"), num_seqs=5, num_heads=16,
                                      num_kv_heads=2, lens="uniform:100,1500"), 128),
    "fp32_d64_part256": (workloads.scaled(workloads.get("tiny_fp32"), num_seqs=5, num_blocks=0,
                                          lens="uniform:1,1300"), 256),
}


@pytest.mark.parametrize("name", list(MULTI))
def test_one_call_is_bitwise_its_two_stages(name):
    w, part = MULTI[name]
    log("case", name)
    p = workloads.plan(w)
    g = GpuState(w, p)
    tables, lens, _, lh = g.tables()
    q, _ = decode_queries(w, p.seqs)
    q = q.to(DEV)
    mc = int(lh.max())
    one = pkv.paged_attention_decode(q, g.kc, g.vc, tables, lens, w.scale, mc, partition_size=part)
    need = pkv.paged_attention_decode_workspace_size(len(p.seqs), w.num_heads, w.num_kv_heads,
                                                     w.head_dim, mc, part)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    two = torch.empty_like(one)
    pkv.paged_attention_decode_partials(q, g.kc, g.vc, tables, lens, w.scale, mc, part, two, ws)
    pkv.paged_attention_decode_merge(lens, w.num_kv_heads, w.block_size, tables.shape[1], mc, part,
                                     two, ws)
    torch.cuda.synchronize()
    assert torch.equal(one, two)


def test_workspace_contents_never_matter():
    # garbage, a previous call's partials or a previous shape's partials
    w, part = MULTI["bf16_part64"]
    p = workloads.plan(w)
    g = GpuState(w, p)
    tables, lens, _, lh = g.tables()
    q, _ = decode_queries(w, p.seqs)
    q = q.to(DEV)
    mc = int(lh.max())
    ref = pkv.paged_attention_decode(q, g.kc, g.vc, tables, lens, w.scale, mc, partition_size=part)
    need = pkv.paged_attention_decode_workspace_size(len(p.seqs), w.num_heads, w.num_kv_heads,
                                                     w.head_dim, mc, part)
    ws = torch.full((need + 4096,), 0xFF, dtype=torch.uint8, device=DEV)
    for fill in (0xFF, 0x00, 0x5A):
        ws.fill_(fill)
        for _ in range(3):
            got = pkv.paged_attention_decode(q, g.kc, g.vc, tables, lens, w.scale, mc,
                                             partition_size=part, workspace=ws)
            assert torch.equal(got, ref)
    # a smaller batch through the same workspace, then the full one again
    small = pkv.paged_attention_decode(q[:2].contiguous(), g.kc, g.vc, tables[:2].contiguous(),
                                       lens[:2].contiguous(), w.scale, mc, partition_size=part,
                                       workspace=ws)
    assert torch.equal(small, ref[:2])
    got = pkv.paged_attention_decode(q, g.kc, g.vc, tables, lens, w.scale, mc,
                                     partition_size=part, workspace=ws)
    assert torch.equal(got, ref)
    # random garbage
    ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device=DEV))
    got = pkv.paged_attention_decode(q, g.kc, g.vc, tables, lens, w.scale, mc,
                                     partition_size=part, workspace=ws)
    assert torch.equal(got, ref)


APPEND = {
    "bf16_auto": (workloads.scaled(workloads.get("llama7b_bf16"), num_seqs=7, num_heads=4,
                                   num_kv_heads=4, lens="uniform:0,1500"), 0),
    "bf16_part64": (MULTI["bf16_part64"][0], 64),
    "gqa8_part128": (MULTI["gqa8_part128"][0], 128),
    "fp16_bs32": (workloads.scaled(workloads.get("llama13b_fp16"), num_seqs=6, num_heads=2,
                                   num_kv_heads=2, lens="uniform:0,700"), 0),
    "fp32_d64_bs8": (workloads.scaled(workloads.get("tiny_fp32"), num_seqs=4, num_blocks=0,
                                      block_size=8, lens="uniform:0,300"), 64),
}


@pytest.mark.parametrize("name", list(APPEND))
def test_decode_append_is_append_then_decode(name):
    """Fused append == pkv_paged_kv_append at the allocator's slots followed by
    pkv_paged_attention_decode: pools and outputs bit for bit, and the
    output within tolerance of the oracle after the oracle's append."""
    w, part = APPEND[name]
    log("case", name)
    p = workloads.plan(w)
    a = GpuState(w, p)
    b = GpuState(w, p)
    o = OracleState(w, p)
    seqs = p.seqs
    slots_a, pairs_a = a.alloc.append_batch(seqs, np.ones(len(seqs), dtype=np.int32))
    slots_b, pairs_b = b.alloc.append_batch(seqs, np.ones(len(seqs), dtype=np.int32))
    slots_o, pairs_o = o.alloc.append_batch(seqs, [1] * len(seqs))
    assert not pairs_a and not pairs_b and not pairs_o
    assert slots_a.tolist() == slots_b.tolist() == list(slots_o)
    k, v = workloads.kv_rows(w, len(p.ops), len(seqs))  # [B, Hkv, D]
    kt, vt = workloads.to_dtype(k, w.dtype), workloads.to_dtype(v, w.dtype)
    q, q64 = decode_queries(w, seqs)
    q = q.to(DEV)
    # a: two calls
    pkv.paged_kv_append(kt.to(DEV), vt.to(DEV), a.kc, a.vc, torch.from_numpy(slots_a).to(DEV))
    ta, la, _, lh = a.tables()
    mc = int(lh.max())
    out_a = pkv.paged_attention_decode(q, a.kc, a.vc, ta, la, w.scale, mc, partition_size=part)
    # b: one launch
    tb, lb, _, _ = b.tables()
    out_b = pkv.paged_attention_decode_append(q, kt.to(DEV), vt.to(DEV), b.kc, b.vc, tb, lb,
                                              w.scale, mc, partition_size=part)
    # c: the fused call's two stages
    c = GpuState(w, p)
    c.alloc.append_batch(seqs, np.ones(len(seqs), dtype=np.int32))
    tc, lc, _, _ = c.tables()
    need = pkv.paged_attention_decode_workspace_size(len(seqs), w.num_heads, w.num_kv_heads,
                                                     w.head_dim, mc, part)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    out_c = torch.empty_like(out_b)
    pkv.paged_attention_decode_append_partials(q, kt.to(DEV), vt.to(DEV), c.kc, c.vc, tc, lc,
                                               w.scale, mc, part, out_c, ws)
    pkv.paged_attention_decode_merge(lc, w.num_kv_heads, w.block_size, tc.shape[1], mc, part,
                                     out_c, ws)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b) and torch.equal(out_b, out_c)
    for x in (b, c):
        assert torch.equal(a.kc.view(torch.uint8), x.kc.view(torch.uint8))
        assert torch.equal(a.vc.view(torch.uint8), x.vc.view(torch.uint8))
    # oracle
    from oracle import kv_append as o_append
    o_append(o.kc, o.vc, workloads.as_f64(kt), workloads.as_f64(vt), slots_o, w.block_size)
    tables, lens = o.tables()
    want = paged_decode(q64, o.kc, o.vc, tables, lens, w.scale, w.block_size)
    err = max_abs_err(out_b.cpu().numpy(), want)
    log(name, "max abs err", err)
    assert err <= TOL[w.dtype]


def test_launcher_is_the_plain_calls():
    """DecodeLauncher (arguments marshalled once) launches exactly what
    paged_attention_decode(_append) launch: bitwise equal outputs."""
    w, part = APPEND["gqa8_part128"]
    p = workloads.plan(w)
    a, b = GpuState(w, p), GpuState(w, p)
    seqs = p.seqs
    for x in (a, b):
        x.alloc.append_batch(seqs, np.ones(len(seqs), dtype=np.int32))
    k, v = workloads.kv_rows(w, len(p.ops), len(seqs))
    kt = workloads.to_dtype(k, w.dtype).to(DEV)
    vt = workloads.to_dtype(v, w.dtype).to(DEV)
    q, _ = decode_queries(w, seqs)
    q = q.to(DEV)
    ta, la, _, lh = a.tables()
    tb, lb, _, _ = b.tables()
    mc = int(lh.max())
    want = pkv.paged_attention_decode_append(q, kt, vt, a.kc, a.vc, ta, la, w.scale, mc,
                                             partition_size=part)
    need = pkv.paged_attention_decode_workspace_size(len(seqs), w.num_heads, w.num_kv_heads,
                                                     w.head_dim, mc + 50, part)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(want)
    launch = pkv.DecodeLauncher(b.kc, b.vc, w.num_heads, len(seqs), tb.shape[1], mc + 50, part,
                                out, ws)
    launch.partials(q, tb, lb, mc, w.scale, kt, vt)
    launch.merge(lb, mc)
    torch.cuda.synchronize()
    assert torch.equal(out, want)
    assert torch.equal(a.kc.view(torch.uint8), b.kc.view(torch.uint8))
    # a decode without the append through the same launcher
    plain = pkv.paged_attention_decode(q, a.kc, a.vc, ta, la, w.scale, mc, partition_size=part)
    launch.partials(q, tb, lb, mc, w.scale)
    launch.merge(lb, mc)
    torch.cuda.synchronize()
    assert torch.equal(out, plain)
    with pytest.raises(pkv.InvalidArgument):
        launch.partials(q, tb, lb, mc + 51, w.scale)


STEP = {
    # 40-token prefix forked into every sequence: not block aligned, so the
    # first append of a sequence with no suffix yet copies the shared last
    # block during the steps (a table change that replaces an entry); 20
    # steps cross block boundaries
    "bf16_shared_cow": workloads.scaled(workloads.get("shared_prefix_bf16"), num_seqs=6,
                                        num_heads=4, num_kv_heads=4, prefix=40,
                                        lens="fixed:0,0,5,100,0,37", chunk=0),
    "gqa8_fp16_bs32": workloads.scaled(workloads.get("llama13b_fp16"), num_seqs=5, num_heads=16,
                                       num_kv_heads=2, lens="uniform:0,900"),
}


# (workload, steps, partition): 64-token partitions keep the grid
# partition-major; 1024-token ones over contexts up to 3000 take the grid
# that dispatches a sequence's partitions together
STEP_RUNS = {"bf16_shared_cow": ("bf16_shared_cow", 20, 64),
             "gqa8_fp16_bs32": ("gqa8_fp16_bs32", 20, 64),
             "bf16_long_part1024": ("bf16_long", 4, 1024)}
STEP["bf16_long"] = workloads.scaled(workloads.get("llama7b_bf16"), num_seqs=7, num_heads=4,
                                     num_kv_heads=2, lens="uniform:1,3000")


@pytest.mark.parametrize("run", list(STEP_RUNS))
def test_step_call_is_full_upload_decode(run):
    """pkv_paged_attention_decode_step (lengths and table changes by value,
    a device table kept across steps) == pkv_paged_attention_decode_append
    with freshly uploaded tables, bit for bit: outputs, caches and, at the
    end, the device table itself."""
    name, steps, part = STEP_RUNS[run]
    w = STEP[name]
    log("case", name, steps, part)
    p = workloads.plan(w)
    a, b = GpuState(w, p), GpuState(w, p)
    seqs = p.seqs
    mb = max(len(a.alloc.block_table(s)) for s in seqs) + steps // w.block_size + 2
    th, _ = b.alloc.build_block_tables(seqs, mb)
    dev_tables = torch.from_numpy(th.copy()).to(DEV)   # b's table, kept on the device
    ones = np.ones(len(seqs), dtype=np.int32)
    for i in range(steps):
        k, v = workloads.kv_rows(w, len(p.ops) + i, len(seqs))
        kt = workloads.to_dtype(k, w.dtype).to(DEV)
        vt = workloads.to_dtype(v, w.dtype).to(DEV)
        q = workloads.to_dtype(workloads.normal([w.seed, 9, i], (len(seqs), w.num_heads,
                                                                  w.head_dim), w.std),
                               w.dtype).to(DEV)
        _, pa = a.alloc.append_batch(seqs, ones)
        _, pb, lens, changes = b.alloc.append_batch_changes(seqs, ones)
        assert pa == pb
        for x, pairs in ((a, pa), (b, pb)):
            if pairs:
                x._copy(pairs)
        ta, la, _, lh = a.tables(seqs)
        ta = torch.nn.functional.pad(ta, (0, mb - ta.shape[1]), value=-1).contiguous()
        mc = int(lh.max())
        want = pkv.paged_attention_decode_append(q, kt, vt, a.kc, a.vc, ta, la, w.scale, mc,
                                                 partition_size=part)
        got = pkv.paged_attention_decode_step(q, kt, vt, b.kc, b.vc, dev_tables, lens, changes,
                                              w.scale, mc, partition_size=part)
        torch.cuda.synchronize()
        assert lens.tolist() == lh.tolist()
        assert torch.equal(got, want), f"step {i}"
    assert torch.equal(a.kc.view(torch.uint8), b.kc.view(torch.uint8))
    assert torch.equal(a.vc.view(torch.uint8), b.vc.view(torch.uint8))
    th, _ = b.alloc.build_block_tables(seqs, mb)
    assert np.array_equal(dev_tables.cpu().numpy(), th)


def test_step_call_limits():
    w = STEP["bf16_shared_cow"]
    kc = torch.zeros((8, 4, 16, 128), dtype=torch.bfloat16, device=DEV)
    q = torch.zeros((300, 4, 128), dtype=torch.bfloat16, device=DEV)
    t = torch.zeros((300, 200), dtype=torch.int32, device=DEV)
    lens = np.ones(300, dtype=np.int32)
    # 193 changes for one sequence: more than one launch can carry
    many = np.array([[0, j, 1] for j in range(193)], dtype=np.int32)
    with pytest.raises(pkv.Unsupported):
        pkv.paged_attention_decode_step(q, None, None, kc, kc, t, lens, many, w.scale, 1)
    with pytest.raises(pkv.InvalidArgument):  # change row outside the batch
        pkv.paged_attention_decode_step(q[:2].contiguous(), None, None, kc, kc, t[:2].contiguous(),
                                        lens[:2], np.array([[5, 0, 1]]), w.scale, 1)


def test_step_call_past_256_sequences():
    """512 sequences: the step call runs as launches of 256 ranks of the
    longest-first order, each with its ranks' lengths and changes.  Over
    three steps it equals the fused-append decode on freshly uploaded
    tables bit for bit (outputs, caches, device table), and the last
    step's every row meets the oracle."""
    w = workloads.scaled(workloads.get("llama7b_bf16"), num_seqs=512, num_heads=4,
                         num_kv_heads=2, lens="uniform:1,700", seed=4610)
    p = workloads.plan(w)
    a, b = GpuState(w, p), GpuState(w, p)
    seqs = p.seqs
    nb, steps, part = len(seqs), 3, 256
    mb = max(len(a.alloc.block_table(s)) for s in seqs) + 2
    th, _ = b.alloc.build_block_tables(seqs, mb)
    dev_tables = torch.from_numpy(th.copy()).to(DEV)
    ones = np.ones(nb, dtype=np.int32)
    new_k, new_v = [], []
    for i in range(steps):
        k, v = workloads.kv_rows(w, len(p.ops) + i, nb)
        kt, vt = workloads.to_dtype(k, w.dtype), workloads.to_dtype(v, w.dtype)
        new_k.append(workloads.as_f64(kt))
        new_v.append(workloads.as_f64(vt))
        kt, vt = kt.to(DEV), vt.to(DEV)
        qt = workloads.to_dtype(workloads.normal([w.seed, 9, i], (nb, w.num_heads, w.head_dim),
                                                 w.std), w.dtype)
        a.alloc.append_batch(seqs, ones)
        _, _, lens, changes = b.alloc.append_batch_changes(seqs, ones)
        ta, la, _, lh = a.tables(seqs)
        ta = torch.nn.functional.pad(ta, (0, mb - ta.shape[1]), value=-1).contiguous()
        mc = int(lh.max())
        want = pkv.paged_attention_decode_append(qt.to(DEV), kt, vt, a.kc, a.vc, ta, la, w.scale,
                                                 mc, partition_size=part)
        got = pkv.paged_attention_decode_step(qt.to(DEV), kt, vt, b.kc, b.vc, dev_tables, lens,
                                              changes, w.scale, mc, partition_size=part)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"step {i}"
    assert torch.equal(a.kc.view(torch.uint8), b.kc.view(torch.uint8))
    assert torch.equal(a.vc.view(torch.uint8), b.vc.view(torch.uint8))
    th, _ = b.alloc.build_block_tables(seqs, mb)
    assert np.array_equal(dev_tables.cpu().numpy(), th)
    got = got.cpu().numpy()
    q64 = workloads.as_f64(qt)
    lkv = LogicalKV(w, p.ops)

    def err(r):
        k, v = lkv.get(seqs[r])
        k = np.concatenate([k] + [x[r][None] for x in new_k])
        v = np.concatenate([v] + [x[r][None] for x in new_v])
        return max_abs_err(got[r], dense_attention(q64[r][None], k, v, w.scale)[0])

    worst = max(parallel_map(err, range(nb)))
    log("512-sequence step, every row: max abs err", worst)
    assert worst <= TOL[w.dtype]


def test_step_mapped_is_step_on_mapped_rows():
    """pkv_paged_attention_decode_step_mapped: 300 sequences whose tables
    sit in scattered rows of a 400-row device table (the rest garbage),
    lengths in lockstep so that every sequence opens a block at the first
    step (300 changes: launches cut by the change limit) -- bitwise the
    fused-append decode on freshly uploaded tables, over four steps; the
    mapped rows end up holding the sequences' tables, the others
    untouched."""
    w = workloads.scaled(workloads.get("llama7b_bf16"), num_seqs=300, num_heads=4,
                         num_kv_heads=2, lens="fixed:32,64,96,128,160,480", seed=4611)
    p = workloads.plan(w)
    a, b = GpuState(w, p), GpuState(w, p)
    seqs = p.seqs
    nb, steps = len(seqs), 4
    mb = max(len(a.alloc.block_table(s)) for s in seqs) + 2
    rows_total = 400
    table_rows = np.random.default_rng(7).permutation(rows_total)[:nb].astype(np.int32)
    th, _ = b.alloc.build_block_tables(seqs, mb)
    lane = np.full((rows_total, mb), -7, dtype=np.int32)
    lane[table_rows] = th
    lane_d = torch.from_numpy(lane.copy()).to(DEV)
    ones = np.ones(nb, dtype=np.int32)
    for i in range(steps):
        k, v = workloads.kv_rows(w, len(p.ops) + i, nb)
        kt = workloads.to_dtype(k, w.dtype).to(DEV)
        vt = workloads.to_dtype(v, w.dtype).to(DEV)
        qt = workloads.to_dtype(workloads.normal([w.seed, 9, i], (nb, w.num_heads, w.head_dim),
                                                 w.std), w.dtype).to(DEV)
        a.alloc.append_batch(seqs, ones)
        _, _, lens, changes = b.alloc.append_batch_changes(seqs, ones)
        if i == 0:
            assert len(changes) == nb        # every sequence opened a block
        ta, la, _, lh = a.tables(seqs)
        ta = torch.nn.functional.pad(ta, (0, mb - ta.shape[1]), value=-1).contiguous()
        mc = int(lh.max())
        want = pkv.paged_attention_decode_append(qt, kt, vt, a.kc, a.vc, ta, la, w.scale, mc,
                                                 partition_size=128)
        got = pkv.paged_attention_decode_step_mapped(qt, kt, vt, b.kc, b.vc, lane_d, table_rows,
                                                     lens, changes, w.scale, mc,
                                                     partition_size=128)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"step {i}"
    assert torch.equal(a.kc.view(torch.uint8), b.kc.view(torch.uint8))
    assert torch.equal(a.vc.view(torch.uint8), b.vc.view(torch.uint8))
    th, _ = b.alloc.build_block_tables(seqs, mb)
    lane_now = lane_d.cpu().numpy()
    assert np.array_equal(lane_now[table_rows], th)
    rest = np.setdiff1d(np.arange(rows_total), table_rows)
    assert (lane_now[rest] == -7).all()
    with pytest.raises(pkv.InvalidArgument):          # a repeated row
        bad = table_rows.copy()
        bad[1] = bad[0]
        pkv.paged_attention_decode_step_mapped(qt, None, None, b.kc, b.vc, lane_d, bad, lens,
                                               np.zeros((0, 3), np.int32), w.scale, mc)
    with pytest.raises(pkv.InvalidArgument):          # a row outside the table
        bad = table_rows.copy()
        bad[3] = rows_total
        pkv.paged_attention_decode_step_mapped(qt, None, None, b.kc, b.vc, lane_d, bad, lens,
                                               np.zeros((0, 3), np.int32), w.scale, mc)


def test_shared_prefix_step_past_256_sequences():
    """The shared-prefix step form over 300 sequences (two launches of the
    suffix kernel and of the merge): bitwise the append followed by the
    plain shared-prefix call on freshly uploaded tables."""
    w = workloads.scaled(workloads.get("shared_prefix_bf16"), num_seqs=300, num_heads=4,
                         num_kv_heads=2, prefix=48, lens="uniform:1,400", chunk=0, seed=4611)
    p = workloads.plan(w)
    a, b = GpuState(w, p), GpuState(w, p)
    seqs = p.seqs
    nb, steps = len(seqs), 2
    mb = max(len(a.alloc.block_table(s)) for s in seqs) + 2
    th, _ = b.alloc.build_block_tables(seqs, mb)
    dev_tables = torch.from_numpy(th.copy()).to(DEV)
    ones = np.ones(nb, dtype=np.int32)
    for i in range(steps):
        k, v = workloads.kv_rows(w, len(p.ops) + i, nb)
        kt = workloads.to_dtype(k, w.dtype).to(DEV)
        vt = workloads.to_dtype(v, w.dtype).to(DEV)
        q = workloads.to_dtype(workloads.normal([w.seed, 17, i], (nb, w.num_heads, w.head_dim),
                                                w.std), w.dtype).to(DEV)
        slots, pa = a.alloc.append_batch(seqs, ones)
        _, pb, lens, changes = b.alloc.append_batch_changes(seqs, ones)
        assert not pa and not pb
        pkv.paged_kv_append(kt, vt, a.kc, a.vc, torch.from_numpy(slots).to(DEV))
        ta, la, _, lh = a.tables(seqs)
        ta = torch.nn.functional.pad(ta, (0, mb - ta.shape[1]), value=-1).contiguous()
        mc = int(lh.max())
        want = pkv.paged_attention_decode_shared_prefix(q, a.kc, a.vc, ta, la, w.prefix, w.scale,
                                                        mc, partition_size=128)
        got = pkv.paged_attention_decode_shared_prefix_step(q, kt, vt, b.kc, b.vc, dev_tables,
                                                            lens, changes, w.prefix, w.scale,
                                                            mc, partition_size=128)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"step {i}"
    th, _ = b.alloc.build_block_tables(seqs, mb)
    assert np.array_equal(dev_tables.cpu().numpy(), th)


def test_launcher_step_rejects_bad_host_arrays():
    """DecodeLauncher's step stages read host lengths and changes through
    raw pointers: wrong dtype, shape or count is refused before the call."""
    w, part = APPEND["gqa8_part128"]
    p = workloads.plan(w)
    g = GpuState(w, p)
    seqs = p.seqs
    nb = len(seqs)
    tables, lens, _, lh = g.tables()
    mc = int(lh.max())
    need = pkv.paged_attention_decode_workspace_size(nb, w.num_heads, w.num_kv_heads,
                                                     w.head_dim, mc, part)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    out = torch.empty((nb, w.num_heads, w.head_dim), dtype=torch.float32, device=DEV)
    launch = pkv.DecodeLauncher(g.kc, g.vc, w.num_heads, nb, tables.shape[1], mc, part, out, ws)
    q, _ = decode_queries(w, seqs)
    q = q.to(DEV)
    good_l = lh.astype(np.int32).copy()
    good_c = np.zeros((1, 3), dtype=np.int32)
    for bad_l in (lh.astype(np.int64), good_l[:-1].copy(), good_l.tolist()):
        with pytest.raises(pkv.InvalidArgument):
            launch.step_partials(q, tables, bad_l, good_c, 0, mc, w.scale)
        with pytest.raises(pkv.InvalidArgument):
            launch.step_merge(bad_l, mc)
    for bad_c, n in ((good_c.astype(np.int64), 0), (np.zeros((2, 2), dtype=np.int32), 0),
                     (good_c, 2), (good_c, -1)):
        with pytest.raises(pkv.InvalidArgument):
            launch.step_partials(q, tables, good_l, bad_c, n, mc, w.scale)
    launch.step_partials(q, tables, good_l, good_c, 0, mc, w.scale)
    launch.step_merge(good_l, mc)
    torch.cuda.synchronize()
    want = pkv.paged_attention_decode(q, g.kc, g.vc, tables, lens, w.scale, mc,
                                      partition_size=part)
    assert torch.equal(out, want)


HINT = ["tiny_fp32_long", "llama13b_small", "gqa_small", "gqa4_d64_bs8", "shared_prefix_small"]


@pytest.mark.parametrize("name", HINT)
def test_shared_blocks_hint_changes_no_bit(name):
    """PKV_DECODE_SHARED_BLOCKS launches the cached-load kernel; it must
    give exactly the output of the streaming-load kernel (the same
    arithmetic), in one call and split into partials + merge."""
    w = SMALL[name]
    log("case", name)
    g = GpuState(w, workloads.plan(w))
    tables, lens, _, lens_h = g.tables()
    q, _ = decode_queries(w, g.p.seqs)
    q = q.to(DEV)
    mc = int(lens_h.max())
    for part in (64, 0):
        want = pkv.paged_attention_decode(q, g.kc, g.vc, tables, lens, w.scale, mc,
                                          partition_size=part)
        got = pkv.paged_attention_decode(q, g.kc, g.vc, tables, lens, w.scale, mc,
                                         partition_size=part, shared_blocks=True)
        torch.cuda.synchronize()
        assert torch.equal(got, want), part


def test_shared_blocks_hint_step_and_launcher():
    """The hint on the step call and on a DecodeLauncher: bitwise the
    unhinted calls, steps with copy-on-write included."""
    w = STEP["bf16_shared_cow"]
    p = workloads.plan(w)
    a, b = GpuState(w, p), GpuState(w, p)
    seqs = p.seqs
    steps, part = 6, 64
    mb = max(len(a.alloc.block_table(s)) for s in seqs) + steps // w.block_size + 2
    dev = []
    for x in (a, b):
        th, _ = x.alloc.build_block_tables(seqs, mb)
        dev.append(torch.from_numpy(th.copy()).to(DEV))
    ones = np.ones(len(seqs), dtype=np.int32)
    for i in range(steps):
        k, v = workloads.kv_rows(w, len(p.ops) + i, len(seqs))
        kt = workloads.to_dtype(k, w.dtype).to(DEV)
        vt = workloads.to_dtype(v, w.dtype).to(DEV)
        q = workloads.to_dtype(workloads.normal([w.seed, 9, i], (len(seqs), w.num_heads,
                                                                  w.head_dim), w.std),
                               w.dtype).to(DEV)
        outs = []
        for x, t, hint in ((a, dev[0], False), (b, dev[1], True)):
            _, pairs, lens, changes = x.alloc.append_batch_changes(seqs, ones)
            if pairs:
                x._copy(pairs)
            outs.append(pkv.paged_attention_decode_step(
                q, kt, vt, x.kc, x.vc, t, lens, changes, w.scale, int(lens.max()),
                partition_size=part, shared_blocks=hint))
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1]), f"step {i}"
    tables, lens, _, lh = b.tables(seqs)
    tables = torch.nn.functional.pad(tables, (0, mb - tables.shape[1]), value=-1).contiguous()
    mc = int(lh.max())
    q, _ = decode_queries(w, seqs)
    q = q.to(DEV)
    want = pkv.paged_attention_decode(q, b.kc, b.vc, tables, lens, w.scale, mc,
                                      partition_size=part)
    need = pkv.paged_attention_decode_workspace_size(len(seqs), w.num_heads, w.num_kv_heads,
                                                     w.head_dim, mc, part)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(want)
    launch = pkv.DecodeLauncher(b.kc, b.vc, w.num_heads, len(seqs), mb, mc, part, out, ws,
                                shared_blocks=True)
    launch.partials(q, tables, lens, mc, w.scale)
    launch.merge(lens, mc)
    torch.cuda.synchronize()
    assert torch.equal(out, want)


@pytest.mark.parametrize("part", [64, 1024])
def test_step_two_stages_are_the_one_call(part):
    """DecodeLauncher.step_partials + step_merge (the two launches bench.py
    times) == pkv_paged_attention_decode_step in one call, bit for bit, over
    steps where some sequences span several partitions and others one (the
    merge covers the leading ranks of the longest-first order only)."""
    w = STEP["bf16_long"]
    p = workloads.plan(w)
    a, b = GpuState(w, p), GpuState(w, p)
    seqs = p.seqs
    nb, steps = len(seqs), 3
    mb = max(len(a.alloc.block_table(s)) for s in seqs) + 2
    mc_bound = max(a.alloc.seq_len(s) for s in seqs) + steps
    dev = []
    for x in (a, b):
        th, _ = x.alloc.build_block_tables(seqs, mb)
        dev.append(torch.from_numpy(th.copy()).to(DEV))
    need = pkv.paged_attention_decode_workspace_size(nb, w.num_heads, w.num_kv_heads, w.head_dim,
                                                     mc_bound, part)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    out = torch.empty((nb, w.num_heads, w.head_dim), dtype=torch.float32, device=DEV)
    launch = pkv.DecodeLauncher(b.kc, b.vc, w.num_heads, nb, mb, mc_bound, part, out, ws)
    ones = np.ones(nb, dtype=np.int32)
    for i in range(steps):
        k, v = workloads.kv_rows(w, len(p.ops) + i, nb)
        kt = workloads.to_dtype(k, w.dtype).to(DEV)
        vt = workloads.to_dtype(v, w.dtype).to(DEV)
        q = workloads.to_dtype(workloads.normal([w.seed, 13, i], (nb, w.num_heads, w.head_dim),
                                                w.std), w.dtype).to(DEV)
        _, _, la, ca = a.alloc.append_batch_changes(seqs, ones)
        _, _, lb, cb = b.alloc.append_batch_changes(seqs, ones)
        mc = int(la.max())
        want = pkv.paged_attention_decode_step(q, kt, vt, a.kc, a.vc, dev[0], la, ca, w.scale, mc,
                                               partition_size=part)
        launch.step_partials(q, dev[1], lb, cb, len(cb), mc, w.scale, kt, vt)
        launch.step_merge(lb, mc)
        torch.cuda.synchronize()
        assert (la > part).any() and (la <= part).any() or part == 64
        assert torch.equal(out, want), f"step {i}"


@pytest.mark.parametrize("dt,d,grp", SWEEP,
                         ids=[f"{str(dt)[6:]}-d{d}-g{g}" for dt, d, g in SWEEP])
def test_step_every_instantiation_is_full_upload_decode(dt, d, grp):
    """Every step-form instantiation (lengths and table changes by value),
    streaming and cached loads alternating by step, against the decode with
    the append fused and freshly uploaded tables: the same bits, with
    128-token partitions so that the merge runs."""
    w = workloads.scaled(workloads.get("llama7b_bf16"), num_seqs=3, num_kv_heads=2,
                         num_heads=2 * grp, head_dim=d, dtype=dt, lens="uniform:1,400",
                         seed=4500 + d + grp)
    log("case", w)
    p = workloads.plan(w)
    a, b = GpuState(w, p), GpuState(w, p)
    seqs = p.seqs
    steps, part = 4, 128
    mb = max(len(a.alloc.block_table(s)) for s in seqs) + 2
    th, _ = b.alloc.build_block_tables(seqs, mb)
    dev_tables = torch.from_numpy(th.copy()).to(DEV)
    ones = np.ones(len(seqs), dtype=np.int32)
    for i in range(steps):
        k, v = workloads.kv_rows(w, len(p.ops) + i, len(seqs))
        kt = workloads.to_dtype(k, w.dtype).to(DEV)
        vt = workloads.to_dtype(v, w.dtype).to(DEV)
        q = workloads.to_dtype(workloads.normal([w.seed, 9, i], (len(seqs), w.num_heads,
                                                                  w.head_dim), w.std),
                               w.dtype).to(DEV)
        a.alloc.append_batch(seqs, ones)
        _, _, lens, changes = b.alloc.append_batch_changes(seqs, ones)
        ta, la, _, lh = a.tables(seqs)
        ta = torch.nn.functional.pad(ta, (0, mb - ta.shape[1]), value=-1).contiguous()
        mc = int(lh.max())
        want = pkv.paged_attention_decode_append(q, kt, vt, a.kc, a.vc, ta, la, w.scale, mc,
                                                 partition_size=part)
        got = pkv.paged_attention_decode_step(q, kt, vt, b.kc, b.vc, dev_tables, lens, changes,
                                              w.scale, mc, partition_size=part,
                                              shared_blocks=bool(i % 2))
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"step {i}"


# ---------------------------------------------------------------------------
# decode with a prefix shared by every sequence (matrix-core prefix part,
# split-K suffixes, merge)
# ---------------------------------------------------------------------------

SHARED = {
    "bf16_mha_bs16": workloads.scaled(workloads.get("shared_prefix_bf16"), num_seqs=6,
                                      num_heads=4, num_kv_heads=4, prefix=64,
                                      lens="uniform:0,300", chunk=0),
    "f16_gqa8_bs32": workloads.scaled(workloads.get("shared_prefix_bf16"), num_seqs=5,
                                      num_heads=16, num_kv_heads=2, block_size=32, prefix=96,
                                      dtype=torch.float16, lens="uniform:1,500", chunk=0),
    "bf16_gqa2_long_prefix": workloads.scaled(workloads.get("shared_prefix_bf16"), num_seqs=4,
                                              num_heads=4, num_kv_heads=2, prefix=400 - 400 % 16,
                                              lens="uniform:0,200", chunk=0),
}


@pytest.mark.parametrize("name", list(SHARED))
@pytest.mark.parametrize("part", [64, 0])
def test_shared_prefix_decode_matches_oracle(name, part):
    """pkv_paged_attention_decode_shared_prefix against the oracle's paged
    decode over the same NaN-poisoned pool: the prefix part (float16 weights
    on the matrix cores) and the suffix partials merged; sequences with no
    suffix token included."""
    w = SHARED[name]
    log("case", name, part)
    p = workloads.plan(w)
    g = GpuState(w, p)
    o = OracleState(w, p)
    tables, lens, _, lh = g.tables()
    q, q64 = decode_queries(w, p.seqs)
    mc = int(lh.max())
    need = pkv.paged_attention_decode_shared_prefix_workspace_size(
        len(p.seqs), w.num_heads, w.num_kv_heads, w.head_dim, w.block_size, mc, w.prefix, part)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)   # NaN garbage
    got = pkv.paged_attention_decode_shared_prefix(q.to(DEV), g.kc, g.vc, tables, lens, w.prefix,
                                                   w.scale, mc, partition_size=part,
                                                   workspace=ws)
    torch.cuda.synchronize()
    ot, ol = o.tables()
    want = paged_decode(q64, o.kc, o.vc, ot, ol, w.scale, w.block_size)
    err = max_abs_err(got.cpu().numpy(), want)
    log(name, "max abs err", err)
    assert err <= TOL[w.dtype]
    # the suffix load hint changes no bit
    hinted = pkv.paged_attention_decode_shared_prefix(q.to(DEV), g.kc, g.vc, tables, lens,
                                                      w.prefix, w.scale, mc, partition_size=part,
                                                      shared_blocks=True)
    torch.cuda.synchronize()
    assert torch.equal(hinted, got)


def test_shared_prefix_decode_rows_below_the_prefix_are_nan():
    w = SHARED["bf16_mha_bs16"]
    p = workloads.plan(w)
    g = GpuState(w, p)
    tables, lens, _, lh = g.tables()
    q, q64 = decode_queries(w, p.seqs)
    bad = lens.clone()
    bad[1] = w.prefix - 1                      # shorter than the shared prefix
    mc = int(lh.max())
    got = pkv.paged_attention_decode_shared_prefix(q.to(DEV), g.kc, g.vc, tables, bad, w.prefix,
                                                   w.scale, mc).cpu().numpy()
    assert np.isnan(got[1]).all()
    ok_rows = [i for i in range(len(p.seqs)) if i != 1]
    assert np.isfinite(got[ok_rows]).all()
    with pytest.raises(pkv.InvalidArgument):   # not a multiple of the block size
        pkv.paged_attention_decode_shared_prefix(q.to(DEV), g.kc, g.vc, tables, lens,
                                                 w.prefix - 8, w.scale, mc)


def test_shared_prefix_decode_full_size_every_sequence():
    """The shared-prefix batch at full size (256 sequences, 1024-token
    prefix) over a NaN-poisoned pool: every sequence and head of the plain
    shared-prefix call, and of the second of two steps of its step form as
    bench.py times it (new rows stored by the suffix kernel, table changes
    by value), against oracle attention over the logical K/V drawn again
    from the generator."""
    w = workloads.scaled(workloads.get("shared_prefix_bf16"), chunk=0)
    p = workloads.plan(w)
    g = GpuState(w, p)
    tables, lens, th, lh = g.tables()
    q, q64 = decode_queries(w, p.seqs)
    mc = int(lh.max())
    got = pkv.paged_attention_decode_shared_prefix(q.to(DEV), g.kc, g.vc, tables, lens, w.prefix,
                                                   w.scale, mc).cpu().numpy()
    seqs = p.seqs
    nb = len(seqs)
    steps = 2
    mb = th.shape[1] + 2
    t0, _ = g.alloc.build_block_tables(seqs, mb)
    dev_tables = torch.from_numpy(t0.copy()).to(DEV)
    max_len = mc + steps
    ws = torch.empty(pkv.paged_attention_decode_shared_prefix_workspace_size(
        nb, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size, max_len, w.prefix),
        dtype=torch.uint8, device=DEV)
    out = torch.empty((nb, w.num_heads, w.head_dim), dtype=torch.float32, device=DEV)
    ones = np.ones(nb, dtype=np.int32)
    new_k, new_v = [], []
    for i in range(steps):
        k, v = workloads.kv_rows(w, len(p.ops) + i, nb)
        kt, vt = workloads.to_dtype(k, w.dtype), workloads.to_dtype(v, w.dtype)
        new_k.append(workloads.as_f64(kt))
        new_v.append(workloads.as_f64(vt))
        qt = workloads.to_dtype(workloads.normal([w.seed, 19, i], (nb, w.num_heads, w.head_dim),
                                                 w.std), w.dtype)
        _, pairs, step_lens, changes = g.alloc.append_batch_changes(seqs, ones)
        assert not pairs
        pkv.paged_attention_decode_shared_prefix_step(
            qt.to(DEV), kt.to(DEV), vt.to(DEV), g.kc, g.vc, dev_tables, step_lens, changes,
            w.prefix, w.scale, int(step_lens.max()), out=out, workspace=ws)
    torch.cuda.synchronize()
    got_step = out.cpu().numpy()
    q64_step = workloads.as_f64(qt)
    lkv = LogicalKV(w, p.ops)

    def errors(b):
        k, v = lkv.get(seqs[b])
        plain = dense_attention(q64[b][None], k, v, w.scale)[0]
        k = np.concatenate([k] + [x[b][None] for x in new_k])
        v = np.concatenate([v] + [x[b][None] for x in new_v])
        step = dense_attention(q64_step[b][None], k, v, w.scale)[0]
        return max_abs_err(got[b], plain), max_abs_err(got_step[b], step)

    errs = np.array(parallel_map(errors, range(nb)))
    log("shared-prefix decode, full size, every sequence and head: max abs err plain",
        errs[:, 0].max(), "step", errs[:, 1].max())
    assert errs[:, 0].max() <= TOL[w.dtype]
    assert errs[:, 1].max() <= TOL[w.dtype]


def test_shared_prefix_table_mismatch_gives_nan_rows():
    """The prefix is read through row 0 of the table; a sequence whose own
    table names other blocks for it gets a NaN row (plain and step form),
    whether or not it has suffix tokens; the other rows are unchanged."""
    w = SHARED["bf16_mha_bs16"]
    p = workloads.plan(w)
    g = GpuState(w, p)
    tables, lens, th, lh = g.tables()
    q, _ = decode_queries(w, p.seqs)
    q = q.to(DEV)
    mc = int(lh.max())
    want = pkv.paged_attention_decode_shared_prefix(q, g.kc, g.vc, tables, lens, w.prefix,
                                                    w.scale, mc)
    # rows other than 0 (row 0's table is the one the prefix is read through)
    long_ = 1 + int(np.argmax(lh[1:]))
    short = 1 if long_ != 1 else 2
    bad = tables.clone()
    bad[long_, 1] = bad[long_, 2]          # a prefix entry of a row with suffix tokens
    bad_lens = lens.clone()
    bad_lens[short] = w.prefix             # no suffix token: only the prefix partial
    bad[short, 0] = int(th[long_, -1])
    got = pkv.paged_attention_decode_shared_prefix(q, g.kc, g.vc, bad, bad_lens, w.prefix,
                                                   w.scale, mc)
    torch.cuda.synchronize()
    got, want = got.cpu().numpy(), want.cpu().numpy()
    assert np.isnan(got[long_]).all() and np.isnan(got[short]).all()
    rest = [i for i in range(len(p.seqs)) if i not in (short, long_)]
    assert np.array_equal(got[rest], want[rest])
    # step form (no new rows; the same device table)
    lens_h = lh.astype(np.int32).copy()
    lens_h[short] = w.prefix
    got = pkv.paged_attention_decode_shared_prefix_step(
        q, None, None, g.kc, g.vc, bad, lens_h, np.zeros((0, 3), dtype=np.int32), w.prefix,
        w.scale, mc).cpu().numpy()
    assert np.isnan(got[long_]).all() and np.isnan(got[short]).all()
    assert np.array_equal(got[rest], want[rest])


def test_shared_prefix_step_rejects_prefix_writes():
    w = SHARED["bf16_mha_bs16"]
    p = workloads.plan(w)
    g = GpuState(w, p)
    tables, lens, th, lh = g.tables()
    q, _ = decode_queries(w, p.seqs)
    q = q.to(DEV)
    nb = len(p.seqs)
    kv = torch.zeros((nb, w.num_kv_heads, w.head_dim), dtype=w.dtype, device=DEV)
    lens_h = lh.astype(np.int32).copy()
    no_changes = np.zeros((0, 3), dtype=np.int32)
    mc = int(lh.max())
    short = lens_h.copy()
    short[0] = w.prefix                    # the new row would land inside the prefix
    with pytest.raises(pkv.InvalidArgument):
        pkv.paged_attention_decode_shared_prefix_step(q, kv, kv, g.kc, g.vc, tables, short,
                                                      no_changes, w.prefix, w.scale, mc)
    with pytest.raises(pkv.InvalidArgument):  # a change to a prefix entry
        pkv.paged_attention_decode_shared_prefix_step(
            q, None, None, g.kc, g.vc, tables, lens_h, np.array([[1, 0, 3]], dtype=np.int32),
            w.prefix, w.scale, mc)
    with pytest.raises(pkv.InvalidArgument):  # out of the wrong shape
        pkv.paged_attention_decode_shared_prefix(q, g.kc, g.vc, tables, lens, w.prefix, w.scale,
                                                 mc, out=torch.empty((nb - 1, w.num_heads,
                                                                      w.head_dim),
                                                                     device=DEV))
    with pytest.raises(pkv.InvalidArgument):
        pkv.paged_attention_decode_shared_prefix_step(
            q, None, None, g.kc, g.vc, tables, lens_h, no_changes, w.prefix, w.scale, mc,
            out=torch.empty((nb, w.num_heads + 1, w.head_dim), device=DEV))


@pytest.mark.parametrize("part", [64, 1024])
def test_shared_prefix_step_is_append_then_shared_prefix_call(part):
    """pkv_paged_attention_decode_shared_prefix_step (host lengths and
    table changes by value, the new rows stored by the suffix kernel, a
    device table kept across steps) == the append followed by the plain
    shared-prefix call on freshly uploaded tables, bit for bit, over steps
    that open new blocks; 1024-token partitions take the grid that
    dispatches a sequence's partitions together."""
    w = workloads.scaled(workloads.get("shared_prefix_bf16"), num_seqs=5, num_heads=8,
                         num_kv_heads=4, prefix=128, lens="uniform:0,1500", chunk=0)
    p = workloads.plan(w)
    a, b = GpuState(w, p), GpuState(w, p)
    seqs = p.seqs
    steps = 20
    mb = max(len(a.alloc.block_table(s)) for s in seqs) + steps // w.block_size + 2
    th, _ = b.alloc.build_block_tables(seqs, mb)
    dev_tables = torch.from_numpy(th.copy()).to(DEV)
    ones = np.ones(len(seqs), dtype=np.int32)
    for i in range(steps):
        k, v = workloads.kv_rows(w, len(p.ops) + i, len(seqs))
        kt = workloads.to_dtype(k, w.dtype).to(DEV)
        vt = workloads.to_dtype(v, w.dtype).to(DEV)
        q = workloads.to_dtype(workloads.normal([w.seed, 17, i], (len(seqs), w.num_heads,
                                                                   w.head_dim), w.std),
                               w.dtype).to(DEV)
        slots, pa = a.alloc.append_batch(seqs, ones)
        _, pb, lens, changes = b.alloc.append_batch_changes(seqs, ones)
        assert not pa and not pb                 # the prefix is block aligned: no copies
        pkv.paged_kv_append(kt, vt, a.kc, a.vc, torch.from_numpy(slots).to(DEV))
        ta, la, _, lh = a.tables(seqs)
        ta = torch.nn.functional.pad(ta, (0, mb - ta.shape[1]), value=-1).contiguous()
        mc = int(lh.max())
        want = pkv.paged_attention_decode_shared_prefix(q, a.kc, a.vc, ta, la, w.prefix, w.scale,
                                                        mc, partition_size=part)
        got = pkv.paged_attention_decode_shared_prefix_step(q, kt, vt, b.kc, b.vc, dev_tables,
                                                            lens, changes, w.prefix, w.scale,
                                                            mc, partition_size=part)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"step {i}"
    assert torch.equal(a.kc.view(torch.uint8), b.kc.view(torch.uint8))
    assert torch.equal(a.vc.view(torch.uint8), b.vc.view(torch.uint8))
    th, _ = b.alloc.build_block_tables(seqs, mb)
    assert np.array_equal(dev_tables.cpu().numpy(), th)
