"""GPU parity of the causal chunked prefill against the float64 oracle.

Small cases build the same cache through the library and through the
oracle (reference allocator, oracle append) and compare every output
element of the chunk rows with the oracle's paged prefill.  They span
several 128-row query tiles and 64-key K/V tiles with ragged tails, chunks
that start from an empty cache (rows with a handful of keys: the hardest
case for 16-bit weights), chunks after a shared and copied-on-write prefix,
grouped-query heads and several block sizes.  The full-size shared-prefix
workload (256 sequences, 512-row chunks), in the launch configuration the
benchmark times over a NaN-poisoned pool, is compared on every row of 34
sequences (the longest and shortest among them) against oracle attention
over each sequence's logical K/V drawn again from the generator.
Tolerance: 2e-3 max-abs (float16/bfloat16 cache, float32 accumulation).
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_420_amd as pkv
import workloads
from cases import (DEV, TOL, GpuState, LogicalKV, OracleState, log, logical_kv,
                   logical_segments, max_abs_err, parallel_map)
from oracle import dense_attention, paged_prefill

pytestmark = pytest.mark.gpu


def ragged_plan(w, prior, chunks, seed=0):
    """Sequences with `prior` cached tokens each, then one chunk of
    `chunks[b]` rows; returns (plan with the prior ops, chunk ops)."""
    rng = np.random.default_rng([w.seed, 77, seed])
    need = sum(-(-(int(a) + int(c)) // w.block_size) for a, c in zip(prior, chunks))
    nb = 2 * need + 4
    seqs = list(range(len(prior)))
    ops = []
    for s, n in zip(seqs, prior):
        ops.append(("add", s))
        if n:
            ops.append(("append", s, int(n)))
    p = workloads.Plan(w, np.asarray(prior), nb, rng.permutation(nb).astype(np.int32), ops, seqs)
    return p, [("append", s, int(c)) for s, c in zip(seqs, chunks)]


def chunk_queries(w, seqs, chunks):
    """Chunk rows of every sequence, stacked: (torch CPU tensor of the cache
    dtype, cu_query_lens)."""
    rows = [workloads.prefill_query(w, s, int(c)) for s, c in zip(seqs, chunks)]
    q = np.concatenate(rows) if rows else np.zeros((0, w.num_heads, w.head_dim), np.float32)
    cu = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    return workloads.to_dtype(q, w.dtype), cu


def run_prefill(g, w, seqs, chunks, max_q=None):
    """GPU prefill of the chunk rows: (float32 output, query tensor, cu)."""
    tables, lens, _, _ = g.tables(seqs)
    q, cu = chunk_queries(w, seqs, chunks)
    mq = int(max(chunks)) if max_q is None else max_q
    out = pkv.paged_attention_prefill(q.to(DEV), g.kc, g.vc, tables, lens,
                                      torch.from_numpy(cu).to(DEV), w.scale, mq)
    torch.cuda.synchronize()
    return out.cpu().numpy(), q, cu


def check_against_oracle(w, prior, chunks, seed=0, prefix_ops=None):
    p, cops = ragged_plan(w, prior, chunks, seed)
    if prefix_ops is not None:
        p.ops = prefix_ops(p)
    g = GpuState(w, p)
    o = OracleState(w, p)
    g.run(cops, first_index=len(p.ops))
    o.run(cops, first_index=len(p.ops))
    got, q, cu = run_prefill(g, w, p.seqs, chunks)
    tables, lens = o.tables()
    want = paged_prefill(workloads.as_f64(q), o.kc, o.vc, tables, lens, cu, w.scale,
                         w.block_size)
    return max_abs_err(got, want)


BF16 = workloads.scaled(workloads.get("shared_prefix_bf16"), num_heads=4, num_kv_heads=4,
                        prefix=0, chunk=0)
FP16 = workloads.scaled(workloads.get("llama13b_fp16"), num_heads=2, num_kv_heads=2)

CASES = {
    # (workload, prior cached tokens, chunk rows)
    "bf16_from_empty": (BF16, [0, 0, 0], [1, 17, 300]),
    "bf16_after_context": (BF16, [5, 200, 1000, 64], [130, 1, 257, 128]),
    "bf16_zero_row_chunk": (BF16, [30, 40], [0, 77]),
    "fp16_bs32": (FP16, [0, 333, 20], [200, 64, 129]),
    "gqa8_bf16": (workloads.scaled(BF16, num_heads=16, num_kv_heads=2), [100, 0], [150, 90]),
    "gqa2_fp16_bs64": (workloads.scaled(FP16, num_heads=4, num_kv_heads=2, block_size=64),
                       [70, 500], [45, 300]),
    "bf16_bs256": (workloads.scaled(BF16, num_heads=2, num_kv_heads=2, block_size=256),
                   [300, 0], [260, 33]),
    "heads8_xcd_order": (workloads.scaled(BF16, num_heads=24, num_kv_heads=8), [50], [140]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_matches_oracle(name):
    w, prior, chunks = CASES[name]
    log("case", name, "prior", prior, "chunks", chunks)
    err = check_against_oracle(w, prior, chunks)
    log(name, "max abs err", err)
    assert err <= TOL[w.dtype]


def test_prefill_after_shared_prefix_with_copy_on_write():
    # a 40-token prefix (not block aligned) forked into three sequences: each
    # sequence's first append copies the shared last block, then its chunk
    w = workloads.scaled(BF16, num_heads=2, num_kv_heads=2)

    def with_prefix(p):
        ops = [("add", workloads.PREFIX_SEQ), ("append", workloads.PREFIX_SEQ, 40)]
        ops += [("fork", workloads.PREFIX_SEQ, s) for s in p.seqs]
        ops += [("free", workloads.PREFIX_SEQ)]
        ops += [op for op in p.ops if op[0] == "append"]
        return ops

    err = check_against_oracle(w, [3, 0, 50], [60, 20, 140], prefix_ops=with_prefix)
    log("shared prefix + cow max abs err", err)
    assert err <= TOL[w.dtype]


def test_chunk_split_only_changes_rounding():
    # one prompt as a single 300-row chunk vs as chunks of 100, 7 and 193 rows
    w = workloads.scaled(BF16, num_heads=2, num_kv_heads=2)
    p, cops = ragged_plan(w, [0], [300])
    g = GpuState(w, p)
    g.run(cops, first_index=len(p.ops))
    whole, _, _ = run_prefill(g, w, [0], [300])
    tables, lens, _, _ = g.tables([0])
    q, _ = chunk_queries(w, [0], [300])
    pieces = []
    for lo, hi in [(0, 100), (100, 107), (107, 300)]:
        lens_k = torch.tensor([hi], dtype=torch.int32, device=DEV)
        cu = torch.tensor([0, hi - lo], dtype=torch.int32, device=DEV)
        pieces.append(pkv.paged_attention_prefill(q[lo:hi].contiguous().to(DEV), g.kc, g.vc,
                                                  tables, lens_k, cu, w.scale, hi - lo))
    split = torch.cat(pieces).cpu().numpy()
    assert np.abs(split - whole).max() <= 2 * TOL[w.dtype]


def test_one_row_chunk_agrees_with_decode():
    w = workloads.scaled(BF16, num_heads=4, num_kv_heads=2)
    p, cops = ragged_plan(w, [400, 31], [1, 1])
    g = GpuState(w, p)
    g.run(cops, first_index=len(p.ops))
    got, q, cu = run_prefill(g, w, p.seqs, [1, 1])
    tables, lens, _, lh = g.tables()
    dec = pkv.paged_attention_decode(q.to(DEV), g.kc, g.vc, tables, lens, w.scale,
                                     int(lh.max())).cpu().numpy()
    assert np.abs(got - dec).max() <= 2 * TOL[w.dtype]


def test_inconsistent_sequences():
    w = workloads.scaled(BF16, num_heads=2, num_kv_heads=2)
    p, cops = ragged_plan(w, [100, 100, 100], [20, 20, 20])
    g = GpuState(w, p)
    g.run(cops, first_index=len(p.ops))
    tables, lens, _, _ = g.tables()
    q, cu = chunk_queries(w, p.seqs, [20, 20, 20])
    lens[0] = 10                            # chunk longer than its context: NaN rows
    tables[1, 2] = p.num_blocks + 5         # table entry outside the pool: NaN rows
    out = torch.full((60, w.num_heads, w.head_dim), 7.0, device=DEV)
    pkv.paged_attention_prefill(q.to(DEV), g.kc, g.vc, tables, lens,
                                torch.from_numpy(cu).to(DEV), w.scale, 20, out=out)
    got = out.cpu().numpy()
    assert np.isnan(got[0:20]).all()
    assert np.isnan(got[20:40]).all()
    assert np.isfinite(got[40:60]).all()
    # decreasing cu entries: that sequence's rows cannot be located, nothing written
    out.fill_(7.0)
    bad_cu = torch.tensor([0, 20, 10, 30], dtype=torch.int32, device=DEV)
    lens2 = torch.tensor([120, 120, 120], dtype=torch.int32, device=DEV)
    pkv.paged_attention_prefill(q[:30].contiguous().to(DEV), g.kc, g.vc, g.tables()[0], lens2,
                                bad_cu, w.scale, 20, out=out[:30])
    got = out.cpu().numpy()
    assert np.isfinite(got[0:20]).all()
    assert (got[20:30] != 7.0).any()        # sequence 2 (rows 10..30) was written
    assert (got[30:] == 7.0).all()          # never touched


def test_prefill_rejects_unsupported():
    w = workloads.scaled(BF16, num_heads=2, num_kv_heads=2, head_dim=64)
    kc = torch.zeros((4, 2, 16, 64), dtype=torch.bfloat16, device=DEV)
    q = torch.zeros((3, 2, 64), dtype=torch.bfloat16, device=DEV)
    t = torch.zeros((1, 4), dtype=torch.int32, device=DEV)
    lens = torch.tensor([3], dtype=torch.int32, device=DEV)
    cu = torch.tensor([0, 3], dtype=torch.int32, device=DEV)
    with pytest.raises(pkv.Unsupported):
        pkv.paged_attention_prefill(q, kc, kc, t, lens, cu, w.scale, 3)
    kc32 = torch.zeros((4, 2, 16, 128), dtype=torch.float32, device=DEV)
    q32 = torch.zeros((3, 2, 128), dtype=torch.float32, device=DEV)
    with pytest.raises(pkv.Unsupported):
        pkv.paged_attention_prefill(q32, kc32, kc32, t, lens, cu, w.scale, 3)


def test_full_size_shared_prefix_prefill():
    """The shared-prefix batch's 512-row chunk per sequence at full size
    (256 sequences, 131,072 rows) over a NaN-poisoned pool: every row and
    head of 34 sequences -- the longest, the shortest and 32 drawn at
    random -- against the oracle's causal attention over the logical K/V
    drawn again from the generator; every output finite."""
    w = workloads.get("shared_prefix_bf16")
    log("full-size shared-prefix prefill", w)
    p = workloads.plan(w)
    cops = workloads.chunk_ops(p)
    g = GpuState(w, p)
    g.run(cops, first_index=len(p.ops))
    seqs = p.seqs
    chunks = [w.chunk] * len(seqs)
    got, q, cu = run_prefill(g, w, seqs, chunks)
    assert np.isfinite(got).all()
    lkv = LogicalKV(w, p.ops + cops)
    rng = np.random.default_rng(11)
    pick = sorted(set(rng.choice(len(seqs), size=32, replace=False).tolist())
                  | {int(np.argmax(p.lens)), int(np.argmin(p.lens))})
    assert len(pick) >= 32

    def err(b):
        k, v = lkv.get(seqs[b])
        n = k.shape[0]
        rows = workloads.as_f64(q[cu[b]:cu[b + 1]])
        want = dense_attention(rows, k, v, w.scale, first_pos=n - w.chunk)
        return max_abs_err(got[cu[b]:cu[b + 1]], want)

    errs = parallel_map(err, pick)
    log("full-size prefill, all", w.chunk, "rows of", len(pick), "sequences: max abs err",
        max(errs))
    assert max(errs) <= TOL[w.dtype]


@pytest.mark.gpu
def test_matrix_loop_runs_and_counts_its_flops():
    """The matrix-core ceiling bench.py reports next to the prefill: the
    launch completes, reports the operations it performs, and leaves the
    sink alone (its products never equal the guard value)."""
    sink = torch.zeros(1, dtype=torch.float32, device=DEV)
    flops = pkv.matrix_loop(100, 8, sink)
    torch.cuda.synchronize()
    assert flops == 8 * 4 * 100 * 4 * 16 * 16 * 32 * 2
    assert sink.item() == 0.0
