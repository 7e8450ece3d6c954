"""GPU parity of the continuous-batching step driver.

A small trace runs to the end through the native scheduler and the
kernels (append, decode, chunked prefill).  Every token's K/V and every
query row are drawn from per-(request, position) streams, so the oracle
rebuilds each request's logical K/V and checks every output row of every
step: decode rows against attention over the whole context, prompt rows
causally.  The pool is small enough that a request is preempted --
recomputed, or swapped to a pinned host pool and back -- which the test
checks happened.  Tolerance 2e-3 (bf16 cache,
float32 accumulation).
"""

import dataclasses

import numpy as np
import pytest
import torch

import paged_kv_cache_420_amd as pkv
import workloads
from cases import DEV, log, max_abs_err
from oracle import dense_attention
from paged_kv_cache_420_amd.serving import ServingDriver

pytestmark = pytest.mark.gpu

TOL = 2e-3

SMALL = dataclasses.replace(
    workloads.SERVING["serve_llama7b"], name="serve_small", num_requests=10,
    prompt="uniform:5,100", output="uniform:1,40", num_heads=4, num_kv_heads=2,
    num_blocks=20, max_num_seqs=4, max_num_batched_tokens=64, chunk_size=32)


class Tokens:
    """Cached per-(request, position) values, float64 after the dtype cast."""

    def __init__(self, t):
        self.t = t
        self.kv = {}
        self.q = {}

    def _cast(self, x):
        return workloads.as_f64(workloads.to_dtype(x, self.t.dtype))

    def kv_row(self, rid, pos):
        if (rid, pos) not in self.kv:
            k, v = workloads.serving_token_kv(self.t, rid, pos)
            self.kv[(rid, pos)] = (k, v, self._cast(k), self._cast(v))
        return self.kv[(rid, pos)]

    def q_row(self, rid, pos):
        if (rid, pos) not in self.q:
            q = workloads.serving_query(self.t, rid, pos)
            self.q[(rid, pos)] = (q, self._cast(q))
        return self.q[(rid, pos)]

    def positions(self, plan):
        for i in range(plan.num_rows):
            rid, ql, ctx = int(plan.seq_ids[i]), int(plan.query_lens[i]), int(plan.context_lens[i])
            for pos in range(ctx - ql, ctx):
                yield i, rid, pos

    def make_rows(self, plan):
        qs, ks, vs = [], [], []
        for _, rid, pos in self.positions(plan):
            k, v, _, _ = self.kv_row(rid, pos)
            qs.append(self.q_row(rid, pos)[0])
            ks.append(k)
            vs.append(v)
        dt = self.t.dtype
        return (workloads.to_dtype(np.stack(qs), dt).to(DEV),
                workloads.to_dtype(np.stack(ks), dt).to(DEV),
                workloads.to_dtype(np.stack(vs), dt).to(DEV))

    def logical(self, rid, n):
        rows = [self.kv_row(rid, p) for p in range(n)]
        return np.stack([r[2] for r in rows]), np.stack([r[3] for r in rows])


@pytest.mark.parametrize("decode", ["step", "upload"])
@pytest.mark.parametrize("host_blocks", [0, 24])
def test_serving_trace_matches_oracle_every_step(host_blocks, decode):
    """host_blocks 0: preemption recomputes; 24: it swaps to a pinned host
    pool and back, and the outputs must not notice.  decode "step": the
    decode rows' tables live in device lanes changed by value each step;
    "upload": they travel whole every step."""
    t = SMALL
    reqs = workloads.serving_requests(t)
    max_tokens = max(p + o for _, p, o in reqs)
    rng = np.random.default_rng(t.seed)
    order = rng.permutation(t.num_blocks).astype(np.int32)
    sched = pkv.Scheduler(t.num_blocks, t.block_size, t.max_num_seqs, t.max_num_batched_tokens,
                          t.chunk_size, 0, order, host_blocks=host_blocks)
    for rid, p, o in reqs:
        sched.add_request(rid, p, o)
    shape = (t.num_blocks, t.num_kv_heads, t.block_size, t.head_dim)
    kc = torch.full(shape, float("nan"), dtype=t.dtype, device=DEV)
    vc = torch.full(shape, float("nan"), dtype=t.dtype, device=DEV)
    hk = hv = None
    if host_blocks:
        hshape = (host_blocks,) + shape[1:]
        hk = torch.full(hshape, float("nan"), dtype=t.dtype).pin_memory()
        hv = torch.full(hshape, float("nan"), dtype=t.dtype).pin_memory()
    drv = ServingDriver(sched, kc, vc, t.num_heads, t.scale, max_tokens,
                        host_key_cache=hk, host_value_cache=hv, decode=decode)
    tok = Tokens(t)
    worst, steps, rows_checked = 0.0, 0, 0
    while True:
        plan, out_dec, out_pre = drv.step(tok.make_rows)
        steps += 1
        st = sched.stats()
        if plan.num_rows == 0 and st["running"] == 0 and st["waiting"] == 0:
            break
        assert steps < 2000
        if plan.num_rows == 0:
            continue
        torch.cuda.synchronize()
        dec = out_dec.cpu().numpy() if out_dec is not None else None
        pre = out_pre.cpu().numpy() if out_pre is not None else None
        k_pre = 0
        for i in range(plan.num_rows):
            rid, ql, ctx = int(plan.seq_ids[i]), int(plan.query_lens[i]), int(plan.context_lens[i])
            k, v = tok.logical(rid, ctx)
            q = np.stack([tok.q_row(rid, p)[1] for p in range(ctx - ql, ctx)])
            if i < plan.num_decode:
                want = dense_attention(q, k, v, t.scale)
                got = dec[i][None]
            else:
                want = dense_attention(q, k, v, t.scale, first_pos=ctx - ql)
                got = pre[k_pre:k_pre + ql]
                k_pre += ql
            worst = max(worst, max_abs_err(got, want))
            rows_checked += 1
    st = sched.stats()
    log("steps", steps, "rows checked", rows_checked, "max abs err", worst, "stats", st)
    assert st["finished"] == len(reqs)
    assert st["preemptions"] > 0          # the preemption path ran
    if host_blocks:
        assert st["swapped_out"] == st["preemptions"] and st["swapped_in"] > 0
    assert worst <= TOL
