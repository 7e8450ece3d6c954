"""pkv_paged_attention_decode_noalloc: the decode entry point that allocates
nothing (split-K partials in the library's fixed per-GPU array), called
through the C ABI and checked against pkv_paged_attention_decode with a
caller workspace -- the same kernels, so the same bits -- and against the
oracle, on two calls in a row, the second with a smaller batch, shorter
contexts and more partitions per sequence; sizes beyond the array are
refused before anything is enqueued."""

import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_420_amd as pkv
import workloads
from cases import DEV, TOL, GpuState, OracleState, decode_queries, log, max_abs_err
from oracle import paged_decode

pytestmark = pytest.mark.gpu


def _noalloc(q, kc, vc, tables, lens, scale, max_ctx, part, out):
    b, hq, d = q.shape
    nb, hkv, bs, _ = kc.shape
    st = pkv._lib.pkv_paged_attention_decode_noalloc(
        q.data_ptr(), kc.data_ptr(), vc.data_ptr(), tables.data_ptr(), lens.data_ptr(), b, hq,
        hkv, d, bs, tables.shape[1], nb, int(max_ctx), ctypes.c_float(scale), int(part),
        out.data_ptr(), pkv._dtype_code(kc), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def test_noalloc_decode_is_the_workspace_decode():
    w = workloads.scaled(workloads.get("llama7b_bf16"), num_seqs=24, num_heads=8, num_kv_heads=4,
                         lens="uniform:1,1500", seed=4700)
    p = workloads.plan(w)
    g = GpuState(w, p)
    o = OracleState(w, p)
    tables, lens, _, lh = g.tables()
    q, q64 = decode_queries(w, p.seqs)
    q = q.to(DEV)
    ot, ol = o.tables()
    want64 = paged_decode(q64, o.kc, o.vc, ot, ol, w.scale, w.block_size)
    # call 1: the whole batch in 256-token partitions; call 2: the first 9
    # sequences cut to at most 700 tokens, in 64-token partitions
    short = torch.clamp(lens[:9], max=700).contiguous()
    cases = [(q, tables, lens, int(lh.max()), 256),
             (q[:9].contiguous(), tables[:9].contiguous(), short, 700, 64)]
    for k, (qq, tt, ll, mc, part) in enumerate(cases):
        out = torch.full((qq.shape[0], w.num_heads, w.head_dim), float("nan"), device=DEV)
        assert _noalloc(qq, g.kc, g.vc, tt, ll, w.scale, mc, part, out) == 0, pkv._lib.pkv_last_error()
        want = pkv.paged_attention_decode(qq, g.kc, g.vc, tt, ll, w.scale, mc, partition_size=part)
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"call {k}"
        if k == 0:
            err = max_abs_err(out.cpu().numpy(), want64)
            log("noalloc decode max abs err vs oracle", err)
            assert err <= TOL[w.dtype]
    # partials beyond the fixed 64 MiB array: refused, nothing launched
    big = pkv.paged_attention_decode_workspace_size(4096, 64, 8, 128, 8192, 512)
    assert big > 64 << 20
    qb = torch.zeros((4096, 64, 128), dtype=w.dtype, device=DEV)
    tb = torch.zeros((4096, 512), dtype=torch.int32, device=DEV)
    lb = torch.zeros(4096, dtype=torch.int32, device=DEV)
    kb = torch.zeros((4, 8, 16, 128), dtype=w.dtype, device=DEV)
    ob = torch.empty((4096, 64, 128), device=DEV)
    assert _noalloc(qb, kb, kb, tb, lb, w.scale, 8192, 512, ob) == 5   # PKV_ERR_BUFFER_TOO_SMALL
    assert b"64" in pkv._lib.pkv_last_error() or b"scratch" in pkv._lib.pkv_last_error()
