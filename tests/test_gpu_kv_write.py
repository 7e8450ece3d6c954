"""GPU parity of the cache writes: slot-mapped append and block copy must be
bit-exact against the oracle's pool, slots and allocator state."""

import numpy as np
import pytest
import torch

import paged_kv_cache_420_amd as pkv
import workloads
from cases import DEV, GpuState, OracleState, log

pytestmark = pytest.mark.gpu


def _pool_f64(t):
    return t.to(torch.float64).cpu().numpy()


SMALL = {
    "tiny_fp32": workloads.get("tiny_fp32"),
    "llama7b_small": workloads.scaled(workloads.get("llama7b_bf16"), num_seqs=5, num_heads=4,
                                      num_kv_heads=4, lens="uniform:1,300"),
    "llama13b_small": workloads.scaled(workloads.get("llama13b_fp16"), num_seqs=6, num_heads=3,
                                       num_kv_heads=3, lens="geometric:60,1,400"),
    "gqa_small": workloads.scaled(workloads.get("gqa_bf16"), num_seqs=4, num_heads=16,
                                  num_kv_heads=2, lens="uniform:1,700"),
    # prefix of 40 tokens: not block aligned, so every fork's first append copies
    "shared_prefix_cow": workloads.scaled(workloads.get("shared_prefix_bf16"), num_seqs=6,
                                          num_heads=2, num_kv_heads=2, prefix=40,
                                          lens="uniform:1,90", chunk=24),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_built_pool_is_bit_exact(name):
    w = SMALL[name]
    log("case", name)
    p = workloads.plan(w)
    g = GpuState(w, p)
    o = OracleState(w, p)
    assert g.slot_log == o.slot_log
    free_g, ref_g = g.alloc.snapshot()
    assert free_g == o.alloc.free_stack() and ref_g == o.alloc.ref
    torch.cuda.synchronize()
    assert np.array_equal(_pool_f64(g.kc), o.kc, equal_nan=True)
    assert np.array_equal(_pool_f64(g.vc), o.vc, equal_nan=True)
    if w.chunk:
        ops = workloads.chunk_ops(p)
        g.run(ops, first_index=len(p.ops))
        o.run(ops, first_index=len(p.ops))
        torch.cuda.synchronize()
        assert g.slot_log == o.slot_log
        assert np.array_equal(_pool_f64(g.kc), o.kc, equal_nan=True)
        assert np.array_equal(_pool_f64(g.vc), o.vc, equal_nan=True)


def test_append_skips_negative_and_out_of_pool_slots():
    nb, h, bs, d = 4, 2, 8, 64
    kc = torch.zeros((nb, h, bs, d), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    key = torch.randn((4, h, d), device=DEV).to(torch.bfloat16)
    val = torch.randn((4, h, d), device=DEV).to(torch.bfloat16)
    slots = torch.tensor([3, -1, nb * bs, 31], dtype=torch.int32, device=DEV)
    pkv.paged_kv_append(key, val, kc, vc, slots)
    torch.cuda.synchronize()
    want_k = torch.zeros_like(kc)
    want_k[0, :, 3] = key[0]
    want_k[3, :, 7] = key[3]
    assert torch.equal(kc, want_k)
    assert torch.equal(vc[3, :, 7], val[3]) and torch.equal(vc[0, :, 3], val[0])
    assert torch.count_nonzero(vc).item() == torch.count_nonzero(val[[0, 3]]).item()


def test_copy_blocks_is_exact_and_skips_bad_pairs():
    nb, h, bs, d = 6, 3, 16, 128
    kc = torch.randn((nb, h, bs, d), device=DEV)
    vc = torch.randn((nb, h, bs, d), device=DEV)
    k0, v0 = kc.clone(), vc.clone()
    src = torch.tensor([1, 4, 9], dtype=torch.int32, device=DEV)
    dst = torch.tensor([0, 5, 2], dtype=torch.int32, device=DEV)
    pkv.copy_blocks(kc, vc, src, dst)
    torch.cuda.synchronize()
    ko, vo = k0.cpu().numpy(), v0.cpu().numpy()
    from oracle import copy_blocks
    copy_blocks(ko, vo, [1, 4], [0, 5])
    assert np.array_equal(kc.cpu().numpy(), ko) and np.array_equal(vc.cpu().numpy(), vo)
