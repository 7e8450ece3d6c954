#!/usr/bin/env python3
"""Paged decode benchmark on one MI355X.

A step is one decode step of one attention layer over the whole batch,
through every stage of the path:
  1. host allocator: one new slot per sequence (batch append, all or
     nothing; copy-on-write pairs if a shared block is hit), reporting the
     lengths and the block-table entries the appends set;
  2. those go to the device by value, in the kernel arguments of the
     decode launches (the block table itself stays on the device);
  3. block copies for copy-on-write pairs (none unless blocks are shared);
  4. paged_attention_decode_step: the split-K decode kernel, which applies
     the table changes, stores each sequence's new K/V row at its newest
     position (the slot the allocator returned) and attends, then the
     log-sum-exp merge kernel.  A batch forked from one prefix (the
     shared-prefix workload) steps through
     paged_attention_decode_shared_prefix_step instead: every query against
     the prefix on the matrix cores, the suffixes by the split-K kernel
     (append fused), one merge; a batch of several prefix groups (the
     grouped-prefix workload) through
     paged_attention_decode_grouped_prefix_step, the same three launches
     with every group's prefix in the one matrix-core launch.
The cache is resident in HBM before timing starts.  ``value`` is the KV
bytes the decode reads per step (sum over sequences of context_len * Hkv *
head_dim * 2 * element size) divided by the wall time of a whole step.
With a shared prefix those logical bytes exceed what HBM delivers (the
prefix is the same K/V for every sequence); the roofline then uses the
unique bytes (prefix counted once).
``roofline`` reports the decode partition kernel alone (with a shared
prefix: the three launches of the shared-prefix call) on the cache state
after the timed steps, 20 launches back to back between one pair of HIP
events on the stream it runs on; its ``traffic`` comes from the committed
rocprofv3 counter summary of the same kernel source, when there is one.
``workloads`` carries the same figures for every other workload (20 steps
after 5; their caches filled with values drawn on the device),
``stream_read`` the achievable HBM read rate: a plain read of 4 GiB with
the decode kernel's load width and policy, and ``matrix_loop`` the
matrix-core rate the GPU sustains with the prefill's product instruction in
a register-only loop (each prefill entry then carries its fraction of it).
``cpu_baseline`` times the float64 CPU oracle on a small sample of the same
workload (reported only; the host's CPU model and core count go into its
``sample``).  For the prefix workloads the line also carries
``decode_shared_prefix`` (the shared- or grouped-prefix call against the
split-K call on the same cache state), and for the shared-prefix one
``prefill``: one causal 512-row chunked
prefill per sequence, timed the same way, against the bf16 matrix-core
peak; its oracle timing (one sequence's chunk) is ``cpu_baseline.prefill``.

Usage: python bench.py [--steps K] [--warmup W] [--workload NAME]
       python bench.py --copy-calibration   (block copy of a known size,
                                             the scale for HBM counters)
       python bench.py --block-size-sweep   (paging overhead, block sizes)
       python bench.py --fp8 [--workload NAME]  (8-bit cache vs 16-bit)
       python bench.py --serve              (continuous batching, paged vs
                                             max-length reservation)
"""

import argparse
import json
import hashlib
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16/fp16 matrix peak, published
METRIC = ("paged decode KV-read GB/s (% of HBM peak) + tokens/s, LLaMA-7B layer, batch 64")
DTYPE_NAMES = {"torch.bfloat16": "bf16", "torch.float16": "fp16", "torch.float32": "fp32"}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama7b_bf16")
    ap.add_argument("--partition-size", type=int, default=None,
                    help="split-K partition in tokens (default: the workload's, else automatic)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (profiling runs)")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only --workload (no other workloads, no stream-read ceiling)")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the chunked-prefill leg of the shared-prefix workload")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time pkv_copy_blocks over a known byte count and exit")
    ap.add_argument("--fp8", action="store_true",
                    help="8-bit (E4M3) cache leg: quantising append builds the workload's "
                         "cache, then decode over it is timed next to the 16-bit cache")
    ap.add_argument("--serve", action="store_true",
                    help="continuous-batching leg: a request trace through the native "
                         "scheduler and the kernels, paged admission vs a max-length "
                         "reservation of the same pool")
    ap.add_argument("--block-size-sweep", action="store_true",
                    help="decode GB/s and slot utilisation at block sizes 8..256, shuffled vs "
                         "identity (contiguous) block placement; one JSON line each")
    return ap.parse_args()


def kv_bytes(w, lens):
    return int(np.sum(lens, dtype=np.int64)) * w.num_kv_heads * w.head_dim * 2 * w.elem_bytes


def kv_bytes_unique(w, lens):
    """KV bytes with each shared prefix counted once (what a step must fetch
    from HBM at least); equal to kv_bytes when nothing is shared."""
    import workloads
    layout = workloads.prefix_layout(w)
    if not layout:
        return kv_bytes(w, lens)
    starts, plens = layout
    tokens = int(np.sum(np.asarray(lens, dtype=np.int64) - workloads.seq_prefixes(w)))
    tokens += sum(n for g, n in enumerate(plens) if starts[g + 1] > starts[g])
    return tokens * w.num_kv_heads * w.head_dim * 2 * w.elem_bytes


def prefix_ws_bytes(pkv, w, b, max_len):
    """Workspace of the workload's prefix call (shared or grouped)."""
    import workloads
    if w.prefix:
        return pkv.paged_attention_decode_shared_prefix_workspace_size(
            b, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size, max_len, w.prefix)
    starts, plens = workloads.prefix_layout(w)
    return pkv.paged_attention_decode_grouped_prefix_workspace_size(
        b, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size, max_len, starts, plens)


def prefix_step(pkv, w, q, k, v, kc, vc, tables, lens, changes, mc, out, ws):
    """One step of the workload's prefix call: the shared-prefix step for one
    prefix, the grouped-prefix step for several groups."""
    import workloads
    if w.prefix:
        return pkv.paged_attention_decode_shared_prefix_step(
            q, k, v, kc, vc, tables, lens, changes, w.prefix, w.scale, mc, out=out, workspace=ws)
    starts, plens = workloads.prefix_layout(w)
    return pkv.paged_attention_decode_grouped_prefix_step(
        q, k, v, kc, vc, tables, lens, changes, starts, plens, w.scale, mc, out=out,
        workspace=ws)


def prefix_call(pkv, w, q, kc, vc, tables, lens, mc, out, ws):
    """The plain (device lengths) form of the workload's prefix call."""
    import workloads
    if w.prefix:
        return pkv.paged_attention_decode_shared_prefix(q, kc, vc, tables, lens, w.prefix,
                                                        w.scale, mc, out=out, workspace=ws)
    starts, plens = workloads.prefix_layout(w)
    return pkv.paged_attention_decode_grouped_prefix(q, kc, vc, tables, lens, starts, plens,
                                                     w.scale, mc, out=out, workspace=ws)


def setup(w, pkv, workloads, torch, dev):
    p = workloads.plan(w)
    shape = (p.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
    kc = torch.zeros(shape, dtype=w.dtype, device=dev)
    vc = torch.zeros(shape, dtype=w.dtype, device=dev)
    alloc = pkv.BlockAllocator(p.num_blocks, w.block_size, p.free_order)

    def on_copy(pairs):
        src = torch.tensor([a for a, _ in pairs], dtype=torch.int32, device=dev)
        dst = torch.tensor([b for _, b in pairs], dtype=torch.int32, device=dev)
        pkv.copy_blocks(kc, vc, src, dst)

    def on_append(i, seq, n, slots):
        k, v = workloads.kv_rows(w, i, n)
        pkv.paged_kv_append(workloads.to_dtype(k, w.dtype).to(dev),
                            workloads.to_dtype(v, w.dtype).to(dev), kc, vc,
                            torch.from_numpy(slots).to(dev))

    workloads.run_schedule(p.ops, alloc, on_append, on_copy)
    torch.cuda.synchronize()
    return p, kc, vc, alloc


def fast_setup(w, pkv, workloads, torch, dev):
    """The cache state of a timing-only leg: the workload's schedule through
    the native allocator, with K/V values drawn on the device (torch's
    generator, seeded) instead of the host generator the parity tests use."""
    p = workloads.plan(w)
    shape = (p.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
    kc = torch.zeros(shape, dtype=w.dtype, device=dev)
    vc = torch.zeros(shape, dtype=w.dtype, device=dev)
    alloc = pkv.BlockAllocator(p.num_blocks, w.block_size, p.free_order)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)

    def on_copy(pairs):
        src = torch.tensor([a for a, _ in pairs], dtype=torch.int32, device=dev)
        dst = torch.tensor([b for _, b in pairs], dtype=torch.int32, device=dev)
        pkv.copy_blocks(kc, vc, src, dst)

    def on_append(i, seq, n, slots):
        kv = (torch.randn((2, n, w.num_kv_heads, w.head_dim), generator=gen, device=dev)
              * w.std).to(w.dtype)
        pkv.paged_kv_append(kv[0], kv[1], kc, vc, torch.from_numpy(slots).to(dev))

    workloads.run_schedule(p.ops, alloc, on_append, on_copy)
    torch.cuda.synchronize()
    return p, kc, vc, alloc


def gpu_run(args, w, torch, pkv, workloads, steps=None, warmup=None, fast=False):
    """``steps`` decode steps after ``warmup`` untimed ones (default: the
    command line's), then the roofline kernel alone in a back-to-back loop
    on the final cache state."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    part_arg = w.partition_size if args.partition_size is None else args.partition_size
    p, kc, vc, alloc = (fast_setup if fast else setup)(w, pkv, workloads, torch, dev)
    seqs = np.asarray(p.seqs, dtype=np.int64)
    b = len(seqs)
    total_steps = warmup + steps
    max_len = int(max(alloc.seq_len(s) for s in p.seqs)) + total_steps
    mb = -(-max_len // w.block_size)
    part = pkv.paged_attention_decode_partition_size(b, w.num_kv_heads, w.block_size, max_len,
                                                     part_arg)

    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed + 99)
    k_new = (torch.randn((total_steps, b, w.num_kv_heads, w.head_dim), generator=gen, device=dev)
             * w.std).to(w.dtype)
    v_new = (torch.randn((total_steps, b, w.num_kv_heads, w.head_dim), generator=gen, device=dev)
             * w.std).to(w.dtype)
    q = (torch.randn((total_steps, b, w.num_heads, w.head_dim), generator=gen, device=dev)
         * w.std).to(w.dtype)
    out = torch.empty((b, w.num_heads, w.head_dim), dtype=torch.float32, device=dev)
    ws_bytes = pkv.paged_attention_decode_workspace_size(b, w.num_heads, w.num_kv_heads,
                                                         w.head_dim, max_len, part)
    workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

    # The block table lives on the device across steps.  Each step's
    # lengths and the table entries its appends set travel by value in the
    # kernel arguments (pkv_paged_attention_decode_step): nothing is copied
    # to the device on the step's path.  Host arrays are reused every step:
    # their contents are copied into the launch when it is enqueued.
    stream = torch.cuda.current_stream(dev)
    th, _ = alloc.build_block_tables(seqs, mb)
    tables_d = torch.from_numpy(th.copy()).to(dev)
    slots_h = np.empty(b, dtype=np.int32)
    lens_h = np.empty(b, dtype=np.int32)
    changes_h = np.empty((b + 1, 3), dtype=np.int32)
    append = alloc.prepared_append_changes(seqs, np.ones(b, dtype=np.int32), slots_h, lens_h,
                                           changes_h)
    # blocks held by several sequences (refcount > 1, a forked prefix) are
    # read once per sequence: the decode then loads K/V with the default
    # cache policy instead of streaming them (PKV_DECODE_SHARED_BLOCKS)
    shared = any(r > 1 for r in alloc.snapshot()[1])
    launch = pkv.DecodeLauncher(kc, vc, w.num_heads, b, mb, max_len, part, out, workspace,
                                shared_blocks=shared)
    # a batch forked from one prefix, or made of prefix groups, steps through
    # the shared- or grouped-prefix call instead: the prefixes on the matrix
    # cores, the suffixes split-K (the append fused), one merge
    ws_sp = None
    prefixed = workloads.prefix_layout(w) is not None
    if prefixed:
        ws_sp = torch.empty(max(prefix_ws_bytes(pkv, w, b, max_len), 16), dtype=torch.uint8,
                            device=dev)
    step_bytes = np.zeros(total_steps, dtype=np.float64)
    step_unique = np.zeros(total_steps, dtype=np.float64)

    def step(i):
        pairs, n_changes = append()                                          # 1, 2
        if pairs:                                                            # 3
            src = torch.tensor([a for a, _ in pairs], dtype=torch.int32).to(dev)
            dst = torch.tensor([c for _, c in pairs], dtype=torch.int32).to(dev)
            pkv.copy_blocks(kc, vc, src, dst)
        mc = int(lens_h.max())
        if prefixed:                                                         # 4
            prefix_step(pkv, w, q[i], k_new[i], v_new[i], kc, vc, tables_d, lens_h,
                        changes_h[:n_changes], mc, out, ws_sp)
        else:
            launch.step_partials(q[i], tables_d, lens_h, changes_h, n_changes, mc, w.scale,  # 4
                                 k_new[i], v_new[i])
            launch.step_merge(lens_h, mc)
        step_bytes[i] = kv_bytes(w, lens_h)
        step_unique[i] = kv_bytes_unique(w, lens_h)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(warmup, total_steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if not torch.isfinite(out).all():
        raise RuntimeError("decode produced non-finite output")

    # The roofline kernel alone, on the final cache state: the step's
    # partition kernel (no new rows, no table changes: the fused store of
    # one row per sequence is left out) -- with a shared prefix, the whole
    # shared-prefix call -- launched back to back between one pair of HIP
    # events on its stream, so the events cost nothing per launch.  Then the
    # merge alone the same way.
    mc = int(lens_h.max())
    no_changes = changes_h[:0]
    if prefixed:
        def kernel():
            prefix_step(pkv, w, q[-1], None, None, kc, vc, tables_d, lens_h, no_changes, mc, out,
                        ws_sp)
        merge = None
    else:
        def kernel():
            launch.step_partials(q[-1], tables_d, lens_h, changes_h, 0, mc, w.scale)

        def merge():
            launch.step_merge(lens_h, mc)
    kernel_us = time_loop(torch, stream, kernel, 20) * 1e3
    merge_us = time_loop(torch, stream, merge, 20) * 1e3 if merge else 0.0
    res = dict(wall=wall, kernel_us=kernel_us, merge_us=merge_us,
               kernel_bytes=float(kv_bytes(w, lens_h)),
               kernel_unique_bytes=float(kv_bytes_unique(w, lens_h)),
               bytes=step_bytes[warmup:], unique_bytes=step_unique[warmup:],
               batch=b, part=part, shared=shared, steps=steps)
    if prefixed:
        res["decode_shared_prefix"] = shared_prefix_decode_run(w, p, alloc, kc, vc, torch, pkv,
                                                               dev)
    if w.chunk and not args.no_prefill:
        res["prefill"] = prefill_run(w, p, alloc, kc, vc, torch, pkv, dev)
    return res


def time_loop(torch, stream, fn, reps, warm=3):
    """Mean milliseconds per call of ``fn`` over ``reps`` calls launched back
    to back between one pair of HIP events on ``stream``."""
    for _ in range(warm):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def stream_read_run(torch, pkv):
    """The achievable HBM read rate: 4 GiB read once per launch with the
    decode kernel's load width and policy (pkv_stream_read), mean of 10
    back-to-back launches after 3."""
    dev = torch.device("cuda:0")
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    best = None
    for wg in (2048, 4096, 8192):
        ms = time_loop(torch, stream, lambda: pkv.stream_read(buf, wg, sink), 10)
        gbps = nbytes / (ms * 1e-3) / 1e9
        if best is None or gbps > best["gbps"]:
            best = {"bytes": nbytes, "workgroups": wg, "us": round(ms * 1e3, 2),
                    "gbps": round(gbps, 1), "hbm_peak_frac": round(gbps / HBM_PEAK_GBPS, 4)}
    del buf
    torch.cuda.empty_cache()
    return best


def matrix_loop_run(torch, pkv):
    """The matrix-core rate this GPU sustains: the chunked prefill's bf16
    16 x 16 x 32 product in a register-only loop (pkv_matrix_loop), 2048
    workgroups of four wavefronts (eight per CU) x 20000 iterations, mean of
    5 back-to-back launches after 2 (the clock settles under the load)."""
    dev = torch.device("cuda:0")
    sink = torch.zeros(1, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    wg, iters = 2048, 20000
    flops = wg * 4 * iters * 4 * 16384
    ms = time_loop(torch, stream, lambda: pkv.matrix_loop(iters, wg, sink), 5, warm=2)
    tflops = flops / (ms * 1e-3) / 1e12
    return {"instruction": "v_mfma_f32_16x16x32_bf16", "workgroups": wg, "iters": iters,
            "flops_per_launch": flops, "ms": round(ms, 4), "tflops": round(tflops, 1),
            "bf16_peak_frac": round(tflops / BF16_PEAK_TFLOPS, 4)}


def shared_prefix_decode_run(w, p, alloc, kc, vc, torch, pkv, dev):
    """On the cache state after the decode steps: the plain split-K decode
    (partials + merge, shared-blocks hint) against the shared-prefix decode
    (prefix on the matrix cores, suffixes split-K, merge), HIP events on
    their stream, mean of 10 launches after 2 untimed."""
    seqs = np.asarray(p.seqs, dtype=np.int64)
    b = len(seqs)
    mb = max(len(alloc.block_table(int(s))) for s in seqs)
    th, lh = alloc.build_block_tables(seqs, mb)
    tables = torch.from_numpy(th.copy()).to(dev)
    lens = torch.from_numpy(lh.copy()).to(dev)
    mc = int(lh.max())
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed + 5)
    q = (torch.randn((b, w.num_heads, w.head_dim), generator=gen, device=dev) * w.std).to(w.dtype)
    out_a = torch.empty((b, w.num_heads, w.head_dim), dtype=torch.float32, device=dev)
    out_b = torch.empty_like(out_a)
    ws_a = torch.empty(max(pkv.paged_attention_decode_workspace_size(
        b, w.num_heads, w.num_kv_heads, w.head_dim, mc, 0), 16), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(max(prefix_ws_bytes(pkv, w, b, mc), 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def plain():
        pkv.paged_attention_decode(q, kc, vc, tables, lens, w.scale, mc, out=out_a,
                                   workspace=ws_a, shared_blocks=True)

    def cascade():
        prefix_call(pkv, w, q, kc, vc, tables, lens, mc, out_b, ws_b)

    times = {}
    for name, fn in (("split_k", plain), ("shared_prefix", cascade)):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        times[name] = e0.elapsed_time(e1) / 10
    diff = float((out_a - out_b).abs().max())
    if not (diff <= 2e-3):
        raise RuntimeError(f"shared-prefix decode differs from split-K decode by {diff}")
    unique = kv_bytes_unique(w, lh)
    us = times["shared_prefix"] * 1e3
    import workloads
    starts, plens = workloads.prefix_layout(w)
    return {"call": ("pkv_paged_attention_decode_shared_prefix" if w.prefix else
                     "pkv_paged_attention_decode_grouped_prefix"),
            "group_starts": starts, "prefix_lens": plens,
            "us": round(us, 2), "split_k_us": round(times["split_k"] * 1e3, 2),
            "speedup": round(times["split_k"] / times["shared_prefix"], 3),
            "unique_kv_bytes": int(unique),
            "unique_gbps": round(unique / (us * 1e-6) / 1e9, 1),
            "unique_hbm_peak_frac": round(unique / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "tokens_per_s": round(b / (us * 1e-6), 1),
            "max_abs_diff_vs_split_k": diff}


def prefill_run(w, p, alloc, kc, vc, torch, pkv, dev):
    """One causal chunk of w.chunk rows per sequence after its decode steps:
    append the chunk's K/V, then time the prefill call (HIP events on its
    stream, mean of 10 launches after 2 untimed)."""
    seqs = np.asarray(p.seqs, dtype=np.int64)
    b, c = len(seqs), w.chunk
    slots, pairs = alloc.append_batch(seqs, np.full(b, c, dtype=np.int32))
    if pairs:
        pkv.copy_blocks(kc, vc, torch.tensor([a for a, _ in pairs], dtype=torch.int32).to(dev),
                        torch.tensor([d for _, d in pairs], dtype=torch.int32).to(dev))
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed + 7)
    kv = (torch.randn((2, b * c, w.num_kv_heads, w.head_dim), generator=gen, device=dev)
          * w.std).to(w.dtype)
    pkv.paged_kv_append(kv[0], kv[1], kc, vc, torch.from_numpy(slots).to(dev))
    del kv
    mb = max(len(alloc.block_table(int(s))) for s in seqs)
    th, lh = alloc.build_block_tables(seqs, mb)
    tables = torch.from_numpy(th.copy()).to(dev)
    lens = torch.from_numpy(lh.copy()).to(dev)
    cu = torch.arange(0, (b + 1) * c, c, dtype=torch.int32, device=dev)
    q = (torch.randn((b * c, w.num_heads, w.head_dim), generator=gen, device=dev)
         * w.std).to(w.dtype)
    out = torch.empty((b * c, w.num_heads, w.head_dim), dtype=torch.float32, device=dev)
    # algorithmic flops: row i of a chunk at position n - c + i attends to
    # n - c + i + 1 keys; 2 flops per multiply-add in QK^T and in PV
    ctx = lh.astype(np.int64) - c
    keys = int(np.sum(c * ctx + c * (c + 1) // 2))
    flops = 4.0 * w.head_dim * w.num_heads * keys
    stream = torch.cuda.current_stream(dev)
    for _ in range(2):
        pkv.paged_attention_prefill(q, kc, vc, tables, lens, cu, w.scale, c, out=out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record(stream)
    for _ in range(reps):
        pkv.paged_attention_prefill(q, kc, vc, tables, lens, cu, w.scale, c, out=out)
    e1.record(stream)
    torch.cuda.synchronize()
    if not torch.isfinite(out).all():
        raise RuntimeError("prefill produced non-finite output")
    ms = e0.elapsed_time(e1) / reps
    tflops = flops / (ms * 1e-3) / 1e12
    return {"kernel": "prefill_kernel", "rows": b * c, "chunk": c, "ms": round(ms, 4),
            "rows_per_s": round(b * c / (ms * 1e-3), 1),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                         "flops_per_launch": flops}}


def copy_calibration(torch, pkv):
    """Copy 2 GiB of K/V blocks (1 GiB per cache) with pkv_copy_blocks: a
    plain copy of known size whose HBM counters give the scale between
    rocprofv3's FETCH_SIZE/WRITE_SIZE and bytes moved."""
    dev = torch.device("cuda:0")
    hkv, bs, d = 8, 16, 128
    block_bytes = hkv * bs * d * 2
    pairs = (1 << 30) // block_bytes
    kc = torch.zeros((2 * pairs, hkv, bs, d), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    src = torch.arange(pairs, dtype=torch.int32, device=dev)
    dst = src + pairs
    for _ in range(3):
        pkv.copy_blocks(kc, vc, src[:min(pairs, 65535)], dst[:min(pairs, 65535)])
    torch.cuda.synchronize()
    per_launch = min(pairs, 65535)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        pkv.copy_blocks(kc, vc, src[:per_launch], dst[:per_launch])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    moved = 2 * per_launch * block_bytes
    print(json.dumps({"calibration": "copy_blocks_kernel", "read_bytes_per_launch": moved,
                      "write_bytes_per_launch": moved, "ms": round(ms, 4),
                      "gbps_read_plus_write": round(2 * moved / (ms * 1e-3) / 1e9, 1)}),
          flush=True)


def block_size_sweep(args, torch, pkv, workloads):
    """Paging overhead and the pages' block-size advice (blocks of 16-32
    tokens recommended; large blocks waste memory): the headline batch at
    each block size, with its blocks either scattered by the seeded
    permutation or placed in order (each sequence's blocks contiguous -- the
    layout of a contiguous per-request cache).  Reports decode GB/s (mean
    of 20 timed calls after 5, HIP events around partials + merge) and slot
    utilisation = cached tokens / allocated slots, next to a reservation of
    the longest context for every sequence."""
    import dataclasses
    dev = torch.device("cuda:0")
    base = workloads.get("llama7b_bf16")
    reserve = int(base.lens.split(",")[-1])  # the longest request the length law allows
    for bs in (8, 16, 32, 64, 128, 256):
        w = workloads.scaled(base, block_size=bs)
        for layout in ("shuffled", "identity"):
            p = workloads.plan(w)
            if layout == "identity":
                p = dataclasses.replace(p, free_order=np.arange(p.num_blocks, dtype=np.int32))
            shape = (p.num_blocks, w.num_kv_heads, bs, w.head_dim)
            kc = torch.zeros(shape, dtype=w.dtype, device=dev)
            vc = torch.zeros(shape, dtype=w.dtype, device=dev)
            alloc = pkv.BlockAllocator(p.num_blocks, bs, p.free_order)
            gen = torch.Generator(device=dev)
            gen.manual_seed(w.seed)

            def on_append(i, seq, n, slots):
                kv = (torch.randn((2, n, w.num_kv_heads, w.head_dim), generator=gen, device=dev)
                      ).to(w.dtype)
                pkv.paged_kv_append(kv[0], kv[1], kc, vc, torch.from_numpy(slots).to(dev))

            workloads.run_schedule(p.ops, alloc, on_append)
            seqs = np.asarray(p.seqs, dtype=np.int64)
            mb = max(len(alloc.block_table(int(s))) for s in seqs)
            th, lh = alloc.build_block_tables(seqs, mb)
            tables = torch.from_numpy(th.copy()).to(dev)
            lens = torch.from_numpy(lh.copy()).to(dev)
            mc = int(lh.max())
            q = torch.randn((len(seqs), w.num_heads, w.head_dim), generator=gen,
                            device=dev).to(w.dtype)
            out = torch.empty((len(seqs), w.num_heads, w.head_dim), dtype=torch.float32, device=dev)
            part = pkv.paged_attention_decode_partition_size(len(seqs), w.num_kv_heads, bs, mc, 0)
            need = pkv.paged_attention_decode_workspace_size(len(seqs), w.num_heads,
                                                             w.num_kv_heads, w.head_dim, mc, part)
            ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
            for _ in range(5):
                pkv.paged_attention_decode(q, kc, vc, tables, lens, w.scale, mc, part, out, ws)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(20):
                pkv.paged_attention_decode(q, kc, vc, tables, lens, w.scale, mc, part, out, ws)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 20
            nbytes = kv_bytes(w, lh)
            used = int(lh.sum())
            allocated = int(sum(-(-int(n) // bs) * bs for n in lh))
            print(json.dumps({
                "sweep": "block_size", "workload": w.name, "block_size": bs, "layout": layout,
                "partition_size": part, "decode_us": round(ms * 1e3, 2),
                "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                "hbm_peak_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "slot_utilisation": round(used / allocated, 4),
                "max_length_reservation_utilisation": round(used / (len(lh) * reserve), 4)}),
                flush=True)
            del kc, vc, alloc
            torch.cuda.empty_cache()


def fp8_leg(args, torch, pkv, workloads):
    """Decode over an 8-bit (E4M3) cache of the workload's batch, built by
    the quantising append with the workload's per-tensor scales, next to
    the same batch in its 16-bit dtype.  Each is timed as partials + merge
    on a fixed cache state (HIP events on the stream, mean over the timed
    calls after the warm-up); bytes are the KV bytes each cache holds for
    the batch (1 byte per element for the 8-bit cache).  Then the causal
    chunked prefill over each cache: every sequence's last min(512, length)
    tokens as its chunk."""
    dev = torch.device("cuda:0")
    w = workloads.get(args.workload)
    ks, vs = workloads.FP8_SCALES
    res = {}
    for kind in ("fp8_e4m3", DTYPE_NAMES[str(w.dtype)]):
        p = workloads.plan(w)
        shape = (p.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
        cdt = torch.uint8 if kind == "fp8_e4m3" else w.dtype
        kc = torch.zeros(shape, dtype=cdt, device=dev)
        vc = torch.zeros(shape, dtype=cdt, device=dev)
        alloc = pkv.BlockAllocator(p.num_blocks, w.block_size, p.free_order)

        def on_copy(pairs):
            src = torch.tensor([a for a, _ in pairs], dtype=torch.int32, device=dev)
            dst = torch.tensor([b for _, b in pairs], dtype=torch.int32, device=dev)
            pkv.copy_blocks(kc, vc, src, dst)

        def on_append(i, seq, n, slots):
            k, v = workloads.kv_rows(w, i, n)
            k = workloads.to_dtype(k, w.dtype).to(dev)
            v = workloads.to_dtype(v, w.dtype).to(dev)
            sl = torch.from_numpy(slots).to(dev)
            if kind == "fp8_e4m3":
                pkv.paged_kv_append_fp8(k, v, kc, vc, sl, ks, vs)
            else:
                pkv.paged_kv_append(k, v, kc, vc, sl)

        workloads.run_schedule(p.ops, alloc, on_append, on_copy)
        seqs = np.asarray(p.seqs, dtype=np.int64)
        mb = max(len(alloc.block_table(int(s))) for s in seqs)
        th, lh = alloc.build_block_tables(seqs, mb)
        tables = torch.from_numpy(th.copy()).to(dev)
        lens = torch.from_numpy(lh.copy()).to(dev)
        mc = int(lh.max())
        b = len(seqs)
        q = workloads.to_dtype(np.stack([workloads.decode_query(w, s) for s in p.seqs]),
                               w.dtype).to(dev)
        out = torch.empty((b, w.num_heads, w.head_dim), dtype=torch.float32, device=dev)
        part = pkv.paged_attention_decode_partition_size(b, w.num_kv_heads, w.block_size, mc,
                                                         w.partition_size)
        need = pkv.paged_attention_decode_workspace_size(b, w.num_heads, w.num_kv_heads,
                                                         w.head_dim, mc, part)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

        def partials():
            if kind == "fp8_e4m3":
                pkv.paged_attention_decode_fp8_partials(q, kc, vc, tables, lens, w.scale, ks, vs,
                                                        mc, part, out, ws)
            else:
                pkv.paged_attention_decode_partials(q, kc, vc, tables, lens, w.scale, mc, part,
                                                    out, ws)

        def merge():
            pkv.paged_attention_decode_merge(lens, w.num_kv_heads, w.block_size, mb, mc, part,
                                             out, ws)

        stream = torch.cuda.current_stream(dev)
        n = args.warmup + args.steps
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
        for i in range(n):
            ev[i][0].record(stream)
            partials()
            ev[i][1].record(stream)
            merge()
            ev[i][2].record(stream)
        torch.cuda.synchronize()
        if not torch.isfinite(out).all():
            raise RuntimeError("decode produced non-finite output")
        timed = range(args.warmup, n)
        kern = float(np.mean([ev[i][0].elapsed_time(ev[i][1]) for i in timed]))
        both = float(np.mean([ev[i][0].elapsed_time(ev[i][2]) for i in timed]))
        elem = 1 if kind == "fp8_e4m3" else w.elem_bytes
        nbytes = int(np.sum(lh, dtype=np.int64)) * w.num_kv_heads * w.head_dim * 2 * elem
        res[kind] = {"kv_bytes": nbytes, "partition_size": part,
                     "decode_partition_us": round(kern * 1e3, 2),
                     "decode_us": round(both * 1e3, 2),
                     "kernel_gbps": round(nbytes / (kern * 1e-3) / 1e9, 1),
                     "kernel_hbm_peak_frac": round(nbytes / (kern * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "tokens_per_s": round(b / (both * 1e-3), 1)}

        # causal chunked prefill over the same cache: each sequence's last
        # min(512, length) cached tokens as its chunk (their K/V already in
        # the cache), random queries; mean of 10 launches after 2
        c_b = np.minimum(lh.astype(np.int64), 512)
        cu_h = np.concatenate([[0], np.cumsum(c_b)]).astype(np.int32)
        gen = torch.Generator(device=dev)
        gen.manual_seed(w.seed + 9)
        qp = (torch.randn((int(cu_h[-1]), w.num_heads, w.head_dim), generator=gen, device=dev)
              * w.std).to(w.dtype)
        cu = torch.from_numpy(cu_h).to(dev)
        outp = torch.empty((int(cu_h[-1]), w.num_heads, w.head_dim), dtype=torch.float32,
                           device=dev)
        mq = int(c_b.max())

        def prefill():
            if kind == "fp8_e4m3":
                pkv.paged_attention_prefill_fp8(qp, kc, vc, tables, lens, cu, w.scale, ks, vs, mq,
                                                out=outp)
            else:
                pkv.paged_attention_prefill(qp, kc, vc, tables, lens, cu, w.scale, mq, out=outp)

        pms = time_loop(torch, stream, prefill, 10, warm=2)
        if not torch.isfinite(outp).all():
            raise RuntimeError("prefill produced non-finite output")
        keys = int(np.sum(c_b * (lh.astype(np.int64) - c_b) + c_b * (c_b + 1) // 2))
        pflops = 4.0 * w.head_dim * w.num_heads * keys
        res[kind]["prefill"] = {"rows": int(cu_h[-1]), "ms": round(pms, 4),
                                "tflops": round(pflops / (pms * 1e-3) / 1e12, 1),
                                "bf16_peak_frac": round(pflops / (pms * 1e-3) / 1e12
                                                        / BF16_PEAK_TFLOPS, 4),
                                "flops_per_launch": pflops}
        del kc, vc, alloc, qp, outp
        torch.cuda.empty_cache()
    k8, k16 = res["fp8_e4m3"], res[DTYPE_NAMES[str(w.dtype)]]
    print(json.dumps({"leg": "fp8_kv_cache", "workload": w.name, "k_scale": ks, "v_scale": vs,
                      "steps": args.steps, "warmup": args.warmup, "caches": res,
                      "decode_speedup_vs_16bit": round(k16["decode_us"] / k8["decode_us"], 3),
                      "prefill_speedup_vs_16bit": round(k16["prefill"]["ms"] / k8["prefill"]["ms"],
                                                        3)}),
          flush=True)


def serve_leg(args, torch, pkv, workloads):
    """The serving trace (all requests queued at the start) run to the end
    through the step driver on the same pool: paged admission, and the
    reservation model (every running request holds room for the longest
    request the length laws allow, as a contiguous per-request cache must);
    paged admission once more with the decode rows' full tables uploaded
    every step (the driver's decode="upload") instead of kept in
    device-resident lanes and changed by value (decode="step").  Reports steps, wall time, generated and prompt tokens per
    second, the mean running set, and the mean over steps of slot
    utilisation (cached tokens / slots held by the running requests) next
    to reservation utilisation (cached tokens / slots reserved)."""
    from paged_kv_cache_420_amd.serving import ServingDriver
    dev = torch.device("cuda:0")
    t = workloads.SERVING["serve_llama7b"]
    reqs = workloads.serving_requests(t)
    reserve = int(t.prompt.split(",")[-1]) + int(t.output.split(",")[-1])
    shape = (t.num_blocks, t.num_kv_heads, t.block_size, t.head_dim)
    kc = torch.zeros(shape, dtype=t.dtype, device=dev)
    vc = torch.zeros(shape, dtype=t.dtype, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(t.seed)
    n = t.max_num_batched_tokens
    q_rows = (torch.randn((n, t.num_heads, t.head_dim), generator=gen, device=dev)).to(t.dtype)
    k_rows = (torch.randn((n, t.num_kv_heads, t.head_dim), generator=gen, device=dev)).to(t.dtype)
    v_rows = (torch.randn((n, t.num_kv_heads, t.head_dim), generator=gen, device=dev)).to(t.dtype)

    def rows(plan):
        m = plan.num_tokens
        return q_rows[:m], k_rows[:m], v_rows[:m]

    order = np.random.default_rng(t.seed).permutation(t.num_blocks).astype(np.int32)
    res = {}
    for policy, rt, mode in (("paged", 0, "step"), ("reservation", reserve, "step"),
                             ("paged_upload", 0, "upload")):
        sched = pkv.Scheduler(t.num_blocks, t.block_size, t.max_num_seqs,
                              t.max_num_batched_tokens, t.chunk_size, rt, order)
        for rid, p, o in reqs:
            sched.add_request(rid, p, o)
        drv = ServingDriver(sched, kc, vc, t.num_heads, t.scale, reserve, decode=mode)
        util, rutil, running, dec_rows, pre_tok = [], [], [], 0, 0
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while True:
            plan, _, _ = drv.step(rows)
            st = sched.stats()
            if plan.num_rows == 0 and st["running"] == 0 and st["waiting"] == 0:
                break
            dec_rows += plan.num_decode
            pre_tok += plan.num_tokens - plan.num_decode
            running.append(st["running"])
            if st["allocated_slots"]:
                util.append(st["cached_tokens"] / st["allocated_slots"])
                rutil.append(st["cached_tokens"] / st["reserved_slots"])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        st = sched.stats()
        if st["finished"] != len(reqs):
            raise RuntimeError(f"{policy}: {st['finished']} of {len(reqs)} requests finished")
        res[policy] = {"decode": mode, "steps": st["steps"], "wall_s": round(wall, 3),
                       "ms_per_step": round(wall / st["steps"] * 1e3, 4),
                       "generated_tokens_per_s": round(dec_rows / wall, 1),
                       "prompt_tokens_per_s": round(pre_tok / wall, 1),
                       "mean_running": round(float(np.mean(running)), 1),
                       "max_running": int(np.max(running)),
                       "preemptions": st["preemptions"],
                       "slot_utilisation": round(float(np.mean(util)), 4),
                       "reserved_slot_utilisation": round(float(np.mean(rutil)), 4)}
        sched.close()
    print(json.dumps({
        "leg": "continuous_batching", "trace": t.name, "requests": len(reqs),
        "prompt_lens": t.prompt, "output_lens": t.output, "reserve_tokens": reserve,
        "layer": {"num_heads": t.num_heads, "num_kv_heads": t.num_kv_heads,
                  "head_dim": t.head_dim, "block_size": t.block_size, "dtype": "bf16",
                  "num_blocks": t.num_blocks},
        "max_num_seqs": t.max_num_seqs, "max_num_batched_tokens": t.max_num_batched_tokens,
        "chunk_size": t.chunk_size, "policies": res,
        "generated_tokens_per_s_ratio": round(res["paged"]["generated_tokens_per_s"] /
                                              res["reservation"]["generated_tokens_per_s"], 3),
        "step_decode_vs_upload_ms_per_step": [res["paged"]["ms_per_step"],
                                              res["paged_upload"]["ms_per_step"]]}),
        flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, workloads):
    """The float64 oracle on a sample of the workload's sequences; for a
    workload with a prefill chunk, also the oracle's causal prefill of one
    sequence's chunk."""
    import threadpoolctl
    from oracle import RefAllocator, copy_blocks, kv_append, paged_decode, paged_prefill

    sample = min(6, w.num_seqs)
    p = workloads.plan(w)
    keep = set(p.seqs[:sample])

    def wanted(op):
        if op[0] == "fork":
            return op[2] in keep
        return op[1] in keep or op[1] >= workloads.PREFIX_SEQ   # a prefix parent

    prefixes = sum(-(-n // w.block_size) for n in (workloads.prefix_layout(w) or [[], []])[1])
    need = sum(-(-int(n) // w.block_size) for n in p.lens[:sample]) + prefixes + \
        -(-w.chunk // w.block_size) + 5
    ref = RefAllocator(need, w.block_size)
    shape = (need, w.num_kv_heads, w.block_size, w.head_dim)
    kc, vc = np.full(shape, np.nan), np.full(shape, np.nan)
    for i, op in enumerate(p.ops):
        if not wanted(op):
            continue
        if op[0] == "append":
            k, v = workloads.kv_rows(w, i, op[2])
            slots, pairs = ref.append(op[1], op[2])
            if pairs:
                copy_blocks(kc, vc, [a for a, _ in pairs], [c for _, c in pairs])
            kv_append(kc, vc, workloads.as_f64(workloads.to_dtype(k, w.dtype)),
                      workloads.as_f64(workloads.to_dtype(v, w.dtype)), slots, w.block_size)
        else:
            workloads.run_schedule([op], ref)
    seqs = sorted(keep)
    tables, lens = ref.build_tables(seqs, max(len(ref.tables[s]) for s in seqs))
    q = np.stack([workloads.as_f64(workloads.to_dtype(workloads.decode_query(w, s), w.dtype))
                  for s in seqs])
    info = threadpoolctl.threadpool_info()
    threads = max([d.get("num_threads", 1) for d in info] or [1])
    reps, t0 = 0, time.perf_counter()
    while True:
        paged_decode(q, kc, vc, np.array(tables), lens, w.scale, w.block_size)
        reps += 1
        el = time.perf_counter() - t0
        if el > 10.0 and reps >= 3:
            break
    per = el / reps
    gbps = kv_bytes(w, np.array(lens)) / per / 1e9
    host = f"host: {cpu_model()}, {len(os.sched_getaffinity(0))} cores available"
    res = {"value": round(gbps, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
           "tokens_per_s": round(len(seqs) / per, 2),
           "sample": f"{len(seqs)} of {w.num_seqs} sequences (context lens "
                     f"{[int(x) for x in lens]}), one decode step each, float64 numpy "
                     f"gather-then-attend, {reps} repetitions in {el:.1f} s; {host}"}
    if w.chunk:
        # one sequence's chunk: seeded rows appended after its context
        s0, c = seqs[0], w.chunk
        slots, pairs = ref.append(s0, c)
        if pairs:
            copy_blocks(kc, vc, [a for a, _ in pairs], [d for _, d in pairs])
        kv = workloads.normal([w.seed, 9, 0], (2, c, w.num_kv_heads, w.head_dim), w.std)
        kv_append(kc, vc, workloads.as_f64(workloads.to_dtype(kv[0], w.dtype)),
                  workloads.as_f64(workloads.to_dtype(kv[1], w.dtype)), slots, w.block_size)
        qr = workloads.as_f64(workloads.to_dtype(
            workloads.normal([w.seed, 9, 1], (c, w.num_heads, w.head_dim), w.std), w.dtype))
        t1, l1 = ref.build_tables([s0], len(ref.tables[s0]))
        n = int(l1[0])
        flops = 4.0 * w.head_dim * w.num_heads * (c * (n - c) + c * (c + 1) // 2)
        reps, t0 = 0, time.perf_counter()
        while True:
            paged_prefill(qr, kc, vc, np.array(t1), l1, [0, c], w.scale, w.block_size)
            reps += 1
            el = time.perf_counter() - t0
            if el > 5.0 and reps >= 2:
                break
        per = el / reps
        res["prefill"] = {"value": round(flops / per / 1e9, 3), "unit": "GFLOP/s",
                          "rows_per_s": round(c / per, 1),
                          "sample": f"one sequence's {c}-row causal chunk at context {n}, "
                                    f"float64 numpy, {reps} repetitions in {el:.1f} s"}
    return res


def traffic_profile(w):
    """The committed counter summary of the workload's roofline kernel:
    profiles/decode_partition_<workload>_traffic.md, else the workload's
    profiles/decode_partition_<workload>.md."""
    for suffix in ("_traffic", ""):
        path = os.path.join(ROOT, "profiles", f"decode_partition_{w.name}{suffix}.md")
        if os.path.exists(path):
            return path
    return None


def traffic_from_profiles(w):
    """HBM bytes per launch (per call, for the prefix workloads) of the
    roofline kernel from its committed counter summary, when it was taken on
    the current kernel sources (decode.hip, and prefill.hip where listed);
    else None."""
    path = traffic_profile(w)
    if path is None:
        return None
    fields = dict(re.findall(r"^- (\w+): (\S+)$", open(path).read(), flags=re.M))
    csrc = os.path.join(ROOT, "paged_kv_cache_420_amd", "csrc")
    for key, src in (("kernel_source_sha256", "decode.hip"),
                     ("prefill_source_sha256", "prefill.hip")):
        if key == "kernel_source_sha256" or key in fields:
            digest = hashlib.sha256(open(os.path.join(csrc, src), "rb").read()).hexdigest()
            if fields.get(key) != digest:
                return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the path has no "
              "multi-GPU mode", file=sys.stderr)
        sys.exit(2)
    import torch
    import paged_kv_cache_420_amd as pkv
    import workloads

    if args.copy_calibration:
        copy_calibration(torch, pkv)
        return
    if args.block_size_sweep:
        block_size_sweep(args, torch, pkv, workloads)
        return
    if args.fp8:
        fp8_leg(args, torch, pkv, workloads)
        return
    if args.serve:
        serve_leg(args, torch, pkv, workloads)
        return
    w = workloads.get(args.workload)
    r = gpu_run(args, w, torch, pkv, workloads)
    leg = summarise(w, r)
    line = {
        "metric": METRIC,
        "value": leg["gbps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": leg["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAMES[str(w.dtype)],
        "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "num_heads": w.num_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size, "context_lens": w.lens,
                   "shared_prefix": w.prefix, "prefix_groups": list(w.prefix_groups),
                   "partition_size": r["part"],
                   "kv_loads": leg["kv_loads"]},
        "hbm_peak_frac": leg["hbm_peak_frac"],
        "tokens_per_s": leg["tokens_per_s"],
        "kv_bytes_per_step": leg["kv_bytes_per_step"],
        "kv_bytes_per_step_unique": leg["kv_bytes_per_step_unique"],
        "decode_partition_us": leg["kernel_us"],
        "decode_merge_us": leg["merge_us"],
        "roofline": {"bound": "hbm", "kernel": leg["kernel"],
                     "achieved": leg["kernel_gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": leg["kernel_hbm_peak_frac"],
                     "traffic": leg["traffic"],
                     "traffic_from": leg["traffic_from"],
                     "bytes_per_launch": leg["kernel_bytes"],
                     "timing": "20 launches back to back between one pair of HIP events on "
                               "the kernel's stream, on the cache state after the timed steps"},
    }
    if "decode_shared_prefix" in r:
        line["decode_shared_prefix"] = r["decode_shared_prefix"]
    if "prefill" in r:
        line["prefill"] = r["prefill"]
    if not args.headline_only:
        # the other workloads, each through the same step (cache values drawn
        # on the device), and the achievable read rate
        extra = {}
        for name in workloads.WORKLOADS:
            if name == w.name:
                continue
            wx = workloads.get(name)
            rx = gpu_run(args, wx, torch, pkv, workloads, steps=20, warmup=5, fast=True)
            extra[name] = summarise(wx, rx)
            for key in ("decode_shared_prefix", "prefill"):
                if key in rx:
                    extra[name][key] = rx[key]
            torch.cuda.empty_cache()
        line["workloads"] = extra
        sr = stream_read_run(torch, pkv)
        sr["decode_kernel_frac_of_stream_read"] = round(leg["kernel_gbps"] / sr["gbps"], 4)
        line["stream_read"] = sr
        ml = matrix_loop_run(torch, pkv)
        line["matrix_loop"] = ml
        for pre in [line.get("prefill")] + [x.get("prefill") for x in extra.values()]:
            if pre:
                pre["frac_of_matrix_loop"] = round(pre["roofline"]["achieved"] / ml["tflops"], 4)
    line["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(w, workloads)
    print(json.dumps(line), flush=True)


def summarise(w, r):
    """Step rate and roofline figures of one gpu_run."""
    ms_step = r["wall"] / r["steps"] * 1e3
    mean_bytes = float(r["bytes"].mean())
    unique = float(r["unique_bytes"].mean())
    # roofline on the bytes HBM must deliver: a shared prefix counts once
    kgbps = r["kernel_unique_bytes"] / (r["kernel_us"] * 1e-6) / 1e9
    return {
        "workload": w.name, "num_seqs": w.num_seqs, "partition_size": r["part"],
        "ms_per_step": round(ms_step, 5),
        "gbps": round(mean_bytes / (ms_step * 1e-3) / 1e9, 2),
        "hbm_peak_frac": round(mean_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "unique_gbps": round(unique / (ms_step * 1e-3) / 1e9, 2),
        "unique_hbm_peak_frac": round(unique / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "tokens_per_s": round(r["batch"] / (ms_step * 1e-3), 1),
        "kv_bytes_per_step": int(mean_bytes), "kv_bytes_per_step_unique": int(unique),
        "kernel": ("shared-prefix decode call: prefix on the matrix cores + "
                   "decode_partition_kernel over the suffixes + merge"
                   if w.prefix else
                   "grouped-prefix decode call: every group's prefix on the matrix cores + "
                   "decode_partition_kernel over the suffixes + merge"
                   if w.prefix_groups else "decode_partition_kernel (step form)"),
        "kernel_us": round(r["kernel_us"], 2), "merge_us": round(r["merge_us"], 2),
        "kernel_bytes": int(r["kernel_unique_bytes"]),
        "kernel_gbps": round(kgbps, 2),
        "kernel_hbm_peak_frac": round(kgbps / HBM_PEAK_GBPS, 4),
        "kv_loads": ("prefix: matrix-core contraction; suffixes: non-temporal"
                     if w.prefix or w.prefix_groups else
                     "cached (shared blocks)" if r["shared"] else "non-temporal"),
        "traffic": traffic_from_profiles(w),
        "traffic_from": (f"{os.path.relpath(traffic_profile(w), ROOT)}: rocprofv3 --pmc "
                         "FETCH_SIZE and WRITE_SIZE of the same kernel sources, scaled by the "
                         "block-copy calibration (null when a source has changed since)"
                         if traffic_profile(w) else None),
    }


if __name__ == "__main__":
    main()
