"""Continuous-batching step driver: the scheduler's plan run through the
kernels, one attention layer.

Each step ("vLLM 初探" tutorial §1.3; explainer, continuous-batching
section; KV-cache article §4.1/§4.2 for the chunks):
  1. the native scheduler (pkv_scheduler_step) retires, admits and plans
     decode rows and prompt chunks, updating the block allocator;
  1b. blocks it swapped in or out (preemption into a host tier; KV-cache
     article §4.2, swap space) are copied: swap-ins first, then swap-outs,
     both before anything of this step writes the pool;
  2. the plan's slot mapping, block tables, lengths and chunk offsets go to
     the device in one copy from pinned host memory;
  3. pkv_paged_kv_append stores every row's new K/V through the slots;
  4. pkv_paged_attention_decode attends the decode rows,
     pkv_paged_attention_prefill the prompt chunks (causal).
The caller supplies each step's query and new K/V rows (row order of the
plan); this module only moves arguments and launches the library's calls.
"""

import numpy as np
import torch

from . import (Scheduler, paged_attention_decode, paged_attention_decode_workspace_size,
               paged_attention_prefill, paged_kv_append, swap_blocks)


class ServingDriver:
    def __init__(self, scheduler, key_cache, value_cache, num_heads, scale, max_request_tokens,
                 partition_size=0, host_key_cache=None, host_value_cache=None):
        if not isinstance(scheduler, Scheduler):
            raise TypeError("scheduler must be a paged_kv_cache_420_amd.Scheduler")
        self.sched = scheduler
        self.kc, self.vc = key_cache, value_cache
        self.hk, self.hv = host_key_cache, host_value_cache
        if scheduler.host_blocks and (self.hk is None or self.hk.shape[0] < scheduler.host_blocks):
            raise ValueError("a scheduler with a host tier needs pinned host caches that hold it")
        nb, self.num_kv_heads, self.block_size, self.head_dim = key_cache.shape
        self.num_heads = num_heads
        self.scale = scale
        self.dev = key_cache.device
        self.part = partition_size
        self.max_ctx = int(max_request_tokens)
        self.max_blocks = -(-self.max_ctx // self.block_size)
        rows, tokens = scheduler.max_num_seqs, scheduler.max_num_batched_tokens
        ws = paged_attention_decode_workspace_size(rows, num_heads, self.num_kv_heads,
                                                   self.head_dim, self.max_ctx, partition_size)
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=self.dev)
        self.out_dec = torch.empty((rows, num_heads, self.head_dim), dtype=torch.float32,
                                   device=self.dev)
        self.out_pre = torch.empty((tokens, num_heads, self.head_dim), dtype=torch.float32,
                                   device=self.dev)
        # packed metadata: slots | tables | lens | cu (prefill rows)
        self._meta_len = tokens + rows * self.max_blocks + rows + rows + 1
        self._host = [torch.empty(self._meta_len, dtype=torch.int32, pin_memory=True)
                      for _ in range(2)]
        self._copied = [None, None]
        self._dev_meta = torch.empty(self._meta_len, dtype=torch.int32, device=self.dev)
        self._flip = 0

    def step(self, make_rows):
        """Plan and run one step.  ``make_rows(plan)`` returns (q [T, Hq, D],
        k [T, Hkv, D], v [T, Hkv, D]) device tensors in the plan's row order
        (T = plan.num_tokens).  Returns (plan, decode outputs [num_decode, Hq,
        D], prefill outputs [prefill tokens, Hq, D]); the outputs are views of
        buffers reused by the next step."""
        plan = self.sched.step(self.max_blocks)
        if len(plan.swap_in):
            swap_blocks(self.hk, self.hv, self.kc, self.vc, plan.swap_in[:, 0], plan.swap_in[:, 1])
        if len(plan.swap_out):
            swap_blocks(self.kc, self.vc, self.hk, self.hv, plan.swap_out[:, 0],
                        plan.swap_out[:, 1])
        if plan.num_rows == 0:
            return plan, None, None
        nd, nr, nt = plan.num_decode, plan.num_rows, plan.num_tokens
        mb = self.max_blocks
        host = self._host[self._flip]
        if self._copied[self._flip] is not None:
            self._copied[self._flip].synchronize()  # its previous copy has finished
        h = host.numpy()
        o_tab = nt
        o_len = o_tab + nr * mb
        o_cu = o_len + nr
        h[:nt] = plan.slots
        h[o_tab:o_len] = plan.block_tables.reshape(-1)
        h[o_len:o_cu] = plan.context_lens
        npre = nr - nd
        h[o_cu] = 0
        if npre:
            h[o_cu + 1:o_cu + 1 + npre] = np.cumsum(plan.query_lens[nd:])
        n = o_cu + 1 + npre
        dm = self._dev_meta
        dm[:n].copy_(host[:n], non_blocking=True)
        ev = torch.cuda.Event()
        ev.record()
        self._copied[self._flip] = ev
        self._flip ^= 1
        slots = dm[:nt]
        tables = dm[o_tab:o_len].view(nr, mb)
        lens = dm[o_len:o_cu]
        q, k, v = make_rows(plan)
        paged_kv_append(k, v, self.kc, self.vc, slots)
        out_dec = out_pre = None
        if nd:
            mc = int(plan.context_lens[:nd].max())
            out_dec = paged_attention_decode(q[:nd], self.kc, self.vc, tables[:nd], lens[:nd],
                                             self.scale, mc, self.part, self.out_dec[:nd],
                                             self.workspace)
        if npre:
            mq = int(plan.query_lens[nd:].max())
            out_pre = paged_attention_prefill(q[nd:], self.kc, self.vc, tables[nd:], lens[nd:],
                                              dm[o_cu:o_cu + 1 + npre], self.scale, mq,
                                              self.out_pre[:nt - nd])
        return plan, out_dec, out_pre
