"""CPU oracle for paged KV-cache attention -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously correct restatement of what the paged
attention path computes, in float64 numpy and pure Python. It exists to check
the HIP library, never to stand in for it: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. It imports nothing from ``paged_kv_cache_420_amd`` and shares no
code, table or helper with it.

Sources, cited by page title and section (the three pages are the only
specification):

* "vLLM 初探" tutorial, §1.4 "PagedAttention 原理简介": the KV cache is cut into
  fixed-size blocks, each sequence owns a logical page table mapping logical
  block i to a physical block in one shared pool (the figure maps logical
  blocks 0, 1, 2 to physical 3, 7, 1); identical prefixes may share physical
  blocks.
* vLLM explainer (openEuler/CSDN summary), sections "LLM serving的基本流程与KV
  缓存", "vLLM的核心创新：PagedAttention", "PagedAttention带来的额外红利：内存
  共享": prefill stores every prompt token's K/V, each decode step appends one
  token's K/V and attends over all earlier ones; blocks are taken on demand and
  returned to the pool when a request ends; block tables of sharing requests
  point at the same blocks; paging leaves the model's output unchanged.
* KV-cache article (intelliparadigm), §2.1 "核心设计原理" and its pseudo-code:
  a token at position p lives in logical block p // block_size, whose physical
  page is block_tables[seq][p // block_size]; the kernel gathers the pages and
  computes softmax(q K^T) V. §4.1/§4.2 name chunked prefill.

Modules:
  attention  -- gather, decode, chunked prefill (float64)
  kvstore    -- slot-mapping append and block copy on host arrays
  allocator  -- the reference block allocator (pure Python)
  fp8        -- E4M3 codes for an 8-bit cache: value table, quantise, dequantise

Parity status: every function here is pinned by tests/test_oracle*.py against
closed forms, hand-worked fixtures under tests/golden/, brute force on tiny
inputs, and torch's own scaled_dot_product_attention in float64 on the CPU.
"""

from .attention import gather_kv, paged_decode, paged_prefill, dense_attention
from .kvstore import kv_append, copy_blocks, slot_of
from .allocator import RefAllocator, OutOfBlocks
from . import fp8

__all__ = [
    "gather_kv",
    "paged_decode",
    "paged_prefill",
    "dense_attention",
    "kv_append",
    "copy_blocks",
    "slot_of",
    "RefAllocator",
    "OutOfBlocks",
    "fp8",
]
