"""Seeded synthetic workloads for paged decode / chunked prefill.

This module only draws inputs: context lengths, the pool's initial free
order, the list of allocator operations that builds each sequence's cache,
and the random K/V/q values.  It holds none of the attention, allocator or
slot arithmetic; both the CPU oracle side and the HIP side of every test,
and bench.py, take their inputs from here.

The pages measure on no public dataset; their workloads are mixed-length
requests (the tutorial §1.1 speaks of outputs from 10 to 2000 tokens, the
KV-cache article §1 of 100- versus 2000-token requests, on LLaMA-7B/13B).
The five configurations below stand in for them with random values.

Recipe (per configuration, ``seed`` fixed):
  1. rng = numpy.random.default_rng(seed); lengths are drawn first, then the
     permutation of the pool, both from this rng, in that order.
  2. The pool holds 2x the blocks the full schedule needs if nothing were
     shared (the tiny configuration states its pool: 32 blocks).
  3. The schedule adds each sequence and appends its tokens in index order;
     the shared-prefix configuration first fills a 1024-token prefix
     sequence, forks every sequence from it, frees the prefix sequence,
     then appends each private suffix.  The grouped-prefix configuration
     does the same per group (consecutive sequences, equal group sizes, the
     last group smaller), group by group, then appends every suffix.
  4. The K/V rows of append op number i come from
     default_rng([seed, 1, i]); queries of sequence b from
     default_rng([seed, 2, b]) (decode) or default_rng([seed, 3, b])
     (prefill chunk), all float32 N(0, std^2), then cast to the cache dtype
     with torch's round-to-nearest-even.  Per-op streams let a test rebuild
     any single sequence without drawing the whole batch.
"""

import dataclasses
import math

import numpy as np
import torch

PREFIX_SEQ = 1 << 40  # id of the shared-prefix sequence in the schedule


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: torch.dtype
    std: float
    seed: int
    lens: str                  # how context lengths are drawn
    num_blocks: int = 0        # 0 = twice the unshared need
    partition_size: int = 0    # split-K partition for decode (0 = library default)
    prefix: int = 0            # shared prefix tokens (shared-prefix workload)
    chunk: int = 0             # chunked-prefill rows per sequence
    prefix_groups: tuple = ()  # per-group prefix tokens (grouped-prefix workload)

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def elem_bytes(self):
        return torch.tensor([], dtype=self.dtype).element_size()


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 4, 4, 4, 64, 16, torch.float32, 1.0, 4201,
                          "fixed:17,33,64,100", num_blocks=32),
    "llama7b_bf16": Workload("llama7b_bf16", 64, 32, 32, 128, 16, torch.bfloat16, 1.0, 4202,
                             "uniform:100,2000"),
    "llama13b_fp16": Workload("llama13b_fp16", 128, 40, 40, 128, 32, torch.float16, 0.5, 4203,
                              "geometric:600,10,5000"),
    "gqa_bf16": Workload("gqa_bf16", 256, 64, 8, 128, 16, torch.bfloat16, 1.0, 4204,
                         "uniform:512,8192", partition_size=512),
    "shared_prefix_bf16": Workload("shared_prefix_bf16", 256, 32, 32, 128, 16, torch.bfloat16,
                                   1.0, 4205, "uniform:10,2000", prefix=1024, chunk=512),
    # the shared-prefix batch as four prompts with 64 samples each
    "grouped_prefix_bf16": Workload("grouped_prefix_bf16", 256, 32, 32, 128, 16,
                                    torch.bfloat16, 1.0, 4207, "uniform:10,2000",
                                    prefix_groups=(1024, 512, 1536, 768)),
}


# Per-tensor scales of the 8-bit (E4M3) cache for the N(0, 1) workloads:
# 8 standard deviations map to the largest code value, 448, so saturation
# is practically never reached and the codes' normal range covers
# |x| >= 8 * 2^-6 / 448 (about 2.8e-4).
FP8_SCALES = (8.0 / 448.0, 8.0 / 448.0)


def get(name):
    return WORKLOADS[name]


def scaled(w, **changes):
    """A copy of workload ``w`` with some fields replaced (smaller test cases)."""
    return dataclasses.replace(w, **changes)


def draw_lengths(w, rng):
    kind, _, arg = w.lens.partition(":")
    if kind == "fixed":
        vals = [int(x) for x in arg.split(",")]
        return np.array((vals * w.num_seqs)[:w.num_seqs], dtype=np.int64)
    if kind == "uniform":
        lo, hi = (int(x) for x in arg.split(","))
        return rng.integers(lo, hi, endpoint=True, size=w.num_seqs).astype(np.int64)
    if kind == "geometric":
        mean, lo, hi = (int(x) for x in arg.split(","))
        return rng.geometric(1.0 / mean, size=w.num_seqs).clip(lo, hi).astype(np.int64)
    raise ValueError(w.lens)


def prefix_layout(w):
    """(group_starts, prefix_lens) of the batch's prefix groups -- group g is
    sequences group_starts[g] .. group_starts[g + 1] - 1, sharing their
    first prefix_lens[g] tokens -- or None when nothing is shared."""
    if w.prefix_groups:
        n = len(w.prefix_groups)
        size = -(-w.num_seqs // n)
        starts = [min(g * size, w.num_seqs) for g in range(n)] + [w.num_seqs]
        return starts, list(w.prefix_groups)
    if w.prefix:
        return [0, w.num_seqs], [w.prefix]
    return None


def seq_prefixes(w):
    """Shared-prefix tokens of each sequence (int64 [num_seqs])."""
    out = np.zeros(w.num_seqs, dtype=np.int64)
    layout = prefix_layout(w)
    if layout:
        starts, lens = layout
        for g, n in enumerate(lens):
            out[starts[g]:starts[g + 1]] = n
    return out


@dataclasses.dataclass
class Plan:
    workload: Workload
    lens: np.ndarray          # per sequence: tokens appended by the schedule (suffix only for shared prefix)
    num_blocks: int
    free_order: np.ndarray    # int32 permutation of the pool
    ops: list                 # ("add", s) | ("append", s, n) | ("fork", parent, child) | ("free", s)
    seqs: list                # sequence ids, batch order


def plan(w):
    rng = np.random.default_rng(w.seed)
    lens = draw_lengths(w, rng)
    per_seq_final = lens + seq_prefixes(w) + w.chunk
    nb = w.num_blocks or 2 * int(sum(-(-int(n) // w.block_size) for n in per_seq_final))
    order = rng.permutation(nb).astype(np.int32)
    ops = []
    seqs = list(range(w.num_seqs))
    if w.prefix:
        ops += [("add", PREFIX_SEQ), ("append", PREFIX_SEQ, w.prefix)]
        ops += [("fork", PREFIX_SEQ, s) for s in seqs]
        ops += [("free", PREFIX_SEQ)]
        ops += [("append", s, int(n)) for s, n in zip(seqs, lens)]
    elif w.prefix_groups:
        starts, plens = prefix_layout(w)
        for g, n in enumerate(plens):
            parent = PREFIX_SEQ + g
            ops += [("add", parent)] + ([("append", parent, n)] if n else [])
            ops += [("fork", parent, s) for s in seqs[starts[g]:starts[g + 1]]]
            ops += [("free", parent)]
        ops += [("append", s, int(n)) for s, n in zip(seqs, lens)]
    else:
        for s, n in zip(seqs, lens):
            ops += [("add", s), ("append", s, int(n))]
    return Plan(w, lens, nb, order, ops, seqs)


def chunk_ops(p):
    """The chunked-prefill growth: one append of ``chunk`` rows per sequence."""
    return [("append", s, p.workload.chunk) for s in p.seqs]


def normal(key, shape, std):
    return (np.random.default_rng(key).standard_normal(shape, dtype=np.float32) * np.float32(std))


def kv_rows(w, op_index, n):
    """K and V rows written by append op number ``op_index``: two float32
    arrays [n, num_kv_heads, head_dim]."""
    shape = (n, w.num_kv_heads, w.head_dim)
    both = normal([w.seed, 1, op_index], (2,) + shape, w.std)
    return both[0], both[1]


def decode_query(w, seq_index):
    return normal([w.seed, 2, seq_index], (w.num_heads, w.head_dim), w.std)


def prefill_query(w, seq_index, rows):
    return normal([w.seed, 3, seq_index], (rows, w.num_heads, w.head_dim), w.std)


def to_dtype(x, dtype):
    """float32 numpy -> torch CPU tensor of ``dtype`` (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype)


def as_f64(t):
    """Exact float64 numpy copy of a torch tensor of any float dtype."""
    return t.detach().to("cpu", torch.float64).numpy()


def run_schedule(ops, alloc, on_append=None, on_copy=None, first_index=0):
    """Apply allocator ops in order through any allocator with the
    add/free/fork/append interface.  ``on_copy(pairs)`` is called before
    ``on_append(op_index, seq, n, slots)`` for each append."""
    for i, op in enumerate(ops, start=first_index):
        kind = op[0]
        if kind == "add":
            alloc.add(op[1])
        elif kind == "free":
            alloc.free(op[1])
        elif kind == "fork":
            alloc.fork(op[1], op[2])
        elif kind == "append":
            slots, pairs = alloc.append(op[1], op[2])
            if on_copy is not None and pairs:
                on_copy(pairs)
            if on_append is not None:
                on_append(i, op[1], op[2], slots)
        else:
            raise ValueError(op)


# ---------------------------------------------------------------------------
# Continuous-batching traces
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class ServingTrace:
    """Requests of a continuous-batching run, all queued at the start (an
    offline batch), with the layer shape their attention runs at."""
    name: str
    num_requests: int
    prompt: str                 # length law of prompts (as Workload.lens)
    output: str                 # length law of decode steps per request
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: torch.dtype
    num_blocks: int
    max_num_seqs: int
    max_num_batched_tokens: int
    chunk_size: int
    seed: int
    std: float = 1.0

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.head_dim)


# The LLaMA-7B-shaped layer under a request mix in the pages' terms: prompts
# of 100-2000 tokens (the KV-cache article's 100- vs 2000-token requests),
# replies mostly short but up to 2000 tokens (the explainer's reserve of
# 2000 with 50 used; the 13B batch's geometric law, mean 600, clipped to
# [10, 2000]); 512-token prompt chunks and a 4096-token step budget (the
# article's chunked prefill); at most 256 running requests; a pool of 16384
# blocks of 16 tokens (4.3 GB of bf16 K and V for one layer).
SERVING = {
    "serve_llama7b": ServingTrace("serve_llama7b", 1024, "uniform:100,2000",
                                  "geometric:600,10,2000", 32, 32, 128, 16, torch.bfloat16,
                                  16384, 256, 4096, 512, 4206),
}


def serving_requests(t):
    """(id, prompt, output) of every request, drawn from default_rng(seed):
    prompt lengths first, then output lengths."""
    rng = np.random.default_rng(t.seed)
    pw = Workload("p", t.num_requests, 1, 1, 1, 1, t.dtype, 1.0, 0, t.prompt)
    ow = Workload("o", t.num_requests, 1, 1, 1, 1, t.dtype, 1.0, 0, t.output)
    prompts = draw_lengths(pw, rng)
    outputs = draw_lengths(ow, rng)
    return [(i, int(p), int(o)) for i, (p, o) in enumerate(zip(prompts, outputs))]


def serving_token_kv(t, rid, pos):
    """K and V row of request ``rid`` at position ``pos``: float32 [Hkv, D]
    each, from default_rng([seed, 1, rid, pos])."""
    both = normal([t.seed, 1, rid, pos], (2, t.num_kv_heads, t.head_dim), t.std)
    return both[0], both[1]


def serving_query(t, rid, pos):
    """Query row of request ``rid`` at position ``pos``: float32 [Hq, D]."""
    return normal([t.seed, 2, rid, pos], (t.num_heads, t.head_dim), t.std)
