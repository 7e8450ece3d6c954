"""Reference continuous-batching scheduler, pure Python.  TEST INFRASTRUCTURE ONLY.

Mechanism, as the pages state it:
* "vLLM 初探" tutorial §1.3: requests join and leave the running batch
  dynamically; a short request that finishes releases its resources at once
  for a new one instead of waiting for the longest; §1.5 contrasts that
  dynamic scheduling with static batches.
* explainer (openEuler/CSDN), continuous-batching section: at every decode
  step the finished requests leave the batch and waiting requests are
  pulled in to fill the places; its over-reservation section: a naive
  engine reserves room for the longest possible reply (2000 tokens in its
  example) for every request.
* KV-cache article (intelliparadigm) §3.2: a cap on concurrent sequences
  (max_num_seqs); §4.1/§4.2: long prompts prefilled in chunks (512 tokens).

Policy (the pages fix none of it; this is the library's stated reading,
which the native scheduler must reproduce step for step):
* A request (id, prompt P, output O) is prefilled in chunks, then gets one
  decode row per step until it has had O of them; its cache holds the
  tokens prefilled plus those generated.
* Each step: (1) retire every running request with O decode rows done
  (release its blocks); (2) admit from the head of the FIFO queue while
  fewer than max_num_seqs run and, for paged admission, the free blocks
  cover the request's whole prompt, the prompt blocks the running requests
  have yet to take, and one block per running request, or,
  for the reservation model, while (running + 1) reservations of
  ceil(reserve_tokens / block_size) blocks fit the pool; (3) give every
  request whose prompt is done one decode row, oldest first, while the
  token budget lasts; when its block does not fit, preempt the youngest
  running request that has no row yet in this step (possibly itself):
  release its blocks, fold its generated tokens into its prompt, reset it
  and put it at the head of the queue; (4) give prompt chunks of
  min(P - prefilled, chunk_size, budget left) tokens, oldest first; a chunk
  that does not fit may preempt younger requests without a row; if it
  still does not fit, prefill stops for this step.
* Rows are reported decode rows first, then chunks: (id, query length,
  context length after the step, block table), plus the slots in row order.
* With a host tier (KV-cache article §4.2: swap space in host memory), a
  preempted request whose blocks fit the tier's free blocks is swapped out
  instead (its progress kept; pairs device -> host reported); when such a
  request heads the queue it is admitted if the free blocks cover its own
  blocks plus the running requests' pending prompt blocks plus one per
  running request, and swapped back in (pairs host -> device).

Parity pins: tests/test_oracle_scheduler.py replays hand-worked traces
(tests/golden/scheduler_traces.json) and checks invariants (budget, cap,
chunk bounds, every request finishing with exactly its tokens, slots
distinct and matching the tables, no preemption under the reservation
model) on random traces.
"""

from collections import deque

from .allocator import OutOfBlocks, RefAllocator


def _cdiv(a, b):
    return -(-a // b)


class _Req:
    def __init__(self, rid, prompt, output):
        self.id, self.prompt, self.output = rid, prompt, output
        self.prefilled = 0
        self.generated = 0
        self.swapped = False


class RefScheduler:
    def __init__(self, num_blocks, block_size, max_num_seqs, max_num_batched_tokens, chunk_size,
                 reserve_tokens=0, init_order=None, host_blocks=0):
        self.alloc = RefAllocator(num_blocks, block_size, init_order)
        self.alloc.set_host_pool(host_blocks)
        self.host_blocks = host_blocks
        self.total_swapped_out = 0
        self.total_swapped_in = 0
        self.num_blocks, self.block_size = num_blocks, block_size
        self.max_num_seqs = max_num_seqs
        self.budget = max_num_batched_tokens
        self.chunk = chunk_size
        self.reserve = reserve_tokens
        self.waiting = deque()
        self.running = []          # oldest first
        self.steps = 0
        self.total_finished = 0
        self.total_preempted = 0

    def add_request(self, rid, prompt, output):
        if prompt < 1 or output < 1:
            raise ValueError("prompt and output must be positive")
        if _cdiv(prompt + output, self.block_size) > self.num_blocks:
            raise ValueError("request never fits the pool")
        if self.reserve and prompt + output > self.reserve:
            raise ValueError("request exceeds the reservation")
        if rid in self.alloc.tables or any(r.id == rid for r in self.waiting):
            raise ValueError("request id in use")
        self.waiting.append(_Req(rid, prompt, output))

    def _admissible(self, r):
        if len(self.running) >= self.max_num_seqs:
            return False
        if self.reserve:
            return (len(self.running) + 1) * _cdiv(self.reserve, self.block_size) <= self.num_blocks
        # the prompt's blocks, the prompt blocks running requests have yet
        # to take, one block per running request
        pending = 0
        for x in self.running:
            if x.prefilled < x.prompt:
                pending += _cdiv(x.prompt, self.block_size) - len(self.alloc.tables[x.id])
        own = len(self.alloc.tables[r.id]) if r.swapped else _cdiv(r.prompt, self.block_size)
        need = own + pending + len(self.running)
        return self.alloc.num_free() >= need

    def _preempt_youngest(self, candidates, has_row, preempted, swap_out):
        """Preempt the youngest request in `candidates` (a list of running
        requests, oldest first) without a row this step; return it or None."""
        for r in reversed(candidates):
            if r.id in has_row:
                continue
            if self.host_blocks and len(self.alloc.tables[r.id]) <= self.alloc.num_free_host():
                swap_out += self.alloc.swap_out(r.id)
                r.swapped = True
                self.total_swapped_out += 1
            else:
                self.alloc.free(r.id)
                r.prompt += r.generated
                r.output -= r.generated
                r.prefilled = r.generated = 0
            self.running.remove(r)
            self.waiting.appendleft(r)
            preempted.append(r.id)
            self.total_preempted += 1
            return r
        return None

    def step(self):
        """Returns a dict: rows [(id, qlen, ctx, table)], num_decode, slots,
        finished, preempted."""
        self.steps += 1
        finished, preempted, swap_in, swap_out = [], [], [], []
        # 1. retire
        for r in list(self.running):
            if r.generated == r.output:
                self.alloc.free(r.id)
                self.running.remove(r)
                finished.append(r.id)
                self.total_finished += 1
        # 2. admit
        while self.waiting and self._admissible(self.waiting[0]):
            r = self.waiting.popleft()
            if r.swapped:
                swap_in += self.alloc.swap_in(r.id)
                r.swapped = False
                self.total_swapped_in += 1
            else:
                self.alloc.add(r.id)
            self.running.append(r)
        budget = self.budget
        rows, slots, has_row = [], [], set()
        # 3. decode rows
        for r in list(self.running):
            if budget == 0:
                break
            if r not in self.running or r.prefilled < r.prompt:
                continue
            got = None
            while got is None:
                try:
                    got, _ = self.alloc.append(r.id, 1)
                except OutOfBlocks:
                    idx = self.running.index(r)
                    victim = self._preempt_youngest(self.running[idx:], has_row, preempted,
                                                    swap_out)
                    if victim is r:
                        break
            if got is None:
                break
            r.generated += 1
            rows.append((r.id, 1, self.alloc.length(r.id), self.alloc.table(r.id)))
            slots += got
            has_row.add(r.id)
            budget -= 1
        num_decode = len(rows)
        # 4. prompt chunks
        for r in list(self.running):
            if budget == 0:
                break
            if r not in self.running or r.prefilled >= r.prompt:
                continue
            c = min(r.prompt - r.prefilled, self.chunk, budget)
            got = None
            while got is None:
                try:
                    got, _ = self.alloc.append(r.id, c)
                except OutOfBlocks:
                    idx = self.running.index(r)
                    if self._preempt_youngest(self.running[idx + 1:], has_row, preempted,
                                              swap_out) is None:
                        break
            if got is None:
                break
            r.prefilled += c
            rows.append((r.id, c, self.alloc.length(r.id), self.alloc.table(r.id)))
            slots += got
            has_row.add(r.id)
            budget -= c
        return {"rows": rows, "num_decode": num_decode, "slots": slots, "finished": finished,
                "preempted": preempted, "swap_in": swap_in, "swap_out": swap_out}

    def stats(self):
        bs = self.block_size
        cached = sum(self.alloc.length(r.id) for r in self.running)
        held = sum(len(self.alloc.tables[r.id]) * bs for r in self.running)
        reserved = (len(self.running) * _cdiv(self.reserve, bs) * bs) if self.reserve else held
        return {"steps": self.steps, "running": len(self.running), "waiting": len(self.waiting),
                "finished": self.total_finished, "preemptions": self.total_preempted,
                "cached_tokens": cached, "allocated_slots": held, "reserved_slots": reserved,
                "free_blocks": self.alloc.num_free(), "swapped_out": self.total_swapped_out,
                "swapped_in": self.total_swapped_in}
