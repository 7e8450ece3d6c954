"""Reference block allocator, pure Python.  TEST INFRASTRUCTURE ONLY.

The pages give the mechanism; the orderings below are this project's stated
reading, and the native allocator must reproduce them bit for bit.

Mechanism, as the pages state it:
* "vLLM 初探" tutorial §1.4 and explainer (openEuler/CSDN) section
  "vLLM的核心创新：PagedAttention": the cache is a pool of equal blocks; a
  sequence takes a new block only when it grows into it; its block table
  lists its blocks in logical order; when the request ends every block goes
  straight back to the pool and any free block can serve any request.
* explainer section "PagedAttention带来的额外红利：内存共享" and tutorial §1.4:
  requests (or beams) with an identical prefix point their tables at the same
  physical blocks, so the prefix is stored once.
* KV-cache article (intelliparadigm) §2.1 pseudo-code: position p lives in
  logical block p // block_size at physical block table[p // block_size],
  i.e. flat slot table[p // block_size] * block_size + p % block_size;
  article §2.2: growth takes a new page and updates the table, nothing moves.

Readings (the pages fix none of these):
* free blocks form a stack; ``create`` pushes ``init_order`` so that
  init_order[0] is popped first; a released block is pushed on top.
* a shared block carries a reference count = number of tables holding it.
* ``fork(parent, child)``: the child gets a copy of the parent's table and
  length, every block's count goes up by one.
* ``append(seq, n)``: copy-on-write happens once, before anything else, when
  n > 0, the length is not a multiple of block_size and the last block's
  count is above 1: a fresh block is popped, the table's last entry is
  replaced, the old block's count drops by one, and the (old, new) pair is
  reported so the caller can copy the data.  Then each position p that starts
  a block pops a new one.  Slots are reported in position order.
* ``free(seq)``: the sequence's blocks are released in logical order; a
  block whose count reaches zero is pushed on the free stack.
* a call that would need more blocks than are free fails and changes nothing;
  a batch append is all-or-nothing over the whole batch.

Swap space (KV-cache article §4.2: host memory as swap space when device
memory runs out; §5: a page pool spanning GPU and CPU memory).  Readings:
* a second pool of host blocks with its own stack (block 0 popped first);
  host blocks are never shared.
* ``swap_out(seq)``: for each block of the table in logical order a host
  block is popped, the pair (device, host) reported, and the device block
  released as ``free`` releases it; the table then lists the host blocks
  and the sequence is marked swapped.  ``swap_in(seq)``: for each host
  block in logical order a device block is popped (count 1), the pair
  (host, device) reported and the host block pushed back.  Each fails
  with nothing changed if its target pool lacks blocks.
* a swapped sequence cannot grow, fork or be packed into device tables;
  ``free`` pushes its host blocks back in logical order.
"""


class OutOfBlocks(Exception):
    """The pool has too few free blocks for the request; state unchanged."""


def _cdiv(a, b):
    return -(-a // b)


class RefAllocator:
    def __init__(self, num_blocks, block_size, init_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if init_order is None else [int(x) for x in init_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("init_order must be a permutation of the pool")
        self.num_blocks = num_blocks
        self.block_size = block_size
        # Python list with the stack top at the END: pop() yields order[0] first.
        self._free = list(reversed(order))
        self.ref = [0] * num_blocks
        self.tables = {}
        self.lens = {}
        self.swapped = set()
        self._host_free = []
        self.num_host_blocks = 0

    # -- queries --------------------------------------------------------
    def num_free(self):
        return len(self._free)

    def free_stack(self):
        """Free blocks, top of the stack first."""
        return list(reversed(self._free))

    def table(self, seq):
        return list(self.tables[seq])

    def length(self, seq):
        return self.lens[seq]

    def snapshot(self):
        return (self.free_stack(), list(self.ref),
                {s: (list(t), self.lens[s]) for s, t in self.tables.items()})

    # -- sequence lifetime ------------------------------------------------
    def add(self, seq):
        if seq in self.tables:
            raise ValueError("sequence already exists")
        self.tables[seq] = []
        self.lens[seq] = 0

    def fork(self, parent, child):
        if parent not in self.tables:
            raise KeyError(parent)
        if parent in self.swapped:
            raise ValueError("sequence is swapped out")
        if child in self.tables:
            raise ValueError("child sequence already exists")
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1

    def free(self, seq):
        if seq not in self.tables:
            raise KeyError(seq)
        if seq in self.swapped:
            self._host_free += self.tables.pop(seq)
            self.swapped.discard(seq)
        else:
            for b in self.tables.pop(seq):
                self.ref[b] -= 1
                if self.ref[b] == 0:
                    self._free.append(b)
        del self.lens[seq]

    # -- swap space -------------------------------------------------------
    def set_host_pool(self, num_host_blocks):
        if num_host_blocks < 0:
            raise ValueError("negative host pool")
        if self.swapped:
            raise ValueError("the host pool is in use")
        self.num_host_blocks = num_host_blocks
        self._host_free = list(reversed(range(num_host_blocks)))

    def num_free_host(self):
        return len(self._host_free)

    def host_free_stack(self):
        return list(reversed(self._host_free))

    def swap_out(self, seq):
        if seq not in self.tables:
            raise KeyError(seq)
        if seq in self.swapped:
            raise ValueError("already swapped out")
        table = self.tables[seq]
        if len(table) > len(self._host_free):
            raise OutOfBlocks(seq)
        pairs, host = [], []
        for b in table:
            h = self._host_free.pop()
            pairs.append((b, h))
            host.append(h)
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self._free.append(b)
        self.tables[seq] = host
        self.swapped.add(seq)
        return pairs

    def swap_in(self, seq):
        if seq not in self.tables:
            raise KeyError(seq)
        if seq not in self.swapped:
            raise ValueError("not swapped out")
        table = self.tables[seq]
        if len(table) > len(self._free):
            raise OutOfBlocks(seq)
        pairs, dev = [], []
        for h in table:
            b = self._free.pop()
            self.ref[b] = 1
            pairs.append((h, b))
            dev.append(b)
            self._host_free.append(h)
        self.tables[seq] = dev
        self.swapped.discard(seq)
        return pairs

    # -- growth -------------------------------------------------------------
    def _needs(self, seq, n):
        """(new blocks, copy-on-write?) for appending n tokens to seq."""
        length, table = self.lens[seq], self.tables[seq]
        fresh = _cdiv(length + n, self.block_size) - _cdiv(length, self.block_size)
        cow = n > 0 and length % self.block_size != 0 and self.ref[table[-1]] > 1
        return fresh, cow

    def append(self, seq, n):
        """Grow seq by n tokens.  Returns (slots, cow_pairs)."""
        if seq not in self.tables:
            raise KeyError(seq)
        if n < 0:
            raise ValueError("negative token count")
        if seq in self.swapped:
            raise ValueError("sequence is swapped out")
        fresh, cow = self._needs(seq, n)
        if fresh + int(cow) > len(self._free):
            raise OutOfBlocks(seq)
        table, bs = self.tables[seq], self.block_size
        pairs = []
        if cow:
            old, new = table[-1], self._free.pop()
            self.ref[new] = 1
            self.ref[old] -= 1
            table[-1] = new
            pairs.append((old, new))
        slots = []
        start = self.lens[seq]
        for p in range(start, start + n):
            if p % bs == 0:
                b = self._free.pop()
                self.ref[b] = 1
                table.append(b)
            slots.append(table[p // bs] * bs + p % bs)
        self.lens[seq] = start + n
        return slots, pairs

    def append_batch(self, seqs, counts):
        """Append counts[i] tokens to seqs[i] in order, all or nothing.
        Returns (slots concatenated in batch order, cow pairs in order)."""
        seqs = list(seqs)
        counts = [int(c) for c in counts]
        if len(seqs) != len(counts):
            raise ValueError("seqs and counts differ in length")
        if len(set(seqs)) != len(seqs):
            raise ValueError("a sequence appears twice in one batch")
        for s, c in zip(seqs, counts):
            if s not in self.tables:
                raise KeyError(s)
            if c < 0:
                raise ValueError("negative token count")
            if s in self.swapped:
                raise ValueError("sequence is swapped out")
        saved = (list(self._free), list(self.ref),
                 {s: list(t) for s, t in self.tables.items()}, dict(self.lens))
        slots, pairs = [], []
        try:
            for s, c in zip(seqs, counts):
                sl, pr = self.append(s, c)
                slots += sl
                pairs += pr
        except OutOfBlocks:
            self._free, self.ref, self.tables, self.lens = saved
            raise
        return slots, pairs

    def build_tables(self, seqs, max_blocks):
        """Padded [len(seqs), max_blocks] table (-1 beyond the used blocks)
        and the lengths, as plain lists."""
        rows, lens = [], []
        for s in seqs:
            t = self.tables[s]
            if s in self.swapped:
                raise ValueError("sequence is swapped out")
            if len(t) > max_blocks:
                raise ValueError("max_blocks too small")
            rows.append(t + [-1] * (max_blocks - len(t)))
            lens.append(self.lens[s])
        return rows, lens
