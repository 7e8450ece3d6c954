"""Host-array versions of the cache writes: slot-mapped append and block copy.
TEST INFRASTRUCTURE ONLY (see the package docstring).

* Slot of a position -- KV-cache article (intelliparadigm) §2.1 pseudo-code:
  position p of a sequence is row p % block_size of physical block
  block_tables[seq][p // block_size]; its flat slot number in the pool is
  physical * block_size + p % block_size.
* Append -- explainer (openEuler/CSDN), serving section: every stored token
  adds one K and one V vector that stays in the cache until the request ends;
  article §2.2: growth only takes a new page and updates the table, no data
  already stored moves.
* Block copy -- the copy-on-write step of sharing (explainer, "内存共享"
  section; tutorial §1.4): before a shared, partly filled block is written,
  its contents are duplicated into a private block.
"""

import numpy as np


def slot_of(block_table, pos, block_size):
    """Flat pool slot of logical position ``pos`` (article §2.1)."""
    physical = int(block_table[pos // block_size])
    return physical * block_size + pos % block_size


def kv_append(k_cache, v_cache, k_new, v_new, slot_mapping, block_size):
    """Write row r of k_new/v_new ([T, Hkv, D]) into the caches
    ([num_blocks, Hkv, block_size, D]) at flat slot slot_mapping[r].

    A negative slot means "skip this row".  Slots outside the pool and a slot
    named twice in one call are rejected (the result would depend on order).
    Modifies the caches in place and returns them.
    """
    slots = np.asarray(slot_mapping, dtype=np.int64)
    total = k_cache.shape[0] * block_size
    live = slots[slots >= 0]
    if live.size and live.max() >= total:
        raise ValueError("slot outside the pool")
    if np.unique(live).size != live.size:
        raise ValueError("slot named twice in one append")
    for r, s in enumerate(slots):
        if s < 0:
            continue
        blk, row = divmod(int(s), block_size)
        k_cache[blk, :, row, :] = k_new[r]
        v_cache[blk, :, row, :] = v_new[r]
    return k_cache, v_cache


def copy_blocks(k_cache, v_cache, src, dst):
    """For each pair i, make physical block dst[i] an exact copy of src[i]
    in both caches.  A block may not be a destination twice, nor be both a
    source and a destination in one call (so pair order cannot matter)."""
    src = [int(x) for x in src]
    dst = [int(x) for x in dst]
    if len(src) != len(dst):
        raise ValueError("src and dst differ in length")
    if len(set(dst)) != len(dst) or set(dst) & set(src):
        raise ValueError("overlapping copy pairs")
    nb = k_cache.shape[0]
    for s, d in zip(src, dst):
        if not (0 <= s < nb and 0 <= d < nb):
            raise ValueError("block outside the pool")
        k_cache[d] = k_cache[s]
        v_cache[d] = v_cache[s]
    return k_cache, v_cache
