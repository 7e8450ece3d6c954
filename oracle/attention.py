"""Float64 paged attention: gather through the block table, then plain softmax
attention.  TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where the pages say so:

* Gather -- KV-cache article (intelliparadigm) §2.1, pseudo-code: the logical
  block of position p is p // block_size, its physical page is
  block_tables[seq][p // block_size], and the token sits at row
  p % block_size of that page.  "vLLM 初探" tutorial §1.4 (figure): logical
  blocks of one request map to scattered physical blocks of a shared pool.
* Attention -- same pseudo-code: scores = q K^T, output = softmax(scores) V,
  over the gathered, logically contiguous keys and values.  The explainer's
  closing section states that paging does not change the model's output, so
  the paged result is by definition the dense result over the gathered KV.
* Decode -- explainer, section on serving and the KV cache: each new token
  attends over the K/V of every token before it; the new token's own K/V is
  stored first, so ``context_lens`` counts it (reading: append, then attend).
* Chunked prefill -- article §4.1/§4.2 (long prompts processed in chunks):
  row i of a chunk of c rows, in a sequence whose cache now holds n tokens
  (chunk included), sits at absolute position n - c + i and attends causally
  to positions 0 .. n - c + i inclusive.

Readings where the pages are silent:
  * the softmax takes an explicit ``scale`` multiplying q.k (the pseudo-code
    has none);
  * query head h reads KV head h // (Hq // Hkv) (consecutive groups);
  * a row with no key to attend (context length 0) outputs zeros;
  * cache layout is [num_blocks, num_kv_heads, block_size, head_dim].
"""

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def gather_kv(cache, block_table, n, block_size):
    """Return the first ``n`` tokens of one sequence, logically contiguous.

    cache:        [num_blocks, num_kv_heads, block_size, head_dim]
    block_table:  1-D int array, logical block -> physical block
    returns:      [n, num_kv_heads, head_dim] float64

    Position p is row p % block_size of physical block
    block_table[p // block_size] (article §2.1 pseudo-code).
    """
    cache = np.asarray(cache)
    table = np.asarray(block_table, dtype=np.int64)
    pos = np.arange(int(n), dtype=np.int64)
    physical = table[pos // block_size]
    if n and (physical.min() < 0 or physical.max() >= cache.shape[0]):
        raise ValueError("block table entry outside the physical pool")
    row = pos % block_size
    return _f64(cache[physical, :, row, :])


def dense_attention(q, k, v, scale, first_pos=None):
    """Softmax attention of query rows over one sequence's contiguous K/V.

    q:  [Lq, Hq, D];  k, v: [n, Hkv, D]
    first_pos: None -> every row sees all n keys (decode);
               an int  -> causal: row i sits at position first_pos + i and
               sees keys 0 .. first_pos + i inclusive (chunked prefill).
    returns [Lq, Hq, D] float64.

    s_t = scale * sum_d q_d k_{t,d};  w_t = exp(s_t - max_t s_t);
    o = sum_t w_t v_t / sum_t w_t  (article §2.1 pseudo-code, softmax(q K^T) V;
    subtracting the max leaves the exact value unchanged).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    lq, hq, d = q.shape
    n, hkv, _ = k.shape
    if hq % hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    group = hq // hkv
    out = np.zeros((lq, hq, d), dtype=np.float64)
    if n == 0 or lq == 0:
        return out
    if first_pos is None:
        visible = np.full(lq, n, dtype=np.int64)
    else:
        visible = np.minimum(first_pos + np.arange(lq, dtype=np.int64) + 1, n)
    allowed = np.arange(n)[None, :] < visible[:, None]  # [Lq, n]
    for h in range(hq):
        g = h // group
        s = scale * (q[:, h, :] @ k[:, g, :].T)  # [Lq, n]
        s = np.where(allowed, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        m = np.where(np.isfinite(m), m, 0.0)
        w = np.where(allowed, np.exp(s - m), 0.0)
        den = w.sum(axis=1, keepdims=True)
        num = w @ v[:, g, :]
        out[:, h, :] = np.where(den > 0, num / np.where(den > 0, den, 1.0), 0.0)
    return out


def paged_decode(q, k_cache, v_cache, block_tables, context_lens, scale,
                 block_size, seqs=None):
    """One decode step: each sequence's single query row over its paged KV.

    q:             [B, Hq, D]
    k_cache/v_cache [num_blocks, Hkv, block_size, D]
    block_tables:  [B, max_blocks] int (entries past the used ones ignored)
    context_lens:  [B] int, tokens in the cache for each sequence
    seqs:          optional iterable of sequence indices to compute (others
                   are left zero) so large batches can be sampled.
    returns [B, Hq, D] float64.
    """
    q = _f64(q)
    b_count = q.shape[0]
    out = np.zeros(q.shape, dtype=np.float64)
    for b in (range(b_count) if seqs is None else seqs):
        n = int(context_lens[b])
        k = gather_kv(k_cache, block_tables[b], n, block_size)
        v = gather_kv(v_cache, block_tables[b], n, block_size)
        out[b] = dense_attention(q[b][None], k, v, scale)[0]
    return out


def paged_prefill(q, k_cache, v_cache, block_tables, context_lens, cu_q_lens,
                  scale, block_size, seqs=None):
    """Causal chunked prefill against the paged cache.

    q:          [sum_b c_b, Hq, D]; rows cu_q_lens[b] .. cu_q_lens[b+1]-1
                belong to sequence b (its chunk of c_b rows).
    context_lens[b] counts the cached tokens including the chunk, so chunk
    row i is at position context_lens[b] - c_b + i.
    returns [sum_b c_b, Hq, D] float64.
    """
    q = _f64(q)
    out = np.zeros(q.shape, dtype=np.float64)
    b_count = len(cu_q_lens) - 1
    for b in (range(b_count) if seqs is None else seqs):
        lo, hi = int(cu_q_lens[b]), int(cu_q_lens[b + 1])
        c, n = hi - lo, int(context_lens[b])
        if c > n:
            raise ValueError("chunk longer than the cached context")
        k = gather_kv(k_cache, block_tables[b], n, block_size)
        v = gather_kv(v_cache, block_tables[b], n, block_size)
        out[lo:hi] = dense_attention(q[lo:hi], k, v, scale, first_pos=n - c)
    return out
