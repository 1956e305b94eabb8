"""Causal attention of the verified positions over a paged KV cache (oracle
side; test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU baseline
may import this package; the library never does.

The target scores every drafted slot in one pass (NVIDIA co-design post,
"What is speculative decoding?"): the T = K + 1 positions of request b sit at
sequence positions ctx_len[b] .. ctx_len[b] + K, and position t attends to
every earlier position and itself.  The cache is paged (publishertech section
4, "Segmented Block Allocation (PagedAttention)"): fixed-size physical blocks
named by a per-request block table; rolling back rejected positions moves the
committed length and returns trailing blocks to a free list, without copying
any cached data (same section; mohashari, "KV Cache Syncing").

Interface layouts (what the library reads and writes):
  k_cache [num_blocks, Hkv, block_size, Dh], v_cache [num_blocks, Hkv, Dh,
  block_size] (V transposed inside a block), token p of request b in block
  block_table[b][p // block_size] at slot p % block_size; q [B, T, Hq, Dh];
  query head h reads KV head h // (Hq / Hkv).

Pinned by: torch's scaled_dot_product_attention in float64 with a causal
mask on a contiguous cache; invariance under any physical block placement;
q = 0 gives the mean of the visible values; a single visible key returns its
value; after a commit the next step sees exactly the committed prefix.
"""
from __future__ import annotations

import numpy as np


def gather(k_cache, v_cache, table_row, n_tokens, block_size):
    """K, V of the first n_tokens positions of one request: [n, Hkv, Dh] each."""
    pos = np.arange(n_tokens)
    blk = np.asarray(table_row)[pos // block_size]
    slot = pos % block_size
    k = k_cache[blk, :, slot, :]
    v = v_cache[blk, :, :, slot]
    return k.astype(np.float64), v.astype(np.float64)


def attention(q, k_cache, v_cache, block_table, ctx_len, block_size, scale):
    """out[b, t, h] = softmax(scale * K q) V over positions 0 .. ctx_len[b] + t."""
    B, T, Hq, Dh = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, T, Hq, Dh), np.float64)
    for b in range(B):
        k, v = gather(k_cache, v_cache, block_table[b], int(ctx_len[b]) + T, block_size)
        for t in range(T):
            n = int(ctx_len[b]) + t + 1
            for h in range(Hq):
                g = h // G
                s = scale * (k[:n, g, :] @ q[b, t, h].astype(np.float64))
                s = s - s.max()
                p = np.exp(s)
                out[b, t, h] = (p / p.sum()) @ v[:n, g, :]
    return out


def append(k_new, v_new, k_cache, v_cache, block_table, ctx_len, block_size):
    """Write the T new positions of every request at ctx_len[b] + t (in place)."""
    B, T = k_new.shape[:2]
    for b in range(B):
        for t in range(T):
            p = int(ctx_len[b]) + t
            blk = block_table[b][p // block_size]
            k_cache[blk, :, p % block_size, :] = k_new[b, t]
            v_cache[blk, :, :, p % block_size] = v_new[b, t]


def commit(ctx_len, accept_len):
    """Committed length after verification: the AL positions that produced
    the emitted tokens stay (the step's input token and AL - 1 accepted
    drafts); a request rejected as invalid (AL = 0) keeps its length."""
    ctx = np.asarray(ctx_len).copy()
    al = np.asarray(accept_len)
    ctx[al >= 1] += al[al >= 1]
    return ctx


class BlockPool:
    """Free list of physical block ids (a stack: the block freed last is
    reused first; a new pool hands out 0, 1, 2, ...)."""

    def __init__(self, num_blocks):
        self.free = list(range(num_blocks - 1, -1, -1))

    def reserve(self, table_row, tokens, block_size, max_blocks):
        """Append blocks until the row covers `tokens` positions."""
        need = -(-tokens // block_size)
        if need > max_blocks or need - len(table_row) > len(self.free):
            raise MemoryError("not enough blocks")
        while len(table_row) < need:
            table_row.append(self.free.pop())
        return table_row

    def trim(self, table_row, tokens, block_size):
        """Return the blocks past the first `tokens` positions (the rollback)."""
        keep = -(-tokens // block_size)
        while len(table_row) > keep:
            self.free.append(table_row.pop())
        return table_row
