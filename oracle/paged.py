"""Tree-verify attention over a paged KV cache.

[P3] section 4 (limitations): dynamic draft trees strain paged cache management
(PagedAttention is named).  The reading implemented here: the cache of each
(sequence, KV head) is cut into pages of page_size rows; a pool holds blocks
[num_blocks][Hkv][page_size][D], and row r of sequence b lives in block
block_table[b][r // page_size] at slot r % page_size.  The attention itself is
unchanged: gather the rows, then the contiguous definition.
"""
from __future__ import annotations

import numpy as np

from .attention import tree_verify_attention


def gather_pages(pool, block_table, rows: int, page_size: int):
    """pool [num_blocks][Hkv][page_size][D], block_table [B][max_pages] ->
    contiguous cache [B][Hkv][rows][D]."""
    pool = np.asarray(pool)
    B = len(block_table)
    Hkv, D = pool.shape[1], pool.shape[3]
    out = np.empty((B, Hkv, rows, D), dtype=pool.dtype)
    for b in range(B):
        for r in range(rows):
            blk = int(block_table[b][r // page_size])
            out[b, :, r, :] = pool[blk, :, r % page_size, :]
    return out


def tree_verify_attention_paged(q, k_pool, v_pool, block_table, parents, P: int, page_size: int,
                                scale: float):
    """q [B][N][Hq][D]; pools [num_blocks][Hkv][page_size][D]; rows 0 .. P+N-1 used."""
    N = np.asarray(q).shape[1]
    k = gather_pages(k_pool, block_table, P + N, page_size)
    v = gather_pages(v_pool, block_table, P + N, page_size)
    return tree_verify_attention(q, k, v, parents, P, scale)
