"""KV-cache commit after acceptance.

[P3] section 4 (limitations): a dynamic draft tree leaves its key/value rows
scattered through the cache, which strains cache management.  The pages do not
spell the commit out; the reading implemented here is the plain one: the tree's
K/V rows sit after the prefix in node order (row P + i holds node i), and once a
root path root = path[0], path[1], ..., path[alpha] has been accepted, those
alpha + 1 rows become the next rows of the prefix, in path order:

    new[P + i] = old[P + path[i]]   for i = 0 .. alpha,

in every layer, sequence and KV head.  All other rows keep their contents.  A
sequence whose acceptance failed (alpha < 0) is left unchanged.
"""
from __future__ import annotations

import numpy as np


def kv_commit(cache: np.ndarray, accept_len: np.ndarray, accept_path: np.ndarray, P: int) -> np.ndarray:
    """cache [L][B][Hkv][kv_cap][D] (any dtype); accept_len [B]; accept_path [B][>= alpha+1].

    Returns a new array; ``cache`` is not modified.
    """
    old = np.asarray(cache)
    new = old.copy()
    L, B = old.shape[0], old.shape[1]
    for layer in range(L):
        for b in range(B):
            alpha = int(accept_len[b])
            for i in range(alpha + 1):
                src = P + int(accept_path[b][i])
                new[layer, b, :, P + i, :] = old[layer, b, :, src, :]
    return new
