"""Ragged batches: sequences of one batch with their own prefix and tree sizes.

[P3] section 4 (batch sizes above one are the method's weak spot) and its closing
remarks (continuous batching).  Nothing about the arithmetic changes: sequence b is
the single-sequence problem on its own prefix_len[b] prefix rows and tree_len[b]
nodes, its tree rows following its own prefix (k, v row prefix_len[b] + i = node i).
Rows of padded arrays past a sequence's tree are not nodes; they come back as NaN.
"""
from __future__ import annotations

import numpy as np

from .attention import tree_verify_attention
from .accept import accept_greedy, accept_spec


def tree_verify_attention_ragged(q, k, v, parents, prefix_len, tree_len, scale: float):
    """q [B][Nmax][Hq][D]; k, v [B][Hkv][cap][D]; parents [B][Nmax]; prefix_len, tree_len [B]."""
    q = np.asarray(q)
    B, Nmax, Hq, D = q.shape
    out = np.full((B, Nmax, Hq, D), np.nan)
    lse = np.full((B, Nmax, Hq), np.nan)
    for b in range(B):
        n, p = int(tree_len[b]), int(prefix_len[b])
        o, s = tree_verify_attention(q[b:b + 1, :n], k[b:b + 1], v[b:b + 1],
                                     np.asarray(parents)[b:b + 1, :n], p, scale)
        out[b, :n] = o[0]
        lse[b, :n] = s[0]
    return out, lse


def accept_greedy_ragged(tokens, parents, target_argmax, tree_len, max_depth: int):
    """Per sequence: accept_greedy on its first tree_len[b] nodes."""
    res = []
    for b in range(len(tree_len)):
        n = int(tree_len[b])
        res.append(accept_greedy(tokens[b][:n], parents[b][:n], target_argmax[b][:n], max_depth))
    return res


def accept_spec_ragged(tokens, parents, target_logits, draft_logits, draft_row, u_accept,
                       u_sample, tree_len, max_depth: int, mode: str = "sampled",
                       target_lse=None, draft_lse=None):
    """Per sequence: accept_spec on its first tree_len[b] nodes (draft rows as given)."""
    res = []
    for b in range(len(tree_len)):
        n = int(tree_len[b])
        res.append(accept_spec(tokens[b][:n], parents[b][:n], target_logits[b][:n], draft_logits[b],
                               draft_row[b][:n], u_accept[b][:n], u_sample[b][:n], max_depth,
                               mode=mode,
                               target_lse=None if target_lse is None else target_lse[b][:n],
                               draft_lse=None if draft_lse is None else draft_lse[b]))
    return res
