"""Frozen LM head: hidden states -> next-token distribution.

[P2] (paragraph on the auto-regression head, and the workflow paragraph): the
frozen classification head maps a feature to the next-token distribution.  Here
the head is a plain linear map logits = hidden @ W^T (W in nn.Linear layout
[V][H]), followed by per-row statistics: the maximum, the first index attaining it
(greedy top-1, [P1] greedy decoding paragraph), the largest logit at any other
index (used to judge near-ties), and the log of the softmax normaliser.
"""
from __future__ import annotations

import numpy as np


def lm_head_logits(hidden, W, block: int = 8192, to_f64=None):
    """logits [M][V] = hidden @ W^T in fp64.

    ``W`` may be huge (the 70B-shaped head is 128256 x 8192); it is widened to fp64
    ``block`` vocabulary rows at a time, which only bounds memory: every logit is
    still one independent dot product.  ``to_f64`` converts a block of W (default:
    ``np.asarray(.., float64)``).
    """
    conv = to_f64 or (lambda a: np.asarray(a, dtype=np.float64))
    h = np.asarray(hidden, dtype=np.float64)
    V = W.shape[0]
    out = np.empty((h.shape[0], V), dtype=np.float64)
    for v0 in range(0, V, block):
        out[:, v0:v0 + block] = h @ conv(W[v0:v0 + block]).T
    return out


def lm_head_row_stats(logits):
    """Per row: max, argmax (first occurrence), second (max over the other
    indices), lse = log sum exp."""
    logits = np.asarray(logits, dtype=np.float64)
    mx = logits.max(axis=1)
    am = logits.argmax(axis=1)
    other = logits.copy()
    other[np.arange(logits.shape[0]), am] = -np.inf
    second = other.max(axis=1) if logits.shape[1] > 1 else np.full(logits.shape[0], -np.inf)
    lse = mx + np.log(np.exp(logits - mx[:, None]).sum(axis=1))
    return mx, am.astype(np.int64), second, lse


def lm_head(hidden, W, **kw):
    logits = lm_head_logits(hidden, W, **kw)
    mx, am, second, lse = lm_head_row_stats(logits)
    return logits, mx, am, second, lse
