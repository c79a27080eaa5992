"""Tree-verify attention, written as its plain definition.

[P1] innovations list, item 2 (tree verification), and [P2] workflow paragraph:
the target checks every draft path in one forward pass by turning the tree into
an attention mask.  Plain reading used here: tree node i, at query head h, attends
to every prefix key 0..P-1 and to the tree keys of its own ancestors and itself
(key P+a for a in anc*(i)); nothing else.  Scores are scale * <q, k>; the output is
the softmax-weighted sum of values.  Grouped-query heads: head h reads KV head
h // (Hq // Hkv).  q and k arrive already position-encoded (the pages do not
mention positions; they only decide the mask).
"""
from __future__ import annotations

import numpy as np

from .tree import ancestor_sets


def tree_verify_attention_node(q_heads, k_bg, v_bg, anc_i, P: int, scale: float):
    """Attention of one tree node for the G query heads of one KV head.

    q_heads [G][D]; k_bg, v_bg [L][D] (prefix rows 0..P-1, then tree rows in node
    order); anc_i = anc*(i).  Returns out [G][D] and lse [G] (natural log of the
    softmax denominator of the scaled scores), both fp64.
    """
    q_heads = np.asarray(q_heads, dtype=np.float64)
    tree_rows = [P + a for a in sorted(anc_i)]
    # the key set is the union of the prefix and the ancestor path
    s_prefix = scale * (np.asarray(k_bg[:P], dtype=np.float64) @ q_heads.T)      # [P][G]
    s_tree = scale * (np.asarray(k_bg[tree_rows], dtype=np.float64) @ q_heads.T)  # [|anc|][G]
    s = np.concatenate([s_prefix, s_tree], axis=0)
    vals = np.concatenate([np.asarray(v_bg[:P], dtype=np.float64),
                           np.asarray(v_bg[tree_rows], dtype=np.float64)], axis=0)
    m = s.max(axis=0)
    w = np.exp(s - m)
    z = w.sum(axis=0)
    out = (w.T @ vals) / z[:, None]
    lse = m + np.log(z)
    return out, lse


def tree_verify_attention(q, k, v, parents, P: int, scale: float):
    """q [B][N][Hq][D]; k, v [B][Hkv][L][D] with L >= P + N; parents [B][N].

    Returns out [B][N][Hq][D] and lse [B][N][Hq] in fp64.
    """
    q = np.asarray(q)
    B, N, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, N, Hq, D), dtype=np.float64)
    lse = np.zeros((B, N, Hq), dtype=np.float64)
    for b in range(B):
        anc = ancestor_sets(parents[b])
        for g in range(Hkv):
            for i in range(N):
                o, l = tree_verify_attention_node(q[b, i, g * G:(g + 1) * G], k[b, g], v[b, g],
                                                  anc[i], P, scale)
                out[b, i, g * G:(g + 1) * G] = o
                lse[b, i, g * G:(g + 1) * G] = l
    return out, lse
