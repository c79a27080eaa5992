"""Per-depth EAGLE-2 draft expansion driven by a one-layer draft head.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[P2], paragraphs on the auto-regression head and the workflow figure: the draft
head reads the target's second-from-top-layer feature together with the embedding
of the token sampled after it, predicts the next feature, and the target's frozen
classification head turns that feature into the next-token distribution;
repeating this grows a token tree (three head passes guess a ten-token tree in
the pages' example).  [P2] training paragraph: the head is a single transformer
layer.  [P3] section 2: EAGLE-2 grows the tree by draft confidence under a fixed
token budget (the expansion of oracle.rerank, whose rows are produced here by the
head, depth by depth).

Readings (the pages fix none of these details):
  * one pre-norm decoder layer (the target family's shape):
        u = [f ; E[t]]                               (2H; f = the parent's feature)
        x = W_fc u                                   (H)
        h = x + W_o Attn(rms(x) * g1)
        y = h + W_down( silu(W_gate b) * (W_up b) ),  b = rms(h) * g2
        logits = W_lm y                              (the frozen LM head)
    with rms(z) = z / sqrt(mean(z^2) + eps), no biases.
  * attention: q = W_q a, k = W_k a, v = W_v a (a = rms(x) * g1), grouped-query
    heads, scale given, no position encoding (positions only enter through the
    mask); a node attends to the draft cache's prefix rows 0..P-1 and to the rows
    of its expanded ancestors and itself (row P + r for expansion row r).
  * the feature a node hands its children is its own y; the root's input feature
    is the target's feature f0 and its token the root token.
  * a bf16 model: weights, embeddings, f0, the draft KV cache and every GEMM input
    (u, a, q/k/v, the attention output, b, the MLP product, y) are bf16 values
    (round to nearest even); accumulation and the residual stream x, h are exact
    here (fp64).
"""
from __future__ import annotations

import numpy as np

from .rerank import grow_tree


def bf16_round(x):
    """Nearest bf16 value (ties to even) of fp64 values, returned as fp64."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    bits = a.view(np.uint64)
    # fp64 keeps 52 fraction bits, bf16 7: drop 45 with round-to-nearest-even
    lsb = (bits >> np.uint64(45)) & np.uint64(1)
    r = (bits + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    return r.view(np.float64)


def rms_norm(z, gain, eps: float):
    z = np.asarray(z, dtype=np.float64)
    return z / np.sqrt(np.mean(z * z) + eps) * np.asarray(gain, dtype=np.float64)


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def draft_layer_row(w, f_in, token: int, k_cache, v_cache, anc_rows, row: int, P: int,
                    scale: float, eps: float):
    """One row of the draft head for one sequence.

    w: dict of fp64 arrays (bf16 values): embed [V][H], fc [H][2H], q [Hq*D][H],
    k [Hkv*D][H], v [Hkv*D][H], o [H][Hq*D], gate [I][H], up [I][H], down [H][I],
    lm [V][H]; g1, g2 [H]; and ints Hq, Hkv, D.  k_cache, v_cache [Hkv][L][D] are
    updated in place at row P + row.  anc_rows: expansion rows of the node's
    ancestors and itself.  Returns (y bf16 [H], logits [V]).
    """
    Hq, Hkv, D = w["Hq"], w["Hkv"], w["D"]
    G = Hq // Hkv
    u = np.concatenate([np.asarray(f_in, dtype=np.float64), w["embed"][token]])
    x = w["fc"] @ u
    a = bf16_round(rms_norm(x, w["g1"], eps))
    q = bf16_round(w["q"] @ a).reshape(Hq, D)
    k_cache[:, P + row] = bf16_round(w["k"] @ a).reshape(Hkv, D)
    v_cache[:, P + row] = bf16_round(w["v"] @ a).reshape(Hkv, D)
    keys = list(range(P)) + [P + r for r in sorted(anc_rows)]
    att = np.zeros((Hq, D))
    for h in range(Hq):
        kk = k_cache[h // G, keys]
        vv = v_cache[h // G, keys]
        s = scale * (kk @ q[h])
        p = np.exp(s - s.max())
        att[h] = (p @ vv) / p.sum()
    hres = x + w["o"] @ bf16_round(att.reshape(-1))
    b2 = bf16_round(rms_norm(hres, w["g2"], eps))
    z = bf16_round(silu(w["gate"] @ b2) * (w["up"] @ b2))
    y = bf16_round(hres + w["down"] @ z)
    return y, w["lm"] @ y


def draft_expand(w, f0, root_token: int, k_prefix, v_prefix, P: int, top_k: int, depth: int,
                 n_nodes: int, scale: float, eps: float):
    """One sequence: grow the EAGLE-2 draft tree, running the head row by row.

    f0 [H] (bf16 values); k_prefix, v_prefix [Hkv][>=P][D] (bf16 values; rows
    0..P-1 are the draft cache's prefix).  Rows are numbered as in eagle2_rerank:
    0 = the root, 1 + (d-1)*top_k + j = frontier slot j at depth d.

    Returns (tree, logits [R][V], features y [R][H], parent_row [R], row_token [R])
    where tree is grow_tree's result.
    """
    R = 1 + (depth - 1) * top_k
    Hkv, D = w["Hkv"], w["D"]
    k_cache = np.zeros((Hkv, P + R, D))
    v_cache = np.zeros((Hkv, P + R, D))
    k_cache[:, :P] = np.asarray(k_prefix, dtype=np.float64)[:, :P]
    v_cache[:, :P] = np.asarray(v_prefix, dtype=np.float64)[:, :P]
    V, H = w["lm"].shape
    logits = np.zeros((R, V))
    feats = np.zeros((R, H))
    parent_row = np.full(R, -1, dtype=np.int64)
    row_token = np.zeros(R, dtype=np.int64)
    anc = {}

    def row_fn(r, token, prow):
        anc[r] = [r] + (anc[prow] if prow >= 0 else [])
        f_in = f0 if prow < 0 else feats[prow]
        y, lg = draft_layer_row(w, f_in, token, k_cache, v_cache, anc[r], r, P, scale, eps)
        feats[r], logits[r] = y, lg
        parent_row[r], row_token[r] = prow, token
        return lg

    tree = grow_tree(row_fn, root_token, top_k, depth, n_nodes)
    return tree, logits, feats, parent_row, row_token
