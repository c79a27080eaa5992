"""EAGLE-2 dynamic draft tree: expansion and reranking under a token budget.

[P3] section 2 ("EAGLE-2 core innovation: dynamic draft tree") scores draft nodes by
the draft's own confidence, grows the tree deep where it is confident and wide
where it is not, and greedily maximises the expected acceptance length within a
fixed draft-token budget; [P1] innovations list items 1 and 3 describe keeping the
top tokens per draft step and pruning to high-probability paths.

Plain reading implemented here (the pages give no algorithm text):
  * a node's value is its path probability, the product of draft probabilities
    along its root path, kept as a cumulative log-probability ("score"); the root
    has score 0.  Expected acceptance length of a tree = sum of its nodes' values,
    and values never grow down a path, so taking the top nodes by value gives an
    ancestor-closed, budget-optimal tree.  (Peak-probability confidence is the
    one-child special case.)
  * draft logits are given per expansion slot: row 0 belongs to the root; row
    1 + (d-1)*k + j to frontier slot j at depth d (d = 1 .. depth-1).
  * each expanded node proposes its row's k highest-logit tokens (ties: lower
    token id), with score = parent score + log-softmax of the token.
  * depth-1 candidates are the root's proposals; for each depth d < depth the
    frontier is the k best depth-d candidates, placed in slots 0..k-1 in that
    order, and each expands.
  * the tree is the root plus the n_nodes-1 best candidates overall.  "Best" sorts
    by score descending, then candidate id ascending, where ids number the
    candidates depth by depth, slot by slot, rank by rank.
  * output order: root, then selected candidates by ascending id (breadth first).
"""
from __future__ import annotations

import numpy as np


def _logsumexp(row):
    x = np.asarray(row, dtype=np.float64)
    m = x.max()
    return m + np.log(np.exp(x - m).sum())


def _topk_tokens(row, k: int):
    x = np.asarray(row, dtype=np.float64)
    order = sorted(range(x.size), key=lambda t: (-x[t], t)) if x.size <= 64 else None
    if order is None:
        # stable sort of -x keeps lower token ids first among equal logits
        order = np.argsort(-x, kind="stable")
    return [int(t) for t in order[:k]]


def grow_tree(row_fn, root_token: int, top_k: int, depth: int, n_nodes: int):
    """The expansion and selection above, with the rows produced on demand.

    row_fn(r, token, parent_row) returns the logits of row r at the moment the tree
    first needs them: r = 0 for the root (token = root_token, parent_row = -1), and
    r = 1 + (d-1)*top_k + j for frontier slot j at depth d, whose node carries
    `token` and was proposed by the node expanded in row `parent_row`.  A row is
    requested only after every row of the depths above it, so a draft model can
    compute it from its ancestors.  Returns what eagle2_rerank returns.
    """
    R = 1 + (depth - 1) * top_k
    lse = [0.0] * R
    props = [None] * R
    rows = {}

    def need(r, token, parent_row):
        x = np.asarray(row_fn(r, token, parent_row), dtype=np.float64)
        rows[r] = x
        lse[r] = _logsumexp(x)
        props[r] = _topk_tokens(x, top_k)

    # candidate records: id -> [depth, score, token, parent_id or -1 for root, row or -1]
    need(0, root_token, -1)
    cand = {}
    level = []
    for rank, t in enumerate(props[0]):
        cid = rank
        cand[cid] = [1, rows[0][t] - lse[0], t, -1, -1]
        level.append(cid)
    base = top_k
    for d in range(1, depth):
        frontier = sorted(level, key=lambda c: (-cand[c][1], c))[:top_k]
        level = []
        for j, fid in enumerate(frontier):
            row = 1 + (d - 1) * top_k + j
            cand[fid][4] = row
            par = cand[fid][3]
            need(row, cand[fid][2], 0 if par < 0 else cand[par][4])
            for rank, t in enumerate(props[row]):
                cid = base + j * top_k + rank
                cand[cid] = [d + 1, cand[fid][1] + (rows[row][t] - lse[row]), t, fid, -1]
                level.append(cid)
        base += top_k * top_k

    chosen = sorted(cand, key=lambda c: (-cand[c][1], c))[:n_nodes - 1]
    chosen.sort()
    pos = {cid: i + 1 for i, cid in enumerate(chosen)}
    N = n_nodes
    tokens = np.zeros(N, dtype=np.int64)
    parents = np.zeros(N, dtype=np.int64)
    depths = np.zeros(N, dtype=np.int64)
    scores = np.zeros(N, dtype=np.float64)
    draft_row = np.full(N, -1, dtype=np.int64)
    tokens[0], parents[0], depths[0], scores[0], draft_row[0] = root_token, -1, 0, 0.0, 0
    for cid in chosen:
        i = pos[cid]
        dd, sc, t, par, row = cand[cid]
        tokens[i] = t
        parents[i] = 0 if par < 0 else pos[par]
        depths[i] = dd
        scores[i] = sc
        draft_row[i] = row
    return {"tokens": tokens, "parents": parents, "depths": depths, "scores": scores,
            "draft_row": draft_row, "draft_lse": np.array(lse)}


def eagle2_rerank(draft_logits, root_token: int, top_k: int, depth: int, n_nodes: int):
    """One sequence.  draft_logits [R][V] with R = 1 + (depth-1)*top_k.

    Returns dict with tokens, parents, depths, scores (fp64), draft_row (row of the
    node's own expansion, -1 if it was not expanded; 0 for the root), draft_lse [R].
    """
    R = 1 + (depth - 1) * top_k
    logits = np.asarray(draft_logits, dtype=np.float64)
    assert logits.shape[0] == R
    return grow_tree(lambda r, token, parent_row: logits[r], root_token, top_k, depth, n_nodes)
