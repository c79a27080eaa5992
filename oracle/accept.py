"""Acceptance of a verified draft tree: greedy and multi-round speculative sampling.

Greedy ([P1] greedy decoding paragraph and the figure paragraph after it; [P2]
speculative sampling paragraph): starting at the first draft token, a draft token
is kept while it equals the target's top-1 at the position before it; the first
mismatch truncates.  On a tree this means: node i survives when every edge on its
root path matches; the deepest surviving node wins (lowest node index among equally
deep ones); alpha = its depth, and alpha + 1 tokens are emitted (the kept drafts
plus the target's top-1 at the winner).

Speculative sampling ([P1] stochastic verification paragraph; [P2] "multi-round
speculative sampling" section; [P3] section 2, speculative decoding basics).
Letters follow [P1]: q is the target distribution, p the draft distribution.  A
draft token t is accepted when a uniform number lies below min(1, q(t)/p(t));
otherwise the target is corrected to the normalised positive part of (q - p) and
the next candidate is tried against the corrected distribution; [P2] makes this
multi-round over a token tree.  The pseudo-code the [P2] section refers to did not
survive in the page text; the reading implemented here:
  * at the current node v, children are tried in ascending node index; all of them
    were drafted from the same draft distribution p_v (the draft row recorded for v);
  * an accepted child becomes the current node, with fresh q and p;
  * after every child of v is rejected, one token is drawn from the corrected
    distribution; at a node with no children (or at max_depth) one token is drawn
    from q_v itself.
Draws use inverse-CDF sampling with the caller's uniforms.
"""
from __future__ import annotations

import numpy as np

from .tree import children_of, node_depths


def _softmax64(logits):
    x = np.asarray(logits, dtype=np.float64)
    e = np.exp(x - x.max())
    return e / e.sum()


def _dist(logits, lse):
    """The distribution of a logit row: softmax in fp64, or, with the normaliser the
    caller recorded for the row (its log-sum-exp), exp(logit - lse) as given."""
    if lse is None:
        return _softmax64(logits)
    return np.exp(np.asarray(logits, dtype=np.float64) - float(lse))


def sample_inverse_cdf(dist, u: float) -> int:
    """Smallest x with sum_{y<=x} dist(y) > u * sum(dist); if rounding leaves none,
    the last x with dist(x) > 0."""
    dist = np.asarray(dist, dtype=np.float64)
    c = np.cumsum(dist)
    target = float(u) * c[-1]
    hit = np.nonzero(c > target)[0]
    if hit.size:
        return int(hit[0])
    nz = np.nonzero(dist > 0)[0]
    return int(nz[-1]) if nz.size else 0


def accept_greedy(tokens, parents, target_argmax, max_depth: int):
    """One sequence.  tokens, parents, target_argmax: [N] ints.

    Returns (alpha, path, out_tokens): path = node indices root..winner,
    out_tokens = tokens[path[1:]] + [target_argmax[winner]] (alpha + 1 tokens).
    Nodes deeper than max_depth are not candidates.
    """
    tokens = [int(t) for t in tokens]
    parents = [int(p) for p in parents]
    top1 = [int(a) for a in target_argmax]
    N = len(parents)
    depth = node_depths(parents)
    ok = [False] * N
    ok[0] = True
    for i in range(1, N):
        ok[i] = ok[parents[i]] and tokens[i] == top1[parents[i]]
    best = 0
    for i in range(1, N):
        if ok[i] and depth[i] <= max_depth and depth[i] > depth[best]:
            best = i
    path = [best]
    while path[-1] != 0:
        path.append(parents[path[-1]])
    path.reverse()
    out = [tokens[c] for c in path[1:]] + [top1[best]]
    return depth[best], path, out


def spec_node_round(q, p, child_tokens, u_accept):
    """Multi-round check of one node's children against target q and draft p.

    Returns (j, q_left, ratios): j is the position of the first accepted child
    (-1 if all were rejected), q_left the corrected target after the rejections,
    ratios the acceptance probabilities used for the children that were tried.
    """
    q_left = np.asarray(q, dtype=np.float64).copy()
    p = np.asarray(p, dtype=np.float64)
    ratios = []
    for j, t in enumerate(child_tokens):
        t = int(t)
        if p[t] > 0:
            ratio = min(1.0, q_left[t] / p[t])
        else:
            ratio = 1.0 if q_left[t] > 0 else 0.0
        ratios.append(ratio)
        if float(u_accept[j]) < ratio:
            return j, q_left, ratios
        resid = np.maximum(0.0, q_left - p)
        z = resid.sum()
        if z > 0:
            q_left = resid / z
    return -1, q_left, ratios


def spec_node_round_point_mass(q, child_tokens, u_accept):
    """The same multi-round check when the siblings are proposed deterministically
    (EAGLE-2's expansion keeps the draft's top-k tokens, [P3] section 2): the draft
    distribution behind child t is then the point mass at t, and the rule of
    spec_node_round with that p reads: accept t when u < q_left(t); on rejection
    max(0, q_left - point mass at t) is q_left with t set to zero, renormalised.
    Returns (j, q_left, ratios) like spec_node_round."""
    q_left = np.asarray(q, dtype=np.float64).copy()
    ratios = []
    for j, t in enumerate(child_tokens):
        t = int(t)
        p = np.zeros_like(q_left)
        p[t] = 1.0
        ratio = min(1.0, q_left[t] / p[t])
        ratios.append(ratio)
        if float(u_accept[j]) < ratio:
            return j, q_left, ratios
        resid = np.maximum(0.0, q_left - p)
        z = resid.sum()
        if z > 0:
            q_left = resid / z
    return -1, q_left, ratios


def accept_spec(tokens, parents, target_logits, draft_logits, draft_row, u_accept, u_sample,
                max_depth: int, trace: list | None = None, mode: str = "sampled",
                target_lse=None, draft_lse=None):
    """One sequence.

    tokens, parents, draft_row: [N] ints (draft_row[i] = row of draft_logits holding
    the draft distribution at node i, -1 if node i was never expanded);
    target_logits [N][V]; draft_logits [R][V]; u_accept, u_sample [N] uniforms
    (u_accept[c] is used when child c is tried, u_sample[v] when a token is drawn
    at node v).  Temperature 1: q = softmax(target_logits[v]), p = softmax(draft row).

    mode "sampled" applies the pages' rule with the draft distribution p of the node
    (siblings drawn from p); mode "point_mass" treats every sibling as proposed
    deterministically (spec_node_round_point_mass; draft_logits are not read, a node
    still needs draft_row >= 0 to have its children tried).

    target_lse [N] / draft_lse [R] (optional): the log-sum-exp recorded for each
    target / draft row ([P2] multi-round section: the draft keeps each sampled
    token's probability as it drafts; the target's come with its LM head).  When
    given, q = exp(target_logits[v] - target_lse[v]) and p likewise, used as they are.

    Returns (alpha, path, out_tokens) like accept_greedy.  If ``trace`` is a list,
    one (node, child_list, ratios, j) tuple per visited node is appended.
    """
    if mode not in ("sampled", "point_mass"):
        raise ValueError(f"unknown mode {mode!r}")
    parents = [int(x) for x in parents]
    depth = node_depths(parents)
    v = 0
    path = [0]
    while True:
        kids = children_of(parents, v) if depth[v] < max_depth else []
        q = _dist(target_logits[v], None if target_lse is None else target_lse[v])
        row = int(draft_row[v])
        if not kids or row < 0:
            if trace is not None:
                trace.append((v, [], [], -1))
            x = sample_inverse_cdf(q, u_sample[v])
            break
        if mode == "point_mass":
            j, q_left, ratios = spec_node_round_point_mass(q, [tokens[c] for c in kids],
                                                           [u_accept[c] for c in kids])
        else:
            p = _dist(draft_logits[row], None if draft_lse is None else draft_lse[row])
            j, q_left, ratios = spec_node_round(q, p, [tokens[c] for c in kids],
                                                [u_accept[c] for c in kids])
        if trace is not None:
            trace.append((v, kids, ratios, j))
        if j < 0:
            x = sample_inverse_cdf(q_left, u_sample[v])
            break
        v = kids[j]
        path.append(v)
    out = [int(tokens[c]) for c in path[1:]] + [int(x)]
    return len(path) - 1, path, out
