"""Draft-tree bookkeeping for the oracle.

A tree of N nodes is a parent array: node 0 is the root (parent -1) and every
other node i has a parent p with 0 <= p < i.  [P2] (workflow figure paragraph)
describes the draft as a token tree grown by repeated draft passes; [P1]
(innovations list, item 2) turns the tree's paths into an attention mask, which
is the ancestor-or-self relation computed here.
"""
from __future__ import annotations

from typing import List, Set


def node_depths(parents) -> List[int]:
    """Depth of every node: the root has depth 0, a child one more than its parent."""
    parents = [int(p) for p in parents]
    d = [0] * len(parents)
    for i in range(1, len(parents)):
        d[i] = d[parents[i]] + 1
    return d


def ancestor_sets(parents) -> List[Set[int]]:
    """anc*(i): the nodes on the path from the root to i, i itself included."""
    parents = [int(p) for p in parents]
    out: List[Set[int]] = []
    for i in range(len(parents)):
        s = {i}
        if i > 0:
            s |= out[parents[i]]
        out.append(s)
    return out


def children_of(parents, v: int) -> List[int]:
    """Children of node v in ascending node index (sibling order)."""
    return [c for c in range(len(parents)) if int(parents[c]) == v]

