"""Pins for the oracle's EAGLE-2 rerank (CPU only)."""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _paths(tree):
    """Token path (root excluded) of every node."""
    toks, par = tree["tokens"], tree["parents"]
    out = []
    for i in range(len(toks)):
        p, n = [], i
        while n != 0:
            p.append(int(toks[n]))
            n = int(par[n])
        out.append(tuple(reversed(p)))
    return out


@pytest.mark.parametrize("seed", range(5))
def test_depth_one_is_topk_of_root_log_softmax(seed):
    rng = np.random.default_rng(seed)
    V, k = 300, 12
    logits = rng.standard_normal((1, V)) * 3
    n_nodes = int(rng.integers(2, k + 2))
    t = oracle.eagle2_rerank(logits, 5, k, 1, n_nodes)
    ls = torch.log_softmax(torch.from_numpy(logits[0]), 0)
    top = torch.topk(ls, n_nodes - 1)
    assert list(t["tokens"][1:]) == top.indices.tolist()
    np.testing.assert_allclose(t["scores"][1:], top.values.numpy(), rtol=1e-12)
    assert list(t["parents"]) == [-1] + [0] * (n_nodes - 1)
    assert t["tokens"][0] == 5 and t["draft_row"][0] == 0


@pytest.mark.parametrize("seed", range(8))
def test_depth_two_full_width_is_global_topn_of_path_probabilities(seed):
    """k = V and depth 2: every depth-1 node is expanded and depth-2 nodes are leaves,
    so the tree must be the n-1 most probable paths among all V + V^2 paths."""
    rng = np.random.default_rng(50 + seed)
    V = 5
    k = V
    logits = rng.standard_normal((1 + k, V)) * 2
    n_nodes = int(rng.integers(2, 1 + V + V * V + 1))
    t = oracle.eagle2_rerank(logits, 0, k, 2, n_nodes)
    ls = torch.log_softmax(torch.from_numpy(logits), 1).numpy()
    # slot of a depth-1 token = its rank by root log-prob
    order1 = sorted(range(V), key=lambda x: -ls[0, x])
    slot = {tok: j for j, tok in enumerate(order1)}
    allp = {(a,): ls[0, a] for a in range(V)}
    for a, b in itertools.product(range(V), repeat=2):
        allp[(a, b)] = ls[0, a] + ls[1 + slot[a], b]
    best = sorted(allp, key=lambda pth: -allp[pth])[:n_nodes - 1]
    got = _paths(t)[1:]
    assert set(got) == set(best)
    for i, pth in enumerate(got):
        np.testing.assert_allclose(t["scores"][i + 1], allp[pth], rtol=1e-12)


def test_k3_m2_gives_nine_paths():
    g = json.load(open(os.path.join(GOLDEN, "tree_k3_m2.json")))
    rng = np.random.default_rng(3)
    k, depth, V = g["top_k"], g["depth"], g["vocab"]
    logits = rng.standard_normal((1 + (depth - 1) * k, V))
    t = oracle.eagle2_rerank(logits, 1, k, depth, g["n_nodes"])
    d = list(t["depths"])
    assert [d.count(x) for x in range(depth + 1)] == g["expect"]["nodes_per_depth"]
    leaves = [i for i in range(len(d)) if i not in set(t["parents"][1:])]
    assert len(leaves) == g["expect"]["leaves"]


@pytest.mark.parametrize("seed", range(6))
def test_invariants_on_deep_trees(seed):
    rng = np.random.default_rng(200 + seed)
    V, k, depth = 40, 4, 5
    R = 1 + (depth - 1) * k
    logits = rng.standard_normal((R, V)) * 3
    n_nodes = int(rng.integers(2, 40))
    t = oracle.eagle2_rerank(logits, 7, k, depth, n_nodes)
    par, tok, dep, sc, row = t["parents"], t["tokens"], t["depths"], t["scores"], t["draft_row"]
    N = len(par)
    assert N == n_nodes and par[0] == -1
    ls = torch.log_softmax(torch.from_numpy(logits), 1).numpy()
    for i in range(1, N):
        assert 0 <= par[i] < i                                   # ancestor-closed, BFS-ish order
        assert dep[i] == dep[par[i]] + 1
        assert dep[i] >= dep[i - 1]                              # breadth first
        r = row[par[i]]
        assert r >= 0                                            # a parent was expanded
        np.testing.assert_allclose(sc[i], sc[par[i]] + ls[r, tok[i]], rtol=1e-12, atol=1e-12)
        assert sc[i] <= sc[par[i]]
    # siblings are their row's best tokens, in rank order, with no gaps
    unselected_best = -np.inf
    for v in range(N):
        kids = [c for c in range(N) if par[c] == v]
        if row[v] < 0:
            assert not kids
            continue
        ranked = sorted(range(V), key=lambda x: (-logits[row[v], x], x))
        assert [int(tok[c]) for c in kids] == ranked[:len(kids)]
        if len(kids) < k:
            unselected_best = max(unselected_best, sc[v] + ls[row[v], ranked[len(kids)]])
    assert sc[1:].min() >= unselected_best - 1e-12
    # frontier rows are handed out in score order within each depth
    for d in range(1, depth):
        exp_nodes = [i for i in range(N) if dep[i] == d and row[i] >= 0]
        by_row = sorted(exp_nodes, key=lambda i: row[i])
        assert [sc[i] for i in by_row] == sorted([sc[i] for i in by_row], reverse=True)
        for i in exp_nodes:
            assert 1 + (d - 1) * k <= row[i] < 1 + d * k
    np.testing.assert_allclose(t["draft_lse"], torch.logsumexp(torch.from_numpy(logits), 1).numpy(),
                               rtol=1e-12)
