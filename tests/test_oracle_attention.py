"""Pins for the oracle's tree-verify attention (CPU only).

Each check compares the oracle with something that is not the oracle: PyTorch's
scaled_dot_product_attention (fp64, explicit boolean mask) on special cases that
reduce to textbook attention, a mask built by transitive closure of the parent
adjacency matrix, and structural invariants (GQA head mapping, relabelling).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _rand_tree(rng, N):
    par = [-1] + [int(rng.integers(0, i)) for i in range(1, N)]
    return np.array(par)


def _closure_mask(parents):
    """Ancestor-or-self matrix via repeated squaring of (I + parent adjacency)."""
    N = len(parents)
    A = np.eye(N, dtype=np.int64)
    for i in range(1, N):
        A[i, parents[i]] = 1
    R = A.copy()
    for _ in range(int(np.ceil(np.log2(max(N, 2)))) + 1):
        R = np.minimum(R @ R, 1)
    return R.astype(bool)            # R[i, j]: j is an ancestor of i or j == i


def _sdpa_with_lse(q, k, v, mask, scale):
    """SDPA plus an extra zero key whose one-hot value reveals the denominator:
    the weight w on that key is 1 / (1 + sum exp(s)), so lse = log((1 - w) / w)."""
    Lk = k.shape[-2]
    D = k.shape[-1]
    k2 = torch.cat([k, torch.zeros_like(k[..., :1, :])], dim=-2)
    v2 = torch.cat([v, torch.zeros_like(v[..., :1, :])], dim=-2)
    v2 = torch.cat([v2, torch.zeros_like(v2[..., :1])], dim=-1)
    v2[..., Lk, D] = 1.0
    m2 = torch.cat([mask, torch.ones_like(mask[..., :1])], dim=-1)
    o = F.scaled_dot_product_attention(q, k2, v2, attn_mask=m2, scale=scale)
    w = o[..., D]
    out = o[..., :D] / (1.0 - w)[..., None]
    lse = torch.log((1.0 - w) / w)
    return out, lse


def _reference_tree(q, k, v, parents, P, scale):
    """q [N][Hq][D], k/v [Hkv][P+N][D] -> out [N][Hq][D], lse [N][Hq] via SDPA."""
    N, Hq, D = q.shape
    Hkv = k.shape[0]
    G = Hq // Hkv
    anc = _closure_mask(parents)
    mask = np.zeros((N, P + N), dtype=bool)
    mask[:, :P] = True
    mask[:, P:] = anc
    qt = torch.from_numpy(q).permute(1, 0, 2)                         # [Hq][N][D]
    kt = torch.from_numpy(k[:, :P + N]).repeat_interleave(G, dim=0)    # [Hq][L][D]
    vt = torch.from_numpy(v[:, :P + N]).repeat_interleave(G, dim=0)
    mt = torch.from_numpy(mask)[None].expand(Hq, N, P + N)
    out, lse = _sdpa_with_lse(qt, kt, vt, mt, scale)
    return out.permute(1, 0, 2).numpy(), lse.permute(1, 0).numpy()


@pytest.mark.parametrize("P,N,Hq,Hkv,D", [(7, 9, 4, 2, 16), (0, 6, 2, 1, 8), (33, 1, 3, 3, 8),
                                           (5, 12, 8, 2, 4)])
def test_chain_equals_causal_attention(P, N, Hq, Hkv, D):
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, N, Hq, D))
    k = rng.standard_normal((1, Hkv, P + N, D))
    v = rng.standard_normal((1, Hkv, P + N, D))
    parents = np.array([[-1] + list(range(N - 1))])
    scale = D ** -0.5
    out, lse = oracle.tree_verify_attention(q, k, v, parents, P, scale)
    # textbook causal attention over the whole sequence; take the last N queries
    G = Hq // Hkv
    L = P + N
    full_q = torch.zeros(Hq, L, D, dtype=torch.float64)
    full_q[:, P:] = torch.from_numpy(q[0]).permute(1, 0, 2)
    causal = torch.ones(L, L, dtype=torch.bool).tril()
    kk = torch.from_numpy(k[0]).repeat_interleave(G, dim=0)
    vv = torch.from_numpy(v[0]).repeat_interleave(G, dim=0)
    ref, ref_lse = _sdpa_with_lse(full_q, kk, vv, causal.expand(Hq, L, L), scale)
    np.testing.assert_allclose(out[0], ref[:, P:].permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse[0], ref_lse[:, P:].permute(1, 0).numpy(), rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("seed", range(6))
def test_random_tree_matches_masked_sdpa(seed):
    rng = np.random.default_rng(100 + seed)
    N = int(rng.integers(1, 40))
    P = int(rng.integers(0, 50))
    Hkv = int(rng.integers(1, 4))
    G = int(rng.integers(1, 4))
    D = int(rng.choice([4, 8, 16]))
    q = rng.standard_normal((2, N, Hkv * G, D))
    k = rng.standard_normal((2, Hkv, P + N + 3, D))      # 3 unused capacity rows
    v = rng.standard_normal((2, Hkv, P + N + 3, D))
    parents = np.stack([_rand_tree(rng, N), _rand_tree(rng, N)])
    scale = 0.37
    out, lse = oracle.tree_verify_attention(q, k, v, parents, P, scale)
    for b in range(2):
        ro, rl = _reference_tree(q[b], k[b], v[b], parents[b], P, scale)
        np.testing.assert_allclose(out[b], ro, rtol=1e-9, atol=1e-11)
        np.testing.assert_allclose(lse[b], rl, rtol=1e-9, atol=1e-9)


def test_single_node_is_decode_attention():
    rng = np.random.default_rng(7)
    P, Hq, Hkv, D = 40, 4, 1, 8
    q = rng.standard_normal((1, 1, Hq, D))
    k = rng.standard_normal((1, Hkv, P + 1, D))
    v = rng.standard_normal((1, Hkv, P + 1, D))
    out, _ = oracle.tree_verify_attention(q, k, v, np.array([[-1]]), P, 0.5)
    ref = F.scaled_dot_product_attention(torch.from_numpy(q[0]).permute(1, 0, 2),
                                         torch.from_numpy(k[0]).expand(Hq, P + 1, D),
                                         torch.from_numpy(v[0]).expand(Hq, P + 1, D), scale=0.5)
    np.testing.assert_allclose(out[0, 0], ref[:, 0].numpy(), rtol=1e-10, atol=1e-12)


def test_gqa_equals_repeated_kv_heads():
    rng = np.random.default_rng(3)
    N, P, Hkv, G, D = 11, 9, 3, 4, 8
    q = rng.standard_normal((1, N, Hkv * G, D))
    k = rng.standard_normal((1, Hkv, P + N, D))
    v = rng.standard_normal((1, Hkv, P + N, D))
    parents = _rand_tree(rng, N)[None]
    a, la = oracle.tree_verify_attention(q, k, v, parents, P, 0.3)
    b, lb = oracle.tree_verify_attention(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1),
                                         parents, P, 0.3)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(la, lb, rtol=1e-12)


def test_topological_relabel_permutes_outputs():
    rng = np.random.default_rng(5)
    N, P, Hq, D = 14, 6, 2, 8
    parents = _rand_tree(rng, N)
    q = rng.standard_normal((1, N, Hq, D))
    k = rng.standard_normal((1, 1, P + N, D))
    v = rng.standard_normal((1, 1, P + N, D))
    out, lse = oracle.tree_verify_attention(q, k, v, parents[None], P, 0.4)
    # a random topological order: repeatedly take an available node at random
    depth = oracle.node_depths(parents)
    order = sorted(range(N), key=lambda i: (depth[i], rng.random()))
    new_of = {old: new for new, old in enumerate(order)}
    parents2 = np.array([-1 if order[n] == 0 else new_of[parents[order[n]]] for n in range(N)])
    q2 = q[:, order]
    k2 = k.copy()
    v2 = v.copy()
    k2[:, :, P:] = k[:, :, P + np.array(order)]
    v2[:, :, P:] = v[:, :, P + np.array(order)]
    out2, lse2 = oracle.tree_verify_attention(q2, k2, v2, parents2[None], P, 0.4)
    np.testing.assert_allclose(out2, out[:, order], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse2, lse[:, order], rtol=1e-12)


def test_tree_helpers_match_three_pass_example():
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tree_three_passes.json")))
    d = oracle.node_depths(g["parents"])
    assert len(d) == g["expect"]["n_nodes"]
    assert max(d) + 1 == g["expect"]["levels"]
    assert [d.count(x) for x in range(max(d) + 1)] == g["expect"]["nodes_per_depth"]
    anc = oracle.ancestor_sets(g["parents"])
    assert (_closure_mask(g["parents"]) == np.array([[j in anc[i] for j in range(10)]
                                                      for i in range(10)])).all()
