"""Pins of the ragged-batch oracle wrappers ([P3] section 4 and closing remarks).

Each sequence of a ragged batch must be the single-sequence problem on its own
prefix and tree: checked against PyTorch's scaled_dot_product_attention (fp64,
explicit mask) per sequence, against the uniform oracle when all sizes are equal,
and for invariance to whatever the padding holds.
"""
import numpy as np
import torch
import torch.nn.functional as F

import oracle


def _batch(rng, B, Nmax, Hq, Hkv, D, cap):
    q = rng.standard_normal((B, Nmax, Hq, D))
    k = rng.standard_normal((B, Hkv, cap, D))
    v = rng.standard_normal((B, Hkv, cap, D))
    par = np.full((B, Nmax), -1, dtype=np.int64)
    for b in range(B):
        for i in range(1, Nmax):
            par[b, i] = rng.integers(0, i)
    return q, k, v, par


def _sdpa_sequence(q, k, v, parents, P, scale):
    """One sequence via SDPA: q [N][Hq][D], k/v [Hkv][cap][D] -> out [N][Hq][D]."""
    N, Hq, D = q.shape
    G = Hq // k.shape[0]
    anc = np.eye(N, dtype=bool)
    for i in range(1, N):
        anc[i] |= anc[parents[i]]
    mask = np.zeros((N, P + N), dtype=bool)
    mask[:, :P] = True
    mask[:, P:] = anc
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(k[:, :P + N]).repeat_interleave(G, dim=0)
    vt = torch.from_numpy(v[:, :P + N]).repeat_interleave(G, dim=0)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask), scale=scale)
    return o.permute(1, 0, 2).numpy()


def test_each_sequence_is_plain_masked_attention():
    rng = np.random.default_rng(3)
    B, Nmax, Hq, Hkv, D, cap = 3, 12, 4, 2, 16, 60
    q, k, v, par = _batch(rng, B, Nmax, Hq, Hkv, D, cap)
    P = np.array([40, 7, 0])
    N = np.array([12, 5, 9])
    out, lse = oracle.tree_verify_attention_ragged(q, k, v, par, P, N, 0.25)
    for b in range(B):
        n, p = N[b], P[b]
        want = _sdpa_sequence(q[b, :n], k[b], v[b], par[b, :n], p, 0.25)
        np.testing.assert_allclose(out[b, :n], want, rtol=1e-10, atol=1e-12)
        assert np.isnan(out[b, n:]).all() and np.isnan(lse[b, n:]).all()
        assert np.isfinite(lse[b, :n]).all()


def test_equal_sizes_reduce_to_the_uniform_oracle():
    rng = np.random.default_rng(4)
    q, k, v, par = _batch(rng, 2, 8, 4, 1, 8, 30)
    out, lse = oracle.tree_verify_attention_ragged(q, k, v, par, [20, 20], [8, 8], 0.3)
    o2, l2 = oracle.tree_verify_attention(q, k, v, par, 20, 0.3)
    np.testing.assert_allclose(out, o2, rtol=1e-12)
    np.testing.assert_allclose(lse, l2, rtol=1e-12)


def test_padding_content_does_not_matter():
    rng = np.random.default_rng(5)
    q, k, v, par = _batch(rng, 2, 10, 2, 1, 8, 40)
    P, N = [25, 3], [6, 10]
    out, lse = oracle.tree_verify_attention_ragged(q, k, v, par, P, N, 0.5)
    q2, k2, v2, par2 = q.copy(), k.copy(), v.copy(), par.copy()
    q2[0, 6:] = 99.0
    par2[0, 6:] = 0
    k2[0, :, 25 + 6:] = -50.0          # rows past sequence 0's tree
    v2[1, :, 3 + 10:] = 7.0            # rows past sequence 1's tree
    out2, lse2 = oracle.tree_verify_attention_ragged(q2, k2, v2, par2, P, N, 0.5)
    np.testing.assert_array_equal(out[0, :6], out2[0, :6])
    np.testing.assert_array_equal(out[1], out2[1])


def test_acceptance_per_sequence_ignores_nodes_past_the_tree():
    # sequence 0: 4 nodes, chain 0-1-2-3 all matching; node 4 (padding) would extend it
    tokens = np.array([[5, 1, 2, 3, 4], [9, 7, 7, 0, 0]])
    parents = np.array([[-1, 0, 1, 2, 3], [-1, 0, 0, 0, 0]])
    amax = np.array([[1, 2, 3, 4, 8], [7, 1, 1, 1, 1]])
    res = oracle.accept_greedy_ragged(tokens, parents, amax, [4, 3], max_depth=6)
    assert res[0][0] == 3 and res[0][1] == [0, 1, 2, 3] and res[0][2] == [1, 2, 3, 4]
    assert res[1][0] == 1 and res[1][1] == [0, 1] and res[1][2] == [7, 1]
