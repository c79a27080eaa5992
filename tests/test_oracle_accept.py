"""Pins for the oracle's greedy and speculative acceptance (CPU only)."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from oracle.accept import spec_node_round

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_tree(rng, N):
    return np.array([-1] + [int(rng.integers(0, i)) for i in range(1, N)])


# ---------------------------------------------------------------- greedy

def test_greedy_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "greedy_worked_example.json")))
    alpha, path, out = oracle.accept_greedy(g["tokens"], g["parents"], g["target_argmax"],
                                            g["max_depth"])
    assert alpha == g["expect"]["alpha"]
    assert path == g["expect"]["path"]
    assert out == g["expect"]["out_tokens"]
    assert len(out) == alpha + 1


@pytest.mark.parametrize("seed", range(20))
def test_greedy_chain_counts_leading_matches(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 12))
    top1 = rng.integers(0, 5, size=N)
    tokens = rng.integers(0, 5, size=N)
    parents = np.array([-1] + list(range(N - 1)))
    lead = 0
    while lead + 1 < N and tokens[lead + 1] == top1[lead]:
        lead += 1
    alpha, path, out = oracle.accept_greedy(tokens, parents, top1, max_depth=64)
    assert alpha == lead
    assert path == list(range(lead + 1))
    assert out == list(tokens[1:lead + 1]) + [top1[lead]]


def test_greedy_all_and_none():
    rng = np.random.default_rng(9)
    parents = _rand_tree(rng, 30)
    top1 = rng.integers(0, 100, size=30)
    depth = oracle.node_depths(parents)
    tokens = np.array([7] + [top1[parents[i]] for i in range(1, 30)])
    alpha, path, out = oracle.accept_greedy(tokens, parents, top1, 64)
    assert alpha == max(depth)
    assert path[-1] == min(i for i in range(30) if depth[i] == max(depth))
    tokens_none = np.array([7] + [top1[parents[i]] + 1 for i in range(1, 30)])
    alpha, path, out = oracle.accept_greedy(tokens_none, parents, top1, 64)
    assert alpha == 0 and path == [0] and out == [top1[0]]


@pytest.mark.parametrize("seed", range(30))
def test_greedy_brute_force_paths(seed):
    """Enumerate every root path; keep those whose drafts all equal the parent's top-1."""
    rng = np.random.default_rng(1000 + seed)
    N = int(rng.integers(1, 16))
    parents = _rand_tree(rng, N)
    top1 = rng.integers(0, 3, size=N)
    tokens = rng.integers(0, 3, size=N)
    max_depth = int(rng.integers(0, 6))
    best = None
    for node in range(N):
        path = [node]
        while path[-1] != 0:
            path.append(int(parents[path[-1]]))
        path.reverse()
        if len(path) - 1 > max_depth:
            continue
        if all(tokens[path[e + 1]] == top1[path[e]] for e in range(len(path) - 1)):
            key = (len(path), -node)
            if best is None or key > best[0]:
                best = (key, path)
    alpha, path, out = oracle.accept_greedy(tokens, parents, top1, max_depth)
    assert path == best[1]
    assert alpha == len(best[1]) - 1
    assert out == [tokens[c] for c in path[1:]] + [top1[path[-1]]]


def test_greedy_speculative_loop_reproduces_autoregressive_greedy():
    """Toy bigram target + noisy bigram draft.  Drafting a tree with the EAGLE-2
    rerank, verifying it with the target's top-1 and accepting greedily must emit
    exactly the target's own greedy sequence ([P3] section 3: identical outputs)."""
    rng = np.random.default_rng(11)
    V = 12
    target = rng.standard_normal((V, V)) * 2           # logits of next token given token
    draft = target + rng.standard_normal((V, V)) * 0.5
    k, depth, n_nodes = 3, 3, 10
    # reference: plain greedy decoding with the target
    seq = [0]
    for _ in range(40):
        seq.append(int(np.argmax(target[seq[-1]])))
    out = [0]
    passes = 0
    while len(out) < 41:
        passes += 1
        root = out[-1]
        # draft rows are keyed by expansion slot: regenerate them for the actual
        # tokens by running the rerank level by level
        tree = _draft_tree(draft, root, k, depth, n_nodes)
        top1 = np.array([int(np.argmax(target[t])) for t in tree["tokens"]])
        alpha, path, emitted = oracle.accept_greedy(tree["tokens"], tree["parents"], top1, depth)
        assert len(emitted) == alpha + 1
        out.extend(emitted)
    assert out[:41] == seq
    assert passes < 40                                  # some drafts were accepted


def _draft_tree(draft, root, k, depth, n_nodes):
    """Fill the slot-keyed draft rows the way a real draft model would (row of slot
    j at depth d = the draft's distribution after that frontier node's token), then
    build the tree with the oracle's rerank."""
    V = draft.shape[0]
    R = 1 + (depth - 1) * k
    rows = np.zeros((R, V))
    rows[0] = draft[root]
    lsm = draft - np.log(np.exp(draft).sum(1, keepdims=True))
    frontier = sorted([((t,), lsm[root, t]) for t in range(V)], key=lambda c: (-c[1], c[0]))[:k]
    for d in range(1, depth):
        for j, (path, sc) in enumerate(frontier):
            rows[1 + (d - 1) * k + j] = draft[path[-1]]
        nxt = []
        for j, (path, sc) in enumerate(frontier):
            props = sorted(range(V), key=lambda t: (-draft[path[-1], t], t))[:k]
            nxt += [(path + (t,), sc + lsm[path[-1], t]) for t in props]
        frontier = sorted(nxt, key=lambda c: -c[1])[:k]
    return oracle.eagle2_rerank(rows, root, k, depth, n_nodes)


# ---------------------------------------------------------------- speculative sampling

def _rand_dist(rng, V, peaky=1.0):
    x = rng.standard_normal(V) * peaky
    e = np.exp(x - x.max())
    return e / e.sum()


@pytest.mark.parametrize("k", [1, 2, 3])
@pytest.mark.parametrize("seed", range(4))
def test_spec_exact_enumeration_preserves_target(k, seed):
    """Siblings drawn i.i.d. from p: summing over every sibling tuple, the first
    emitted token is distributed exactly as q ([P1] stochastic verification;
    [P2] multi-round speculative sampling keeps the target distribution)."""
    rng = np.random.default_rng(seed)
    V = 8
    q = _rand_dist(rng, V, 1.5)
    p = _rand_dist(rng, V, 2.0)
    law = np.zeros(V)
    for tup in itertools.product(range(V), repeat=k):
        w = np.prod([p[t] for t in tup])
        j, q_left, ratios = spec_node_round(q, p, tup, [1.0] * k)   # u = 1 rejects every child
        assert j == -1 and len(ratios) == k
        reach = 1.0
        for t, r in zip(tup, ratios):
            law[t] += w * reach * r
            reach *= 1.0 - r
        law += w * reach * q_left
    np.testing.assert_allclose(law, q, rtol=0, atol=1e-12)


def test_spec_single_draft_acceptance_rate_is_one_minus_tv():
    rng = np.random.default_rng(4)
    V = 8
    q = _rand_dist(rng, V)
    p = _rand_dist(rng, V, 2.0)
    acc = 0.0
    for t in range(V):
        _, _, ratios = spec_node_round(q, p, [t], [1.0])
        acc += p[t] * ratios[0]
    np.testing.assert_allclose(acc, 1.0 - 0.5 * np.abs(p - q).sum(), atol=1e-14)


def test_spec_equal_distributions_accept_first_child():
    rng = np.random.default_rng(5)
    V = 8
    logits = rng.standard_normal(V)
    parents = [-1, 0, 0, 0]
    tokens = [0, 3, 5, 1]
    u = rng.random(4) * 0.999999
    alpha, path, out = oracle.accept_spec(tokens, parents, np.tile(logits, (4, 1)), logits[None],
                                          [0, -1, -1, -1], u, u, max_depth=5)
    assert path == [0, 1] and out[0] == 3 and alpha == 1 and len(out) == 2


def test_spec_one_hot_target_always_emits_its_token():
    rng = np.random.default_rng(6)
    V = 8
    tl = np.full((4, V), -1e4)
    tl[:, 6] = 0.0                      # q is (numerically) a point mass at token 6
    draft = rng.standard_normal((1, V))
    for trial in range(200):
        tokens = [0] + list(rng.integers(0, V, size=3))
        u = rng.random(4)
        alpha, path, out = oracle.accept_spec(tokens, [-1, 0, 0, 0], tl, draft, [0, -1, -1, -1],
                                              u, u, max_depth=5)
        assert out[0] == 6


def _chi2_sf(stat, dof):
    from scipy.stats import chi2
    return chi2.sf(stat, dof)


def test_spec_monte_carlo_chi_square_two_levels():
    """Black-box Monte Carlo: V = 8, root with 3 children, each with 2 children,
    sibling tokens drawn i.i.d. from their parent's draft distribution.  The first
    emitted token must follow q_root; given child c accepted first, the next token
    must follow q_c."""
    rng = np.random.default_rng(12345)
    V = 8
    parents = [-1, 0, 0, 0, 1, 1, 2, 2, 3, 3]
    N = len(parents)
    tl = rng.standard_normal((N, V)) * 1.2
    dl = rng.standard_normal((4, V)) * 2.0            # rows: root, children 1..3
    draft_row = [0, 1, 2, 3, -1, -1, -1, -1, -1, -1]
    pd = np.exp(dl - dl.max(1, keepdims=True))
    pd /= pd.sum(1, keepdims=True)
    qd = np.exp(tl - tl.max(1, keepdims=True))
    qd /= qd.sum(1, keepdims=True)
    T = 200_000
    first = np.zeros(V)
    second = {c: np.zeros(V) for c in (1, 2, 3)}
    cdf = np.cumsum(pd, axis=1)
    for _ in range(T):
        tokens = [0] * N
        for i in range(1, N):
            r = draft_row[parents[i]]
            tokens[i] = min(int(np.searchsorted(cdf[r], rng.random(), side="right")), V - 1)
        ua = rng.random(N)
        us = rng.random(N)
        alpha, path, out = oracle.accept_spec(tokens, parents, tl, dl, draft_row, ua, us, 5)
        first[out[0]] += 1
        if alpha >= 1:
            second[path[1]][out[1]] += 1
    stat = ((first - T * qd[0]) ** 2 / (T * qd[0])).sum()
    assert _chi2_sf(stat, V - 1) > 1e-3
    for c in (1, 2, 3):
        n = second[c].sum()
        assert n > 1000
        stat = ((second[c] - n * qd[c]) ** 2 / (n * qd[c])).sum()
        assert _chi2_sf(stat, V - 1) > 1e-3


def test_sample_inverse_cdf_edges():
    d = np.array([0.0, 0.25, 0.0, 0.75, 0.0])
    assert oracle.sample_inverse_cdf(d, 0.0) == 1
    assert oracle.sample_inverse_cdf(d, 0.2499) == 1
    assert oracle.sample_inverse_cdf(d, 0.25) == 3
    assert oracle.sample_inverse_cdf(d, 0.9999999) == 3
    assert oracle.sample_inverse_cdf(d, 1.0) == 3      # overshoot: last nonzero entry


# ---------------------------------------------------------------- deterministic siblings

@pytest.mark.parametrize("k", [1, 2, 3, 4])
@pytest.mark.parametrize("seed", range(3))
def test_spec_point_mass_exact_for_every_fixed_sibling_set(k, seed):
    """Deterministic siblings ([P3] section 2: the expansion keeps the draft's top-k):
    for EVERY fixed tuple of sibling tokens, duplicates included, the first emitted token
    of the point-mass rule is distributed exactly as q (sum over the accept/reject
    branches of the node's rounds)."""
    rng = np.random.default_rng(100 + seed)
    V = 8
    q = _rand_dist(rng, V, 1.5)
    for tup in itertools.product(range(V), repeat=k):
        j, q_left, ratios = oracle.spec_node_round_point_mass(q, tup, [1.0] * k)
        assert j == -1 and len(ratios) == k
        law = np.zeros(V)
        reach = 1.0
        for t, r in zip(tup, ratios):
            law[t] += reach * r
            reach *= 1.0 - r
        law += reach * q_left
        np.testing.assert_allclose(law, q, rtol=0, atol=1e-12)


def test_spec_point_mass_closed_form():
    """Distinct siblings t1, t2, t3: ratio_j = q(t_j) / (1 - q(t_1) - ... - q(t_{j-1})),
    and the residual after all three is q without them, renormalised."""
    rng = np.random.default_rng(7)
    q = _rand_dist(rng, 8, 1.0)
    tup = (5, 2, 6)
    _, q_left, ratios = oracle.spec_node_round_point_mass(q, tup, [1.0] * 3)
    np.testing.assert_allclose(ratios, [q[5], q[2] / (1 - q[5]), q[6] / (1 - q[5] - q[2])],
                               rtol=1e-13)
    want = q.copy()
    want[list(tup)] = 0.0
    np.testing.assert_allclose(q_left, want / want.sum(), rtol=1e-13)


def test_spec_sampled_rule_is_not_exact_for_fixed_siblings():
    """Why the point-mass mode exists: with the siblings fixed to the draft's top-2
    (not drawn from p), the pages' rule with p itself does not reproduce q."""
    rng = np.random.default_rng(3)
    V = 8
    q = _rand_dist(rng, V, 1.5)
    p = _rand_dist(rng, V, 2.0)
    tup = tuple(int(t) for t in np.argsort(-p)[:2])
    _, q_left, ratios = oracle.spec_node_round(q, p, tup, [1.0] * 2)
    law = np.zeros(V)
    reach = 1.0
    for t, r in zip(tup, ratios):
        law[t] += reach * r
        reach *= 1.0 - r
    law += reach * q_left
    assert np.abs(law - q).max() > 1e-3


def test_spec_point_mass_monte_carlo_through_accept_spec():
    """accept_spec(mode="point_mass") on a depth-2 tree whose siblings are the draft's
    top-3 at each level: the first and second emitted tokens follow q (chi-square, 7 d.o.f.)."""
    rng = np.random.default_rng(11)
    V, T = 8, 20000
    tl0 = rng.standard_normal(V) * 1.2
    tl1 = rng.standard_normal(V) * 1.2
    dl = rng.standard_normal((2, V)) * 2.0
    q0 = np.exp(tl0 - tl0.max()); q0 /= q0.sum()
    top0 = [int(t) for t in np.argsort(-dl[0])[:3]]
    top1 = [int(t) for t in np.argsort(-dl[1])[:3]]
    # node 1 (first child, token top0[0]) is expanded with top1; nodes 2, 3 are leaves
    parents = [-1, 0, 0, 0, 1, 1, 1]
    tokens = [0] + top0 + top1
    draft_row = [0, 1, -1, -1, -1, -1, -1]
    target = np.stack([tl0, tl1, tl0, tl0, tl0, tl0, tl0])
    first = np.zeros(V)
    second = np.zeros(V)
    n_second = 0
    u = rng.random((T, 2, 7))
    for n in range(T):
        alpha, path, out = oracle.accept_spec(tokens, parents, target, dl, draft_row, u[n, 0],
                                              u[n, 1], 5, mode="point_mass")
        first[out[0]] += 1
        if alpha >= 1 and path[1] == 1:
            second[out[1]] += 1
            n_second += 1
    from scipy.stats import chi2
    stat = ((first - T * q0) ** 2 / (T * q0)).sum()
    assert chi2.sf(stat, V - 1) > 1e-3
    q1 = np.exp(tl1 - tl1.max()); q1 /= q1.sum()
    stat2 = ((second - n_second * q1) ** 2 / (n_second * q1)).sum()
    assert chi2.sf(stat2, V - 1) > 1e-3


@pytest.mark.parametrize("mode", ["sampled", "point_mass"])
def test_spec_given_normalisers_reduce_to_softmax(mode):
    """accept_spec with the rows' log-sum-exp supplied (scipy's logsumexp) takes the same
    decisions, with the same acceptance ratios to rounding, and emits the same tokens as
    with the normalisers formed from the logits: q = exp(l - lse) is softmax(l)."""
    from scipy.special import logsumexp
    rng = np.random.default_rng(21)
    V = 50
    for trial in range(40):
        N = int(rng.integers(2, 12))
        parents = _rand_tree(rng, N)
        tl = rng.standard_normal((N, V)) * 1.5
        dl = rng.standard_normal((N, V)) * 2.5
        draft_row = np.where(rng.random(N) < 0.8, np.arange(N), -1)
        tokens = rng.integers(0, V, size=N)
        ua, us = rng.random(N), rng.random(N)
        t0, t1 = [], []
        a = oracle.accept_spec(tokens, parents, tl, dl, draft_row, ua, us, 4, trace=t0, mode=mode)
        b = oracle.accept_spec(tokens, parents, tl, dl, draft_row, ua, us, 4, trace=t1, mode=mode,
                               target_lse=logsumexp(tl, axis=1), draft_lse=logsumexp(dl, axis=1))
        assert a == b
        assert [(v, k, j) for v, k, _, j in t0] == [(v, k, j) for v, k, _, j in t1]
        for (_, _, r0, _), (_, _, r1, _) in zip(t0, t1):
            np.testing.assert_allclose(r1, r0, rtol=1e-12, atol=1e-15)
