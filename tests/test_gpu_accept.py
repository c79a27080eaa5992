"""GPU parity: eagle_accept_greedy (bit-exact) and eagle_accept_spec (decisions
bit-exact for the same uniforms; the resampled token in distribution)."""
import json
import os

import numpy as np
import pytest
import torch
from scipy.stats import chi2

import oracle
import synth
from inputs import to_dev

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _greedy_gpu(lib, tokens, parents, top1, max_depth):
    a, p, o = lib.eagle_accept_greedy(to_dev(tokens), to_dev(parents), to_dev(top1), max_depth)
    torch.cuda.synchronize()
    return a.cpu().numpy(), p.cpu().numpy(), o.cpu().numpy()


def _padded(seq, cap):
    return list(seq) + [-1] * (cap - len(seq))


def test_greedy_worked_example(gpu_lib):
    g = json.load(open(os.path.join(GOLDEN, "greedy_worked_example.json")))
    a, p, o = _greedy_gpu(gpu_lib, np.array([g["tokens"]], np.int32),
                          np.array([g["parents"]], np.int32),
                          np.array([g["target_argmax"]], np.int32), g["max_depth"])
    cap = g["max_depth"] + 1
    assert a[0] == g["expect"]["alpha"]
    assert list(p[0]) == _padded(g["expect"]["path"], cap)
    assert list(o[0]) == _padded(g["expect"]["out_tokens"], cap)


@pytest.mark.parametrize("seed", range(4))
def test_greedy_random_trees(gpu_lib, seed):
    B, N, V = 97, int([5, 26, 60, 64][seed]), 7
    parents = synth.random_parents(B, N, seed, 500, 1)
    top1 = synth.integers((B, N), 0, V, seed, 500, 2)
    noise = synth.integers((B, N), 0, V, seed, 500, 3)
    u = synth.uniform_f32((B, N), seed, 500, 4)
    tokens = np.where(u < 0.7, np.take_along_axis(top1, np.maximum(parents, 0), 1), noise)
    tokens = tokens.astype(np.int32)
    max_depth = [2, 5, 8, 63][seed]
    a, p, o = _greedy_gpu(gpu_lib, tokens, parents, top1, max_depth)
    cap = max_depth + 1
    for b in range(B):
        alpha, path, out = oracle.accept_greedy(tokens[b], parents[b], top1[b], max_depth)
        assert a[b] == alpha and len(out) == alpha + 1
        assert list(p[b]) == _padded(path, cap)
        assert list(o[b]) == _padded(out, cap)


def _spec_gpu(lib, tokens, parents, draft_row, tl, dl, ua, us, max_depth, mode="sampled",
              tlse=None, dlse=None):
    a, p, o = lib.eagle_accept_spec(to_dev(tokens), to_dev(parents), to_dev(draft_row), to_dev(tl),
                                    to_dev(dl), to_dev(ua), to_dev(us), max_depth, mode=mode,
                                    target_lse=None if tlse is None else to_dev(tlse),
                                    draft_lse=None if dlse is None else to_dev(dlse))
    torch.cuda.synchronize()
    return a.cpu().numpy(), p.cpu().numpy(), o.cpu().numpy()


def _lse32(logits):
    """Row log-sum-exp of fp32 logits, computed on the CPU (scipy) and rounded to fp32:
    the normaliser a caller hands over (the LM head's out_lse is fp32)."""
    from scipy.special import logsumexp
    return logsumexp(np.asarray(logits, dtype=np.float64), axis=-1).astype(np.float32)


# (seed, B, N, V): the last two force vocabulary chunks of more than 4096 entries per
# workgroup (at most 256 workgroups in all: 64 sequences get 4 chunks of 5000, 16
# sequences at the Llama-3 vocabulary 16 chunks of 8016), the strided path
SPEC_CASES = [(0, 64, 8, 8), (1, 16, 20, 1000), (2, 4, 60, 5003), (3, 2, 64, 40000),
              (4, 64, 8, 20000), (5, 16, 8, 128256)]


def _spec_case(seed, B, N, V, R_per, k_sib, tl_std, dl_std, plant_p):
    """Trees whose internal nodes have their own draft row; sibling tokens drawn
    from the parent's draft distribution (a mix of i.i.d. draws and fixed tokens)."""
    parents = synth.random_parents(B, N, seed, 600, 1)
    tl = synth.normal_f32((B, N, V), tl_std, seed, 600, 2)
    dl = synth.normal_f32((B, R_per, V), dl_std, seed, 600, 3)
    ua = synth.uniform_f32((B, N), seed, 600, 4)
    us = synth.uniform_f32((B, N), seed, 600, 5)
    rowpick = synth.integers((B, N), 0, R_per, seed, 600, 6)
    draft_row = np.full((B, N), -1, np.int32)
    for b in range(B):
        internal = sorted(set(parents[b, 1:].tolist()))
        for v in internal:
            draft_row[b, v] = rowpick[b, v]
    # tokens: draft samples from the parent's draft row
    pu = synth.uniform_f32((B, N), seed, 600, 7)
    tokens = np.zeros((B, N), np.int32)
    for b in range(B):
        for i in range(1, N):
            row = dl[b, draft_row[b, parents[b, i]]].astype(np.float64)
            p = np.exp(row - row.max())
            p /= p.sum()
            tokens[b, i] = min(int(np.searchsorted(np.cumsum(p), pu[b, i] * p.sum(), side="right")), V - 1)
    return tokens, parents, draft_row, tl, dl, ua, us


@pytest.mark.parametrize("with_lse", [False, True])
@pytest.mark.parametrize("seed,B,N,V", SPEC_CASES)
def test_spec_decisions_match_oracle(gpu_lib, seed, B, N, V, with_lse):
    tokens, parents, draft_row, tl, dl, ua, us = _spec_case(seed, B, N, V, 5, 0, 1.0, 1.5, 0)
    tlse, dlse = (_lse32(tl), _lse32(dl)) if with_lse else (None, None)
    max_depth = 64
    print(f"spec parity seed={seed} B={B} N={N} V={V} lse={with_lse}", flush=True)
    a, p, o = _spec_gpu(gpu_lib, tokens, parents, draft_row, tl, dl, ua, us, max_depth,
                        tlse=tlse, dlse=dlse)
    cap = max_depth + 1
    near = 0
    tok_diff = 0
    for b in range(B):
        trace = []
        alpha, path, out = oracle.accept_spec(
            tokens[b], parents[b], tl[b], dl[b], draft_row[b], ua[b], us[b], max_depth, trace=trace,
            target_lse=None if tlse is None else tlse[b], draft_lse=None if dlse is None else dlse[b])
        margins = [abs(float(ua[b, kid]) - r) for (_, kids, ratios, _) in trace
                   for kid, r in zip(kids, ratios)]
        if margins and min(margins) <= 1e-6:
            near += 1
            continue
        assert a[b] == alpha
        assert list(p[b]) == _padded(path, cap)
        assert list(o[b, :alpha]) == out[:alpha]
        assert 0 <= o[b, alpha] < V
        tok_diff += int(o[b, alpha] != out[alpha])
    assert near <= max(1, B // 20)
    # the resampled token is compared in distribution (chi-square test below); with
    # fp64 arithmetic on both sides it also agrees here except next to a CDF boundary
    assert tok_diff <= max(1, B // 20)


def test_spec_chi_square_on_gpu(gpu_lib):
    """2e5 independent trials in one launch, V = 8, root with 3 children drawn i.i.d.
    from the draft: the first emitted token must follow q."""
    T, V, N = 200_000, 8, 4
    tlrow = synth.normal_f32((V,), 1.2, 0, 650, 1)
    dlrow = synth.normal_f32((V,), 2.0, 0, 650, 2)
    q = np.exp(tlrow - tlrow.max()); q /= q.sum()
    p = np.exp(dlrow - dlrow.max()); p /= p.sum()
    parents = np.tile(np.array([-1, 0, 0, 0], np.int32), (T, 1))
    draft_row = np.tile(np.array([0, -1, -1, -1], np.int32), (T, 1))
    pu = synth.uniform_f32((T, N), 0, 650, 3)
    tokens = np.minimum(np.searchsorted(np.cumsum(p), pu, side="right"), V - 1).astype(np.int32)
    tokens[:, 0] = 0
    tl = np.broadcast_to(tlrow, (T, N, V)).copy()
    dl = np.broadcast_to(dlrow, (T, 1, V)).copy()
    ua = synth.uniform_f32((T, N), 0, 650, 4)
    us = synth.uniform_f32((T, N), 0, 650, 5)
    a, path, o = _spec_gpu(gpu_lib, tokens, parents, draft_row, tl, dl, ua, us, 5)
    first = np.bincount(o[:, 0], minlength=V)[:V].astype(np.float64)
    stat = ((first - T * q) ** 2 / (T * q)).sum()
    assert chi2.sf(stat, V - 1) > 1e-3, (first / T, q)


def test_spec_full_c4_tree(gpu_lib):
    """C4 shapes: a 60-node tree from the oracle's rerank of the C4 draft logits; target
    logits N(0,1) over 128256 tokens, draft logits N(0,9): every root child is rejected
    (q is flat, p peaky), so this runs the 10 residual rounds."""
    cfg = synth.CONFIGS["C4"]
    V = cfg.V
    dl = synth.normal_f32((1, cfg.rows, V), cfg.draft_std, 0, cfg.index, 6)
    root = int(synth.integers((1,), 0, V, 0, cfg.index, 7)[0])
    tree = oracle.eagle2_rerank(dl[0], root, cfg.top_k, cfg.depth, cfg.N)
    tl = synth.normal_f32((1, cfg.N, V), 1.0, 0, cfg.index, 10)
    ua = synth.uniform_f32((1, cfg.N), 0, cfg.index, 8)
    us = synth.uniform_f32((1, cfg.N), 0, cfg.index, 9)
    toks = tree["tokens"][None].astype(np.int32)
    par = tree["parents"][None].astype(np.int32)
    drow = tree["draft_row"][None].astype(np.int32)
    for with_lse in (False, True):
        tlse, dlse = (_lse32(tl), _lse32(dl)) if with_lse else (None, None)
        a, p, o = _spec_gpu(gpu_lib, toks, par, drow, tl, dl, ua, us, cfg.max_depth, tlse=tlse,
                            dlse=dlse)
        trace = []
        alpha, path, out = oracle.accept_spec(
            toks[0], par[0], tl[0], dl[0], drow[0], ua[0], us[0], cfg.max_depth, trace=trace,
            target_lse=None if tlse is None else tlse[0], draft_lse=None if dlse is None else dlse[0])
        assert a[0] == alpha and list(p[0, :alpha + 1]) == path
        assert len(trace[0][2]) == 10 and trace[0][3] == -1       # ten rejections at the root
        assert 0 <= o[0, alpha] < V


@pytest.mark.parametrize("nk", [1, 2, 3])
def test_spec_vanishing_residual(gpu_lib, nk):
    """q = p, supported on one or two tokens, and every child's token outside that
    support: each child is rejected (ratio 0) and the residual max(0, q - c p) at the
    next c is exactly zero, so the draw falls back to q itself (the pages' rule keeps the
    corrected target when the residual has no mass)."""
    V, N = 16, nk + 1
    B = 4
    tl = np.zeros((B, N, V), np.float32)
    dl = np.zeros((B, 1, V), np.float32)
    support = [(5,), (2, 11), (0,), (7, 8)]
    for b, sup in enumerate(support):
        row = np.full(V, -1000.0, np.float32)   # exp(-1000) is 0 in fp64: exact zeros
        row[list(sup)] = 0.0
        tl[b, :] = row
        dl[b, 0] = row
    parents = np.tile(np.array([-1] + [0] * nk, np.int32), (B, 1))
    draft_row = np.tile(np.array([0] + [-1] * nk, np.int32), (B, 1))
    tokens = np.zeros((B, N), np.int32)
    for b, sup in enumerate(support):
        outside = [t for t in range(V) if t not in sup]
        tokens[b, 1:] = outside[:nk]
    ua = np.full((B, N), 0.5, np.float32)
    us = np.array([[0.3] * N, [0.25] * N, [0.9] * N, [0.75] * N], np.float32)
    print(f"spec vanishing residual nk={nk}", flush=True)
    a, p, o = _spec_gpu(gpu_lib, tokens, parents, draft_row, tl, dl, ua, us, 5)
    for b, sup in enumerate(support):
        alpha, path, out = oracle.accept_spec(tokens[b], parents[b], tl[b], dl[b], draft_row[b],
                                              ua[b], us[b], 5)
        expect = sup[0] if len(sup) == 1 or us[b, 0] < 0.5 else sup[1]
        assert alpha == 0 and path == [0] and out == [expect]
        assert a[b] == 0 and p[b, 0] == 0 and o[b, 0] == expect


# ---------------------------------------------------------------- deterministic siblings

@pytest.mark.parametrize("with_lse", [False, True])
@pytest.mark.parametrize("seed,B,N,V", SPEC_CASES)
def test_spec_point_mass_decisions_match_oracle(gpu_lib, seed, B, N, V, with_lse):
    """mode="point_mass": siblings are each node's top tokens of its draft row (ties and
    repeats included by taking some siblings twice); accept lengths, paths and accepted
    tokens bit-exact against the oracle's point-mass rule, with the same uniforms."""
    tokens, parents, draft_row, tl, dl, ua, us = _spec_case(seed, B, N, V, 5, 0, 1.0, 1.5, 0)
    rng = np.random.default_rng(900 + seed)
    for b in range(B):
        for v in range(N):
            kids = [c for c in range(1, N) if parents[b, c] == v]
            if not kids or draft_row[b, v] < 0:
                continue
            order = np.argsort(-dl[b, draft_row[b, v]], kind="stable")
            for j, c in enumerate(kids):
                tokens[b, c] = order[j % 3] if rng.random() < 0.2 else order[j]
    # plant acceptances: some uniforms small enough to accept a likely child (a child's
    # target probability is ~1/V, so the factor shrinks with the vocabulary)
    scale = 1e-3 if V < 50000 else 1e-7
    ua = np.where(rng.random(ua.shape) < 0.3, ua * scale, ua).astype(np.float32)
    max_depth = 64
    # point-mass mode reads no draft distribution: only the target normaliser matters
    tlse = _lse32(tl) if with_lse else None
    print(f"spec point-mass parity seed={seed} B={B} N={N} V={V} lse={with_lse}", flush=True)
    a, p, o = _spec_gpu(gpu_lib, tokens, parents, draft_row, tl, dl, ua, us, max_depth,
                        mode="point_mass", tlse=tlse)
    cap = max_depth + 1
    near = 0
    tok_diff = 0
    accepted_any = 0
    for b in range(B):
        trace = []
        alpha, path, out = oracle.accept_spec(tokens[b], parents[b], tl[b], dl[b], draft_row[b],
                                              ua[b], us[b], max_depth, trace=trace,
                                              mode="point_mass",
                                              target_lse=None if tlse is None else tlse[b])
        margins = [abs(float(ua[b, kid]) - r) for (_, kids, ratios, _) in trace
                   for kid, r in zip(kids, ratios)]
        if margins and min(margins) <= 1e-6:
            near += 1
            continue
        accepted_any += alpha > 0
        assert a[b] == alpha
        assert list(p[b]) == _padded(path, cap)
        assert list(o[b, :alpha]) == out[:alpha]
        assert 0 <= o[b, alpha] < V
        tok_diff += int(o[b, alpha] != out[alpha])
    # at V = 128256 some children's target probability is itself below the 1e-6 margin,
    # which makes their sequences "near" whatever the uniform
    assert near <= max(2, B // 8)
    assert tok_diff <= max(1, B // 20)
    assert accepted_any > 0 or B < 4   # tiny batches over large vocabularies may accept nothing


def test_spec_point_mass_chi_square_on_gpu(gpu_lib):
    """2e5 trials, V = 8, the root's three children fixed to the draft's top-3 (the
    same tokens in every trial): with the point-mass rule the first emitted token
    follows q; with the sampled rule it would not (see the oracle's contrast test)."""
    T, V, N = 200_000, 8, 4
    tlrow = synth.normal_f32((V,), 1.2, 0, 660, 1)
    dlrow = synth.normal_f32((V,), 2.0, 0, 660, 2)
    q = np.exp(tlrow.astype(np.float64) - tlrow.max())
    q /= q.sum()
    top3 = np.argsort(-dlrow, kind="stable")[:3].astype(np.int32)
    parents = np.tile(np.array([-1, 0, 0, 0], np.int32), (T, 1))
    draft_row = np.tile(np.array([0, -1, -1, -1], np.int32), (T, 1))
    tokens = np.tile(np.concatenate([[0], top3]).astype(np.int32), (T, 1))
    tl = np.broadcast_to(tlrow, (T, N, V)).copy()
    dl = np.broadcast_to(dlrow, (T, 1, V)).copy()
    ua = synth.uniform_f32((T, N), 0, 660, 4)
    us = synth.uniform_f32((T, N), 0, 660, 5)
    a, path, o = _spec_gpu(gpu_lib, tokens, parents, draft_row, tl, dl, ua, us, 5,
                           mode="point_mass")
    first = np.bincount(o[:, 0], minlength=V)[:V].astype(np.float64)
    stat = ((first - T * q) ** 2 / (T * q)).sum()
    assert chi2.sf(stat, V - 1) > 1e-3, (first / T, q)


def test_spec_point_mass_full_c4_tree(gpu_lib):
    """C4 shapes with the point-mass rule (the rule that is exact for EAGLE-2's top-k
    siblings): decisions against the oracle on the rerank tree."""
    cfg = synth.CONFIGS["C4"]
    V = cfg.V
    dl = synth.normal_f32((1, cfg.rows, V), cfg.draft_std, 0, cfg.index, 6)
    root = int(synth.integers((1,), 0, V, 0, cfg.index, 7)[0])
    tree = oracle.eagle2_rerank(dl[0], root, cfg.top_k, cfg.depth, cfg.N)
    tl = synth.normal_f32((1, cfg.N, V), 1.0, 0, cfg.index, 10)
    ua = synth.uniform_f32((1, cfg.N), 0, cfg.index, 8)
    us = synth.uniform_f32((1, cfg.N), 0, cfg.index, 9)
    toks = tree["tokens"][None].astype(np.int32)
    par = tree["parents"][None].astype(np.int32)
    drow = tree["draft_row"][None].astype(np.int32)
    a, p, o = _spec_gpu(gpu_lib, toks, par, drow, tl, dl, ua, us, cfg.max_depth, mode="point_mass")
    trace = []
    alpha, path, out = oracle.accept_spec(toks[0], par[0], tl[0], dl[0], drow[0], ua[0], us[0],
                                          cfg.max_depth, trace=trace, mode="point_mass")
    assert a[0] == alpha and list(p[0, :alpha + 1]) == path
    assert list(o[0, :alpha]) == out[:alpha]
    assert 0 <= o[0, alpha] < V
