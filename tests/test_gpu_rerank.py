"""GPU parity: eagle2_rerank against the fp64 oracle.

Tree indices (tokens, parents, depths, draft rows) are bit-exact whenever every
selection cutoff is clear by more than 1e-4 in score; scores within 1e-4; row lse
within 1e-4."""
import numpy as np
import pytest
import torch

import oracle
import synth
from inputs import to_dev

pytestmark = pytest.mark.gpu


def _gpu(lib, logits, roots, k, depth, n):
    res = lib.eagle2_rerank(to_dev(logits), to_dev(roots.astype(np.int32)), k, depth, n)
    torch.cuda.synchronize()
    return {key: v.cpu().numpy() for key, v in res.items()}


def _compare(res, logits, roots, k, depth, n):
    for b in range(logits.shape[0]):
        ref = oracle.eagle2_rerank(logits[b], int(roots[b]), k, depth, n)
        np.testing.assert_allclose(res["draft_lse"][b], ref["draft_lse"], atol=1e-4, rtol=0)
        for key in ("tokens", "parents", "depths", "draft_row"):
            assert (res[key][b] == ref[key]).all(), (b, key, res[key][b], ref[key])
        np.testing.assert_allclose(res["scores"][b], ref["scores"], atol=1e-4, rtol=0)


CASES = [
    # (B, V, k, depth, n_nodes)
    (1, 50, 3, 2, 13),
    (2, 1000, 4, 3, 20),
    (3, 5000, 10, 6, 60),
    (1, 4097, 1, 5, 5),
    (2, 300, 8, 1, 9),
    (1, 20000, 16, 4, 64),
    (1, 64, 64, 1, 64),
    # the last 8192-entry vocabulary chunk holds fewer than k entries (16-byte and
    # 4-byte load paths)
    (1, 16388, 10, 3, 25),
    (2, 8195, 6, 3, 15),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_rerank_parity(gpu_lib, case):
    B, V, k, depth, n = CASES[case]
    R = 1 + (depth - 1) * k
    logits = synth.normal_f32((B, R, V), 3.0, 0, 700 + case, 6)
    roots = synth.integers((B,), 0, V, 0, 700 + case, 7)
    print(f"rerank case {case}: B={B} V={V} k={k} depth={depth} n={n}", flush=True)
    _compare(_gpu(gpu_lib, logits, roots, k, depth, n), logits, roots, k, depth, n)


@pytest.mark.parametrize("name", ["C3", "C5"])
def test_rerank_full_size(gpu_lib, name):
    cfg = synth.CONFIGS[name]
    logits = synth.normal_f32((cfg.B, cfg.rows, cfg.V), cfg.draft_std, 0, cfg.index, 6)
    roots = synth.integers((cfg.B,), 0, cfg.V, 0, cfg.index, 7)
    print(f"rerank full size {name}", flush=True)
    _compare(_gpu(gpu_lib, logits, roots, cfg.top_k, cfg.depth, cfg.N), logits, roots, cfg.top_k,
             cfg.depth, cfg.N)


def test_rerank_ties_go_to_lower_token(gpu_lib):
    """Exact logit ties, within a row and across vocabulary chunks: the lower token
    id wins on both sides (depth 1 keeps the tied scores exactly tied in fp32)."""
    V, k, depth, n = 9000, 12, 1, 13
    R = 1 + (depth - 1) * k
    logits = np.round(synth.normal_f32((1, R, V), 2.0, 0, 760, 6) * 2) / 2   # many exact ties
    logits = logits.astype(np.float32)
    roots = np.array([3], np.int32)
    _compare(_gpu(gpu_lib, logits, roots, k, depth, n), logits, roots, k, depth, n)


def test_rerank_constant_rows_take_lowest_tokens(gpu_lib):
    """Rows where every logit ties (thousands of equal candidates per vocabulary
    chunk): each row's proposals are its lowest token ids, on both sides."""
    V, k, depth, n = 9000, 4, 3, 15
    R = 1 + (depth - 1) * k
    logits = synth.normal_f32((2, R, V), 1.0, 0, 770, 6)
    logits[0, 0, :] = 0.5          # root row of sequence 0 is constant
    logits[1, 1:, 4096:] = 7.0     # a constant tail across chunks in sequence 1
    roots = np.array([1, 2], np.int32)
    _compare(_gpu(gpu_lib, logits, roots, k, depth, n), logits, roots, k, depth, n)


def test_rerank_signed_zeros_tie(gpu_lib):
    """Rows whose top-k cut falls among logits of +0.0 and -0.0 (equal values): the two
    zeros rank as one value, so the lower token ids win whatever the sign, on both
    sides; across vocabulary chunks too.  Depth 2 takes the zero ties into the frontier
    rows as well; 16 nodes = the root, the 6 depth-1 nodes and the 9 depth-2 children
    of the three clear winners, a cut 2.0 clear of the next candidates."""
    V, k, depth, n = 9000, 6, 2, 16
    R = 1 + (depth - 1) * k
    base = synth.normal_f32((2, R, V), 1.0, 0, 780, 6)
    logits = np.where(base > 0, -np.abs(base) - 1.0, 0.0).astype(np.float32)   # <= 0 everywhere
    sign = synth.uniform_f32((2, R, V), 0, 780, 7) < 0.5
    logits = np.where((logits == 0.0) & sign, np.float32(-0.0), logits).astype(np.float32)
    logits[:, :, [7, 4100, 8999]] = 2.0          # three clear winners, then the zero ties
    assert np.signbit(logits[logits == 0.0]).any() and (~np.signbit(logits[logits == 0.0])).any()
    roots = np.array([5, 6], np.int32)
    _compare(_gpu(gpu_lib, logits, roots, k, depth, n), logits, roots, k, depth, n)
