"""Pins for the oracle's LM head and its per-row statistics (CPU only)."""
import numpy as np
import torch

import oracle


def test_row_stats_against_log_softmax_and_topk():
    rng = np.random.default_rng(0)
    M, H, V = 7, 33, 501
    hidden = rng.standard_normal((M, H))
    W = rng.standard_normal((V, H)) / np.sqrt(H)
    logits, mx, am, second, lse = oracle.lm_head(hidden, W, block=64)
    t = torch.from_numpy(logits)
    ls = torch.log_softmax(t, dim=1)
    # log-softmax at the argmax is max - lse
    np.testing.assert_allclose(ls[np.arange(M), am].numpy(), mx - lse, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(torch.exp(ls).sum(1).numpy(), 1.0, rtol=1e-12)
    top2 = torch.topk(t, 2, dim=1)
    np.testing.assert_array_equal(top2.indices[:, 0].numpy(), am)
    np.testing.assert_allclose(top2.values[:, 0].numpy(), mx, rtol=0, atol=0)
    np.testing.assert_allclose(top2.values[:, 1].numpy(), second, rtol=0, atol=0)


def test_logits_of_one_hot_rows_select_hidden_entries():
    rng = np.random.default_rng(1)
    M, H, V = 5, 12, 40
    hidden = rng.standard_normal((M, H))
    cols = rng.integers(0, H, size=V)
    W = np.zeros((V, H))
    W[np.arange(V), cols] = np.arange(1, V + 1)        # row v picks hidden[:, cols[v]] * (v+1)
    logits = oracle.lm_head_logits(hidden, W, block=7)
    np.testing.assert_array_equal(logits, hidden[:, cols] * np.arange(1, V + 1))


def test_ties_take_lowest_index_and_second_equals_max():
    rng = np.random.default_rng(2)
    M, H, V = 4, 16, 50
    hidden = rng.standard_normal((M, H))
    W = rng.standard_normal((V, H))
    logits = hidden @ W.T
    best = logits.argmax(1)
    W2 = np.concatenate([W, W], axis=0)                 # index v and v+V tie everywhere
    _, mx, am, second, _ = oracle.lm_head(hidden, W2)
    np.testing.assert_array_equal(am, best)
    np.testing.assert_array_equal(mx, second)
