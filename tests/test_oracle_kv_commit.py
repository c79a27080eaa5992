"""Pins of the KV-commit oracle ([P3] section 4; the reading new[P+i] = old[P+path[i]]).

The expected arrays below are written out by hand from that reading, not computed
by the oracle: rows are labelled with their own index so a wrong source row, a
shifted destination or a missed layer shows up as a wrong label.
"""
import numpy as np

from oracle.kv_commit import kv_commit


def labelled(L, B, H, cap, D):
    c = np.zeros((L, B, H, cap, D), dtype=np.int64)
    for layer in range(L):
        for b in range(B):
            for h in range(H):
                for r in range(cap):
                    c[layer, b, h, r, :] = 100000 * layer + 10000 * b + 1000 * h + r
    return c


def row_labels(c, layer, b, h):
    return [int(x) % 1000 for x in c[layer, b, h, :, 0]]


def test_worked_example_path_0_2_5():
    # prefix of 3 rows (0..2), tree rows 3..9 (nodes 0..6); accepted path 0 -> 2 -> 5
    c = labelled(1, 1, 1, 10, 2)
    out = kv_commit(c, np.array([2]), np.array([[0, 2, 5, -1]]), P=3)
    #            prefix  | committed: nodes 0, 2, 5 = rows 3, 5, 8 | untouched rows 6..9
    assert row_labels(out, 0, 0, 0) == [0, 1, 2, 3, 5, 8, 6, 7, 8, 9]


def test_every_layer_sequence_and_head():
    c = labelled(2, 2, 2, 8, 1)
    out = kv_commit(c, np.array([1, 3]), np.array([[0, 4, -1, -1], [0, 1, 2, 4]]), P=2)
    for layer in range(2):
        for h in range(2):
            # sequence 0: nodes 0, 4 -> rows 2, 6
            assert row_labels(out, layer, 0, h) == [0, 1, 2, 6, 4, 5, 6, 7]
            # sequence 1: nodes 0, 1, 2, 4 -> rows 2, 3, 4, 6
            assert row_labels(out, layer, 1, h) == [0, 1, 2, 3, 4, 6, 6, 7]
            assert out[layer, 1, h, 5, 0] // 1000 == c[layer, 1, h, 6, 0] // 1000   # same layer/seq/head


def test_root_only_and_failed_acceptance_leave_the_cache_unchanged():
    c = labelled(1, 2, 1, 6, 3)
    out = kv_commit(c, np.array([0, -1]), np.array([[0, -1], [-1, -1]]), P=1)
    np.testing.assert_array_equal(out, c)


def test_identity_path_is_a_no_op_and_input_is_not_modified():
    rng = np.random.default_rng(0)
    c = rng.standard_normal((1, 1, 3, 12, 4))
    keep = c.copy()
    out = kv_commit(c, np.array([4]), np.array([[0, 1, 2, 3, 4]]), P=5)
    np.testing.assert_array_equal(out, keep)
    np.testing.assert_array_equal(c, keep)
