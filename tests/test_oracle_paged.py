"""Pins of the paged-KV oracle ([P3] section 4; reading: row r of sequence b sits in
block block_table[b][r // page_size] at slot r % page_size).

The gather is checked on a hand-written example with labelled rows; the attention
on pages must equal the contiguous attention for any placement of the blocks,
whatever the unused blocks hold.
"""
import numpy as np

import oracle


def test_gather_worked_example():
    # 4 blocks of 2 rows, 1 head, D=1; block k holds rows labelled 10k, 10k+1
    pool = np.array([[[[10 * k + s] for s in range(2)]] for k in range(4)], dtype=np.int64)
    # sequence 0 uses blocks 2, 0, 3 (rows 0..5); sequence 1 uses blocks 1, 1 (rows 0..3)
    table = [[2, 0, 3], [1, 1, 0]]
    out = oracle.gather_pages(pool, table, rows=5, page_size=2)
    assert out[0, 0, :, 0].tolist() == [20, 21, 0, 1, 30]
    assert out[1, 0, :, 0].tolist() == [10, 11, 10, 11, 0]


def _contig(rng, B, Hkv, L, D):
    return rng.standard_normal((B, Hkv, L, D)), rng.standard_normal((B, Hkv, L, D))


def test_paged_equals_contiguous_for_any_block_placement():
    rng = np.random.default_rng(8)
    B, N, Hq, Hkv, D, P, ps = 2, 9, 4, 2, 8, 21, 4
    L = P + N
    pages = (L + ps - 1) // ps
    k, v = _contig(rng, B, Hkv, L, D)
    q = rng.standard_normal((B, N, Hq, D))
    par = np.array([[-1] + [int(rng.integers(0, i)) for i in range(1, N)] for _ in range(B)])
    nblk = B * pages + 5
    perm = rng.permutation(nblk)
    kp = np.full((nblk, Hkv, ps, D), np.nan)      # unused blocks: NaN, must not be read
    vp = np.full((nblk, Hkv, ps, D), np.nan)
    table = np.zeros((B, pages + 2), dtype=np.int64)
    for b in range(B):
        for pg in range(pages):
            blk = perm[b * pages + pg]
            table[b, pg] = blk
            rows = range(pg * ps, min(L, (pg + 1) * ps))
            for s, r in enumerate(rows):
                kp[blk, :, s] = k[b, :, r]
                vp[blk, :, s] = v[b, :, r]
    out, lse = oracle.tree_verify_attention_paged(q, kp, vp, table, par, P, ps, 0.3)
    o2, l2 = oracle.tree_verify_attention(q, k, v, par, P, 0.3)
    np.testing.assert_array_equal(out, o2)
    np.testing.assert_array_equal(lse, l2)
