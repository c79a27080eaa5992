"""GPU parity of eagle_tree_verify_attn_paged ([P3] section 4; rows of each
(sequence, KV head) in fixed-size pages of a shared pool) against the paged oracle on
the same seeded inputs, with the attention tolerance (max-abs 2e-2, rel-L2 5e-3, lse
2e-3).  Blocks are placed by a seeded permutation; unused blocks and block-table
entries past the rows hold NaN / garbage and must not be read."""
import numpy as np
import pytest
import torch

import oracle
import synth
from inputs import assert_close_attn, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def _paged_case(cfg, B, N, Hq, Hkv, D, P, ps, spare=7, plant=()):
    L = P + N
    pages = (L + ps - 1) // ps
    nblk = B * pages + spare
    perm = np.random.default_rng(cfg).permutation(nblk)   # block placement only
    kc = synth.normal_bf16_bits((B, Hkv, pages * ps, D), 1.0, 0, cfg, 2)
    vc = synth.normal_bf16_bits((B, Hkv, pages * ps, D), 1.0, 0, cfg, 3)
    for row in plant:   # key rows with every dim 60.0 (bf16 bits 0x4270)
        kc[:, :, row] = 0x4270
    kp = np.full((nblk, Hkv, ps, D), 0x7FC0, np.uint16)
    vp = np.full((nblk, Hkv, ps, D), 0x7FC0, np.uint16)
    table = np.full((B, pages + 3), 123456789, np.int32)   # past the rows: garbage
    for b in range(B):
        for pg in range(pages):
            blk = int(perm[b * pages + pg])
            table[b, pg] = blk
            kp[blk] = kc[b, :, pg * ps:(pg + 1) * ps]
            vp[blk] = vc[b, :, pg * ps:(pg + 1) * ps]
    qb = synth.normal_bf16_bits((B, N, Hq, D), 1.0, 0, cfg, 1)
    parents = synth.random_parents(B, N, 0, cfg, 9)
    return qb, kp, vp, table, parents


@pytest.mark.parametrize("shape", [
    # B, N, Hq, Hkv, D, P, page_size
    (2, 60, 16, 2, 128, 3000, 16),
    (1, 26, 8, 8, 128, 1024, 32),
    (3, 17, 6, 3, 64, 700, 1),
    (2, 40, 8, 1, 128, 5000, 64),
    # one split of 9 chunks: the eight-wave kernel's two-iterations-per-pass loop on pages
    (1, 30, 8, 1, 128, 500, 16),
])
def test_paged_attention(gpu_lib, shape):
    B, N, Hq, Hkv, D, P, ps = shape
    print(f"paged attention B={B} N={N} Hq={Hq} Hkv={Hkv} D={D} P={P} page={ps}", flush=True)
    qb, kp, vp, table, parents = _paged_case(800 + ps + D, B, N, Hq, Hkv, D, P, ps)
    out, lse = gpu_lib.eagle_tree_verify_attn_paged(to_dev_bf16(qb), to_dev_bf16(kp), to_dev_bf16(vp),
                                                    to_dev(table), to_dev(parents), P)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    ref, ref_lse = oracle.tree_verify_attention_paged(
        synth.bf16_bits_to_f64(qb), synth.bf16_bits_to_f64(kp), synth.bf16_bits_to_f64(vp), table,
        parents, P, ps, D ** -0.5)
    assert np.isfinite(got).all()
    assert_close_attn(got, ref)
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, atol=2e-3, rtol=0)


def test_paged_matches_contiguous_bitwise(gpu_lib):
    # same split plan (pages of 32 rows, modest prefix): identical arithmetic
    B, N, Hq, Hkv, D, P, ps = 2, 30, 8, 2, 128, 2000, 32
    qb, kp, vp, table, parents = _paged_case(880, B, N, Hq, Hkv, D, P, ps)
    kc = np.stack([np.concatenate([kp[table[b, pg]] for pg in range((P + N + ps - 1) // ps)], axis=1)
                   for b in range(B)])
    vc = np.stack([np.concatenate([vp[table[b, pg]] for pg in range((P + N + ps - 1) // ps)], axis=1)
                   for b in range(B)])
    a, la = gpu_lib.eagle_tree_verify_attn_paged(to_dev_bf16(qb), to_dev_bf16(kp), to_dev_bf16(vp),
                                                 to_dev(table), to_dev(parents), P)
    c, lc = gpu_lib.eagle_tree_verify_attn(to_dev_bf16(qb), to_dev_bf16(kc), to_dev_bf16(vc),
                                           to_dev(parents), P)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), c.view(torch.int16)) and torch.equal(la, lc)


def test_paged_late_dominant_key(gpu_lib):
    """Keys far into their split whose scores exceed the split's first chunk by more than
    2^64 in weight: the paged kernel must redo the split with the exact row max (wrong
    results would be inf/NaN)."""
    B, N, Hq, Hkv, D, P, ps = 2, 60, 16, 2, 128, 3000, 16
    qb, kp, vp, table, parents = _paged_case(861, B, N, Hq, Hkv, D, P, ps, plant=(P // 2 + 40, 700))
    out, lse = gpu_lib.eagle_tree_verify_attn_paged(to_dev_bf16(qb), to_dev_bf16(kp), to_dev_bf16(vp),
                                                    to_dev(table), to_dev(parents), P)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    ref, ref_lse = oracle.tree_verify_attention_paged(
        synth.bf16_bits_to_f64(qb), synth.bf16_bits_to_f64(kp), synth.bf16_bits_to_f64(vp), table,
        parents, P, ps, D ** -0.5)
    assert np.isfinite(got).all() and np.isfinite(lse.cpu().numpy()).all()
    assert_close_attn(got, ref)
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, atol=2e-3, rtol=1e-6)
