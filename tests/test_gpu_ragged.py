"""GPU parity of the ragged-batch calls ([P3] section 4 and closing remarks: batches
whose sequences have their own prefix and tree sizes) against the ragged oracle on
the same seeded inputs.  Attention: the attention tolerance (max-abs 2e-2, rel-L2
5e-3, lse 2e-3); rows past a sequence's tree must be left untouched and cache rows
past its prefix + tree (NaN here) must never be read.  Acceptance: bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import synth
from inputs import assert_close_attn, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

SENTINEL = 0x7F7F   # a bf16 pattern the kernel never produces for these inputs


def _ragged_attention_case(cfg, B, Nmax, Hq, Hkv, D, P_list, N_list, plant=()):
    P_list, N_list = np.array(P_list, np.int32), np.array(N_list, np.int32)
    cap = int(P_list.max()) + Nmax + 5   # the layouts are sized for the maxima
    qb = synth.normal_bf16_bits((B, Nmax, Hq, D), 1.0, 0, cfg, 1)
    kb = synth.normal_bf16_bits((B, Hkv, cap, D), 1.0, 0, cfg, 2)
    vb = synth.normal_bf16_bits((B, Hkv, cap, D), 1.0, 0, cfg, 3)
    for b, row in plant:   # key rows with every dim 60.0 (bf16 bits 0x4270)
        kb[b, :, row] = 0x4270
    for b in range(B):   # rows past this sequence's prefix + tree: NaN, never read
        kb[b, :, P_list[b] + N_list[b]:] = 0x7FC0
        vb[b, :, P_list[b] + N_list[b]:] = 0x7FC0
    parents = synth.random_parents(B, Nmax, 0, cfg, 9)
    return qb, kb, vb, parents, P_list, N_list


@pytest.mark.parametrize("shape", [
    # B, Nmax, Hq, Hkv, D, prefix lengths, tree sizes, planted dominant keys (sequence, row)
    (4, 60, 16, 2, 128, [2048, 300, 0, 1111], [60, 17, 40, 1], ()),
    (3, 33, 4, 4, 64, [64, 4000, 513], [33, 2, 30], ()),
    (2, 26, 8, 1, 128, [9000, 31], [26, 26], ()),
    # keys whose weights overflow the first chunk's reference max: the split is redone
    (4, 60, 16, 2, 128, [6000, 300, 0, 1111], [60, 17, 40, 1], ((0, 3040), (3, 700))),
])
def test_ragged_attention(gpu_lib, shape):
    B, Nmax, Hq, Hkv, D, P_list, N_list, plant = shape
    print(f"ragged attention B={B} Nmax={Nmax} Hq={Hq} Hkv={Hkv} D={D} P={P_list} N={N_list} "
          f"planted={plant}", flush=True)
    qb, kb, vb, parents, P_arr, N_arr = _ragged_attention_case(700 + D + B, B, Nmax, Hq, Hkv, D,
                                                               P_list, N_list, plant)
    Pmax = int(P_arr.max())
    dev = torch.device("cuda:0")
    out = torch.full((B, Nmax, Hq, D), 0, dtype=torch.int16, device=dev)
    out.fill_(SENTINEL)
    out = out.view(torch.bfloat16)
    lse = torch.full((B, Nmax, Hq), 12345.0, dtype=torch.float32, device=dev)
    gpu_lib.eagle_tree_verify_attn(to_dev_bf16(qb), to_dev_bf16(kb), to_dev_bf16(vb), to_dev(parents),
                                   Pmax, D ** -0.5, out=out, lse=lse, prefix_len=to_dev(P_arr),
                                   tree_len=to_dev(N_arr))
    torch.cuda.synchronize()
    got_bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
    got = synth.bf16_bits_to_f64(got_bits)
    got_lse = lse.cpu().numpy()
    ref, ref_lse = oracle.tree_verify_attention_ragged(
        synth.bf16_bits_to_f64(qb), synth.bf16_bits_to_f64(kb), synth.bf16_bits_to_f64(vb),
        parents, P_arr, N_arr, D ** -0.5)
    for b in range(B):
        n = N_arr[b]
        assert_close_attn(got[b, :n], ref[b, :n])
        np.testing.assert_allclose(got_lse[b, :n], ref_lse[b, :n], atol=2e-3, rtol=0)
        assert (got_bits[b, n:] == SENTINEL).all(), "rows past the tree were written"
        assert (got_lse[b, n:] == 12345.0).all()


@pytest.mark.parametrize("shape", [
    (2, 20, 8, 2, 128, 700),   # four-wave workgroups (256-key minimum split)
    (2, 20, 2, 2, 128, 700),   # one-wave workgroups (128-key minimum split)
])
def test_ragged_attention_equals_uniform_when_sizes_agree(gpu_lib, shape):
    B, N, Hq, Hkv, D, P = shape
    qb, kb, vb, parents, P_arr, N_arr = _ragged_attention_case(760, B, N, Hq, Hkv, D, [P, P], [N, N])
    args = (to_dev_bf16(qb), to_dev_bf16(kb), to_dev_bf16(vb), to_dev(parents), P, D ** -0.5)
    a, la = gpu_lib.eagle_tree_verify_attn(*args)
    r, lr = gpu_lib.eagle_tree_verify_attn(*args, prefix_len=to_dev(P_arr), tree_len=to_dev(N_arr))
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), r.view(torch.int16)) and torch.equal(la, lr)


def test_ragged_greedy(gpu_lib):
    B, Nmax, maxd = 16, 40, 7
    parents = synth.random_parents(B, Nmax, 0, 770, 1)
    amax = synth.integers((B, Nmax), 0, 30, 0, 770, 2).astype(np.int32)
    tok = synth.integers((B, Nmax), 0, 30, 0, 770, 3).astype(np.int32)
    plant = synth.uniform_f32((B, Nmax), 0, 770, 4) < 0.8
    for b in range(B):
        for i in range(1, Nmax):
            if plant[b, i]:
                tok[b, i] = amax[b, parents[b, i]]
    N_arr = synth.integers((B,), 1, Nmax + 1, 0, 770, 5).astype(np.int32)
    a, p, o = gpu_lib.eagle_accept_greedy(to_dev(tok), to_dev(parents), to_dev(amax), maxd,
                                          tree_len=to_dev(N_arr))
    torch.cuda.synchronize()
    a, p, o = a.cpu().numpy(), p.cpu().numpy(), o.cpu().numpy()
    want = oracle.accept_greedy_ragged(tok, parents, amax, N_arr, maxd)
    for b, (alpha, path, out) in enumerate(want):
        assert a[b] == alpha
        assert list(p[b]) == list(path) + [-1] * (maxd + 1 - len(path))
        assert list(o[b]) == list(out) + [-1] * (maxd + 1 - len(out))


@pytest.mark.parametrize("with_lse", [False, True])
@pytest.mark.parametrize("mode", ["sampled", "point_mass"])
def test_ragged_spec(gpu_lib, mode, with_lse):
    B, Nmax, V, R_per, maxd = 8, 24, 700, 5, 64
    parents = synth.random_parents(B, Nmax, 0, 780, 1)
    tl = synth.normal_f32((B, Nmax, V), 1.0, 0, 780, 2)
    dl = synth.normal_f32((B, R_per, V), 1.5, 0, 780, 3)
    ua = synth.uniform_f32((B, Nmax), 0, 780, 4)
    us = synth.uniform_f32((B, Nmax), 0, 780, 5)
    rowpick = synth.integers((B, Nmax), 0, R_per, 0, 780, 6)
    N_arr = synth.integers((B,), 2, Nmax + 1, 0, 780, 7).astype(np.int32)
    draft_row = np.full((B, Nmax), -1, np.int32)
    tokens = synth.integers((B, Nmax), 0, V, 0, 780, 8).astype(np.int32)
    for b in range(B):
        for v in sorted(set(parents[b, 1:].tolist())):
            draft_row[b, v] = rowpick[b, v]
    tlse = dlse = None
    if with_lse:   # the rows' normalisers as a caller hands them over: fp32, from the CPU
        from scipy.special import logsumexp
        tlse = logsumexp(tl.astype(np.float64), axis=-1).astype(np.float32)
        dlse = logsumexp(dl.astype(np.float64), axis=-1).astype(np.float32)
    a, p, o = gpu_lib.eagle_accept_spec(to_dev(tokens), to_dev(parents), to_dev(draft_row), to_dev(tl),
                                        to_dev(dl), to_dev(ua), to_dev(us), maxd, tree_len=to_dev(N_arr),
                                        mode=mode, target_lse=None if tlse is None else to_dev(tlse),
                                        draft_lse=None if dlse is None else to_dev(dlse))
    torch.cuda.synchronize()
    a, p, o = a.cpu().numpy(), p.cpu().numpy(), o.cpu().numpy()
    checked = 0
    for b in range(B):
        n = int(N_arr[b])
        trace = []
        alpha, path, out = oracle.accept_spec(tokens[b][:n], parents[b][:n], tl[b][:n], dl[b],
                                              draft_row[b][:n], ua[b][:n], us[b][:n], maxd, trace=trace,
                                              mode=mode,
                                              target_lse=None if tlse is None else tlse[b][:n],
                                              draft_lse=None if dlse is None else dlse[b])
        margins = [abs(float(ua[b, kid]) - r) for (_, kids, ratios, _) in trace
                   for kid, r in zip(kids, ratios)]
        if margins and min(margins) <= 1e-6:
            continue
        checked += 1
        assert a[b] == alpha
        assert list(p[b, :alpha + 1]) == list(path)
        assert list(o[b, :alpha]) == out[:alpha]
        assert all(int(x) < n for x in p[b, :alpha + 1])   # only nodes of this tree
    assert checked >= B - 1
