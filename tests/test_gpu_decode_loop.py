"""GPU end to end: many decoding passes through the HIP calls reproduce plain greedy
decoding of the target.

[P3] section 3 (EAGLE-2's outputs are identical to the target's own decoding) and [P2]
speculative sampling paragraph (a pass that accepts alpha drafts emits alpha + 1
tokens).  The target is a bigram model carried by the LM head alone: the hidden row
of a node is the one-hot row of its token, so eagle_lm_head_argmax gives the target's
greedy next token after every node.  The draft proposes, along its best path, the
target's next token with probability 0.8 and a random token otherwise (so passes
accept anything from 0 to the full depth).  Each pass runs, on the device:

    eagle2_rerank -> eagle_lm_head_argmax -> eagle_accept_greedy -> eagle_kv_commit

with the tree's K/V rows (a per-token table, one per layer and KV head) written after
the sequence's prefix before the commit.  The emitted tokens, concatenated over the
passes, must equal the oracle's autoregressive greedy sequence from the same first
token, and the committed cache rows must be the rows of that sequence, in order.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from inputs import to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

V = H = 512          # one-hot hidden rows: H = V
TOP_K, DEPTH, N_NODES = 4, 5, 20
R = 1 + (DEPTH - 1) * TOP_K
L, HKV, D = 2, 2, 64
PASSES = 24
CFG = 810            # generator workload id of this test


def _bigram_target(seed):
    """W [V][H] bf16 bits: column t holds the logits after token t; the next token
    nxt[t] gets 4.0, every other entry N(0, 0.5^2)."""
    nxt = synth.integers((V,), 0, V, seed, CFG, 1)
    w = synth.normal_f32((V, H), 0.5, seed, CFG, 2)
    w[nxt, np.arange(H)] = 4.0
    return synth.round_f32_to_bf16_bits(w)


def _draft_logits(seq_roots, seed, step, truth):
    """Draft logits [B][R][V] for one pass: N(0, 1) noise; along the best path (slot 0
    of every depth) the row proposing depth d + 1 gets +10 on the draft's guess, which
    is the target's next token with probability 0.8."""
    B = len(seq_roots)
    dl = synth.normal_f32((B, R, V), 1.0, seed, CFG, 100 + step)
    hit = synth.uniform_f32((B, DEPTH), seed, CFG, 400 + step)
    wrong = synth.integers((B, DEPTH), 0, V, seed, CFG, 700 + step)
    for b, root in enumerate(seq_roots):
        g = int(root)
        for d in range(DEPTH):
            g = truth[g] if hit[b, d] < 0.8 else int(wrong[b, d])
            row = 0 if d == 0 else 1 + (d - 1) * TOP_K
            dl[b, row, g] += 10.0
    return dl


@pytest.mark.parametrize("seed", [0, 1])
def test_decode_loop_reproduces_greedy(gpu_lib, seed):
    B = 3
    wbits = _bigram_target(seed)
    # the oracle's greedy next token after every token (one-hot hidden rows), with the
    # margin that makes it unique
    logits, mx, am, second, _ = oracle.lm_head(np.eye(V), synth.bf16_bits_to_f64(wbits))
    assert (mx - second).min() > 1e-2
    truth = [int(a) for a in am]
    first = synth.integers((B,), 0, V, seed, CFG, 3)
    kvtab = synth.normal_bf16_bits((2, L, HKV, V, D), 1.0, seed, CFG, 4)   # K and V rows per token

    dev = torch.device("cuda")
    W = to_dev_bf16(wbits)
    E = torch.eye(V, dtype=torch.bfloat16, device=dev)
    ktab, vtab = to_dev_bf16(kvtab[0]), to_dev_bf16(kvtab[1])
    cap = PASSES * (DEPTH + 1) + N_NODES + 8
    caches = [(torch.zeros((L, 1, HKV, cap, D), dtype=torch.bfloat16, device=dev),
               torch.zeros((L, 1, HKV, cap, D), dtype=torch.bfloat16, device=dev)) for _ in range(B)]
    seqs = [[int(t)] for t in first]
    P = [0] * B
    alphas = []
    print(f"decode loop seed={seed} B={B} passes={PASSES}", flush=True)
    for step in range(PASSES):
        roots = [s[-1] for s in seqs]
        dl = to_dev(_draft_logits(roots, seed, step, truth))
        tree = gpu_lib.eagle2_rerank(dl, to_dev(np.array(roots, np.int32)), TOP_K, DEPTH, N_NODES)
        toks = tree["tokens"]                                     # [B][N], node 0 = root
        hidden = E[toks.view(-1).long()].contiguous()             # one-hot rows of the nodes' tokens
        lm = gpu_lib.eagle_lm_head_argmax(hidden, W)
        alen, path, out = gpu_lib.eagle_accept_greedy(toks, tree["parents"],
                                                      lm["argmax"].view(B, N_NODES), DEPTH)
        for b in range(B):
            k, v = caches[b]
            rows = toks[b].long()
            k[:, 0, :, P[b]:P[b] + N_NODES] = ktab[:, :, rows]
            v[:, 0, :, P[b]:P[b] + N_NODES] = vtab[:, :, rows]
            gpu_lib.eagle_kv_commit(k, v, alen[b:b + 1].contiguous(), path[b:b + 1].contiguous(), P[b])
        torch.cuda.synchronize()
        a_h, o_h = alen.cpu().numpy(), out.cpu().numpy()
        for b in range(B):
            a = int(a_h[b])
            assert 0 <= a <= DEPTH
            seqs[b] += [int(t) for t in o_h[b, :a + 1]]
            P[b] += a + 1
            alphas.append(a)
    for b in range(B):
        ar = [int(first[b])]
        while len(ar) < len(seqs[b]):
            ar.append(truth[ar[-1]])
        assert seqs[b] == ar, f"sequence {b} departs from greedy decoding"
        k, v = caches[b]
        want = np.array(seqs[b][:P[b]])
        np.testing.assert_array_equal(k[:, 0, :, :P[b]].cpu().view(torch.int16).numpy().view(np.uint16),
                                      kvtab[0][:, :, want])
        np.testing.assert_array_equal(v[:, 0, :, :P[b]].cpu().view(torch.int16).numpy().view(np.uint16),
                                      kvtab[1][:, :, want])
    mean_alpha = float(np.mean(alphas))
    print(f"   tokens per pass {mean_alpha + 1:.2f}, lengths {[len(s) for s in seqs]}", flush=True)
    assert mean_alpha > 1.0 and max(alphas) == DEPTH and min(alphas) < DEPTH
