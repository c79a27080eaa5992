"""Pins of the per-depth draft expansion oracle (oracle/draft.py).

[P2] auto-regression head and workflow paragraphs; [P3] section 2.  The pins tie
the oracle to things other than itself:
  * bf16 rounding against the float32 -> bf16 path of the input generator and
    hand-picked ties;
  * every expansion row against a textbook causal decoder layer run with torch's
    own building blocks (linear, silu, scaled_dot_product_attention) on the row's
    root path as a plain sequence: this fixes the wiring of features, tokens, the
    KV rows and the ancestor sets;
  * a worked example whose head reduces to a bigram table, with the tree derived
    by hand;
  * greedy decoding as the one-child special case.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from inputs import DRAFT_CASES, DRAFT_TAU, draft_case, draft_weights_for
from oracle.draft import bf16_round, draft_expand
from oracle.rerank import eagle2_rerank


def test_bf16_round_matches_generator_path_and_ties():
    x = synth.normal_f32((4096,), 3.0, 0, 91, 1)
    want = synth.bf16_bits_to_f64(synth.round_f32_to_bf16_bits(x))
    np.testing.assert_array_equal(bf16_round(x.astype(np.float64)), want)
    # halfway cases go to the even neighbour; just above halfway goes up
    assert bf16_round(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert bf16_round(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    assert bf16_round(np.array([1.0 + 2.0 ** -8 + 2.0 ** -30]))[0] == 1.0 + 2.0 ** -7
    assert bf16_round(np.array([-(1.0 + 2.0 ** -8)]))[0] == -1.0


def _bf(t):
    return t.to(torch.bfloat16).to(torch.float64)


def _rms(z, g, eps):
    return z * torch.rsqrt((z * z).mean(-1, keepdim=True) + eps) * g


def torch_layer_sequence(w, f0, tokens, k_pre, v_pre, P, scale, eps):
    """A plain causal decoder layer over a token sequence, position i fed the output
    feature of position i-1 (f0 for position 0).  Returns (y [T][H], logits [T][V])."""
    T = len(tokens)
    tt = {k: torch.from_numpy(np.asarray(v, dtype=np.float64)) for k, v in w.items()
          if not isinstance(v, int)}
    Hq, Hkv, D = w["Hq"], w["Hkv"], w["D"]
    G = Hq // Hkv
    feats = torch.zeros(T, tt["fc"].shape[0], dtype=torch.float64)
    kp = torch.from_numpy(np.asarray(k_pre, dtype=np.float64)[:, :P])
    vp = torch.from_numpy(np.asarray(v_pre, dtype=np.float64)[:, :P])
    # the inputs of position i depend on the output of i-1, so the whole sequence is
    # recomputed once per new position (a causal layer gives earlier positions the
    # same output each time)
    y = None
    for n in range(1, T + 1):
        f_in = torch.cat([torch.from_numpy(np.asarray(f0, dtype=np.float64))[None], feats[:n - 1]])
        u = torch.cat([f_in, tt["embed"][torch.tensor(tokens[:n])]], dim=1)
        x = F.linear(u, tt["fc"])
        a = _bf(_rms(x, tt["g1"], eps))
        q = _bf(F.linear(a, tt["q"])).view(n, Hq, D).transpose(0, 1)
        k = _bf(F.linear(a, tt["k"])).view(n, Hkv, D).transpose(0, 1)
        v = _bf(F.linear(a, tt["v"])).view(n, Hkv, D).transpose(0, 1)
        K = torch.cat([kp, k], dim=1).repeat_interleave(G, dim=0)
        Vv = torch.cat([vp, v], dim=1).repeat_interleave(G, dim=0)
        mask = torch.ones(n, P + n, dtype=torch.bool)
        mask[:, P:] = torch.tril(torch.ones(n, n, dtype=torch.bool))
        att = F.scaled_dot_product_attention(q, K, Vv, attn_mask=mask, scale=scale)
        att = _bf(att.transpose(0, 1).reshape(n, Hq * D))
        h = x + F.linear(att, tt["o"])
        b2 = _bf(_rms(h, tt["g2"], eps))
        z = _bf(F.silu(F.linear(b2, tt["gate"])) * F.linear(b2, tt["up"]))
        y = _bf(h + F.linear(z, tt["down"]))
        feats[:n] = y
    return y.numpy(), F.linear(y, tt["lm"]).numpy()


SMALL = dict(B=2, H=64, Hq=4, Hkv=2, D=16, I=96, V=50, P=7)


@pytest.mark.parametrize("top_k,depth,n_nodes", [(3, 4, 10), (2, 3, 6)])
def test_every_row_is_the_causal_layer_on_its_root_path(top_k, depth, n_nodes):
    bits, vals = draft_case(3, 90, **SMALL)
    w = draft_weights_for(vals)
    scale, eps = SMALL["D"] ** -0.5, 1e-5
    for b in range(SMALL["B"]):
        tree, logits, feats, prow, rtok = draft_expand(
            w, vals["f0"][b], int(vals["root"][b]), vals["k_cache"][b], vals["v_cache"][b],
            SMALL["P"], top_k, depth, n_nodes, scale, eps)
        R = 1 + (depth - 1) * top_k
        assert prow[0] == -1 and rtok[0] == vals["root"][b]
        for r in range(R):
            path = [r]
            while prow[path[-1]] >= 0:
                path.append(int(prow[path[-1]]))
            path.reverse()
            assert path[0] == 0 and all(p < c for p, c in zip(path, path[1:]))
            y, lg = torch_layer_sequence(w, vals["f0"][b], [int(rtok[p]) for p in path],
                                         vals["k_cache"][b], vals["v_cache"][b], SMALL["P"], scale, eps)
            np.testing.assert_allclose(feats[r], y[-1], rtol=1e-9, atol=1e-9)
            np.testing.assert_allclose(logits[r], lg[-1], rtol=1e-9, atol=1e-9)
        # the tree is the dynamic-tree selection on the rows the head produced
        ref = eagle2_rerank(logits, int(vals["root"][b]), top_k, depth, n_nodes)
        for key in ("tokens", "parents", "depths", "draft_row"):
            np.testing.assert_array_equal(tree[key], ref[key])


def test_one_child_per_node_is_greedy_decoding():
    bits, vals = draft_case(4, 90, **SMALL)
    w = draft_weights_for(vals)
    depth = 5
    tree, logits, feats, prow, rtok = draft_expand(
        w, vals["f0"][0], int(vals["root"][0]), vals["k_cache"][0], vals["v_cache"][0],
        SMALL["P"], 1, depth, depth + 1, SMALL["D"] ** -0.5, 1e-5)
    np.testing.assert_array_equal(tree["parents"], [-1] + list(range(depth)))
    for r in range(depth):
        assert rtok[r + 1] == int(np.argmax(logits[r])) if r + 1 < depth else True
        assert tree["tokens"][r + 1] == int(np.argmax(logits[r]))


def test_bigram_head_worked_example():
    """The head reduced to a lookup: zero attention and MLP weights, W_fc passes the
    token embedding, one-hot embeddings, so row logits = L[token of the row].  Each
    row of L is a permutation of {0, -1, -2, -3}, so every row has the same
    log-normaliser c = log(1 + e^-1 + e^-2 + e^-3) and scores are -(sum of ranks) - d*c.
    Derivation (root token 0, k = 2, depth 3, 6 nodes):
      depth 1 from L[0]: id0 tok1 (-c), id1 tok2 (-1-c)        -> rows 1, 2
      row 1 (tok1) L[1]: id2 tok0 (-2c), id3 tok2 (-1-2c)
      row 2 (tok2) L[2]: id4 tok3 (-1-2c), id5 tok2 (-2-2c)
      depth-2 frontier: id2, then id3 (ties id4, lower id)     -> rows 3, 4
      row 3 (tok0) L[0]: id6 tok1 (-3c), id7 tok2 (-1-3c)
      row 4 (tok2) L[2]: id8 tok3 (-1-3c), id9 tok2 (-2-3c)
      best 5 of all: id0 -0.41, id2 -0.82, id6 -1.22, id1 -1.41, id3 -1.82 (ties id4)
    """
    L = np.array([[-2, 0, -1, -3],
                  [0, -3, -1, -2],
                  [-3, -2, -1, 0],
                  [-1, 0, -3, -2]], dtype=np.float64)
    H = V = 4
    z = lambda *s: np.zeros(s)
    w = {"embed": np.eye(V), "fc": np.concatenate([z(H, H), np.eye(H)], axis=1),
         "q": z(4, H), "k": z(4, H), "v": z(4, H), "o": z(H, 4), "gate": z(4, H), "up": z(4, H),
         "down": z(H, 4), "lm": L.T.copy(), "g1": np.ones(H), "g2": np.ones(H), "Hq": 1, "Hkv": 1, "D": 4}
    tree, logits, feats, prow, rtok = draft_expand(w, np.zeros(H), 0, z(1, 0, 4), z(1, 0, 4), 0,
                                                   2, 3, 6, 0.5, 1e-6)
    c = math.log(1 + math.exp(-1) + math.exp(-2) + math.exp(-3))
    np.testing.assert_array_equal(rtok, [0, 1, 2, 0, 2])
    np.testing.assert_array_equal(prow, [-1, 0, 0, 1, 1])
    np.testing.assert_array_equal(logits, L[[0, 1, 2, 0, 2]])
    np.testing.assert_array_equal(tree["tokens"], [0, 1, 2, 0, 2, 1])
    np.testing.assert_array_equal(tree["parents"], [-1, 0, 0, 1, 1, 3])
    np.testing.assert_array_equal(tree["depths"], [0, 1, 1, 2, 2, 3])
    np.testing.assert_array_equal(tree["draft_row"], [0, 1, 2, 3, 4, -1])
    np.testing.assert_allclose(tree["scores"], [0, -c, -1 - c, -2 * c, -1 - 2 * c, -3 * c], atol=1e-12)


def model_layer_sequence_fp32(w, f0, tokens, k_pre, v_pre, P, scale, eps):
    """The arithmetic of the GPU kernels, modelled on the CPU: the same layer as
    torch_layer_sequence, with every value rounded to bf16 at the same points, but
    float32 accumulation and the softmax weights rounded to bf16 before they multiply
    the values (the attention kernel feeds them to a bf16 matrix product).  Returns
    (y [T][H], logits [T][V]) as float64 arrays."""
    f32 = torch.float32
    bf = lambda t: t.to(torch.bfloat16).to(f32)
    T = len(tokens)
    tt = {k: torch.from_numpy(np.asarray(v, dtype=np.float64)).to(f32) for k, v in w.items()
          if not isinstance(v, int)}
    Hq, Hkv, D = w["Hq"], w["Hkv"], w["D"]
    G = Hq // Hkv
    feats = torch.zeros(T, tt["fc"].shape[0], dtype=f32)
    kp = torch.from_numpy(np.asarray(k_pre, dtype=np.float64)[:, :P]).to(f32)
    vp = torch.from_numpy(np.asarray(v_pre, dtype=np.float64)[:, :P]).to(f32)
    y = None
    for n in range(1, T + 1):
        f_in = torch.cat([torch.from_numpy(np.asarray(f0, dtype=np.float64)).to(f32)[None],
                          feats[:n - 1]])
        u = torch.cat([f_in, tt["embed"][torch.tensor(tokens[:n])]], dim=1)
        x = F.linear(u, tt["fc"])
        a = bf(x * torch.rsqrt((x * x).mean(-1, keepdim=True) + eps) * tt["g1"])
        q = bf(F.linear(a, tt["q"])).view(n, Hq, D).transpose(0, 1)
        k = bf(F.linear(a, tt["k"])).view(n, Hkv, D).transpose(0, 1)
        v = bf(F.linear(a, tt["v"])).view(n, Hkv, D).transpose(0, 1)
        K = torch.cat([kp, k], dim=1).repeat_interleave(G, dim=0)
        Vv = torch.cat([vp, v], dim=1).repeat_interleave(G, dim=0)
        mask = torch.ones(n, P + n, dtype=torch.bool)
        mask[:, P:] = torch.tril(torch.ones(n, n, dtype=torch.bool))
        s = (q @ K.transpose(1, 2)) * scale
        s = s.masked_fill(~mask, float("-inf"))
        e = torch.exp(s - s.amax(-1, keepdim=True))
        att = (bf(e) @ Vv) / e.sum(-1, keepdim=True)
        att = bf(att.transpose(0, 1).reshape(n, Hq * D))
        h = x + F.linear(att, tt["o"])
        b2 = bf(h * torch.rsqrt((h * h).mean(-1, keepdim=True) + eps) * tt["g2"])
        z = bf(F.silu(F.linear(b2, tt["gate"])) * F.linear(b2, tt["up"]))
        y = bf(h + F.linear(z, tt["down"]))
        feats[:n] = y
    return y.double().numpy(), F.linear(y, tt["lm"]).double().numpy()


def test_draft_tolerance_covers_the_kernel_arithmetic():
    """The float tolerance of the GPU draft-expansion parity test, derived from the
    arithmetic rather than from the GPU's output: on every GPU parity case, each row of
    the oracle's expansion recomputed with the kernels' arithmetic (the fp32 model
    above, on the oracle's own row paths) stays within DRAFT_TAU / 1.5 of the oracle's
    logits and features.  The deviation comes from the bf16 softmax weights: they move
    every pre-rounding feature by ~2^-9 relative, so a share of the bf16-rounded
    features lands one bf16 spacing apart (0.031 for features in [4, 8)), and the
    logits differ by the weighted sum of those one-spacing steps."""
    worst_logit, worst_feat = 0.0, 0.0
    for (seed, B, H, Hq, Hkv, D, I, V, P, top_k, depth, n_nodes, _) in DRAFT_CASES:
        R = 1 + (depth - 1) * top_k
        bits, vals = draft_case(seed, 91, B, H, Hq, Hkv, D, I, V, P, cap=P + R + 3)
        w = draft_weights_for(vals)
        scale, eps = D ** -0.5, 1e-5
        for b in range(B):
            tree, logits, feats, prow, rtok = draft_expand(
                w, vals["f0"][b], int(vals["root"][b]), vals["k_cache"][b], vals["v_cache"][b], P,
                top_k, depth, n_nodes, scale, eps)
            for r in range(R):
                path = [r]
                while prow[path[-1]] >= 0:
                    path.append(int(prow[path[-1]]))
                path.reverse()
                y, lg = model_layer_sequence_fp32(w, vals["f0"][b], [int(rtok[p]) for p in path],
                                                  vals["k_cache"][b], vals["v_cache"][b], P, scale, eps)
                worst_logit = max(worst_logit, float(np.abs(lg[-1] - logits[r]).max()))
                worst_feat = max(worst_feat, float(np.abs(y[-1] - feats[r]).max()))
    print(f"fp32 model vs oracle: logits {worst_logit:.4f}, features {worst_feat:.4f}")
    assert worst_logit * 1.5 <= DRAFT_TAU and worst_feat * 1.5 <= DRAFT_TAU
    assert worst_logit > 0.0   # the model does reproduce the effect it accounts for
