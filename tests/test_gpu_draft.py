"""Per-depth draft expansion on the GPU against the oracle (oracle/draft.py).

Indices (each row's token and proposing row, the final tree) bit-exact; draft
logits and features within a float tolerance derived from the arithmetic (not from
the GPU's output): tests/test_oracle_draft.py recomputes the oracle's rows with the
kernels' arithmetic modelled on the CPU (fp32 accumulation, bf16 storage at the same
points, softmax weights rounded to bf16 before the value product) and finds logits
within 0.027 and features within 0.031 (one bf16 spacing in [4, 8)) of the oracle; so
logits and features get max-abs DRAFT_TAU = 0.05 (at least 1.5 x that) and relative
L2 1e-2.

The expansion's decisions compare cumulative log-probabilities, so a decision whose
margin is below that error may go either way.  What the decisions make unique is
compared: a node is identified by its token path from the root (its row number and
output position also depend on the order among the chosen candidates, which may be
a near-tie without changing which candidates are chosen).  Rows are compared down to
the last depth whose choices (each proposing row's top-k cut, the frontier's cut)
all have a margin above DRAFT_TAU in the oracle, matched by token path; the tree, as
the set of token paths with their depths and scores, when every cut including the
final selection's is that clear.
"""
import numpy as np
import pytest
import torch

import synth
from inputs import (DRAFT_CASES, DRAFT_TAU, draft_case, draft_weights_for, rel_l2, to_dev,
                    to_dev_bf16)
from oracle.draft import draft_expand, draft_layer_row
import speculative_decoding_attn_amd as sda

pytestmark = pytest.mark.gpu

TAU = DRAFT_TAU


def assert_close_draft(got, ref):
    """Logits and features: max-abs TAU and relative L2 1e-2."""
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref).max()
    rl = rel_l2(got, ref)
    assert err <= TAU and rl <= 1e-2, f"max-abs {err:.3g}, rel-L2 {rl:.3g}"


def device_head(bits):
    cat = lambda *names: np.concatenate([bits[n] for n in names], axis=0)
    return {"embed": to_dev_bf16(bits["embed"]), "w_fc": to_dev_bf16(bits["fc"]),
            "w_qkv": to_dev_bf16(cat("q", "k", "v")), "w_o": to_dev_bf16(bits["o"]),
            "w_gate_up": to_dev_bf16(cat("gate", "up")), "w_down": to_dev_bf16(bits["down"]),
            "w_lm": to_dev_bf16(bits["lm"]), "g1": to_dev(bits["g1"]), "g2": to_dev(bits["g2"])}


def _cut_clear(values, count):
    """True if the `count` best of `values` are more than TAU above the rest."""
    v = np.asarray(values, dtype=np.float64)
    if v.size <= count:
        return True
    s = np.sort(v)[::-1]
    return bool(s[count - 1] - s[count] > TAU)


def decided(logits, prow, top_k, depth, n_nodes):
    """(deepest depth whose rows are decided clearly, whether the whole tree is)."""
    R = logits.shape[0]
    lse = np.array([r.max() + np.log(np.exp(r - r.max()).sum()) for r in logits])
    row_depth = np.array([0] + [1 + (r - 1) // top_k for r in range(1, R)])
    score = np.zeros(R)   # a row's node score (filled as its depth is reached)
    level, every = {}, []
    for d in range(1, depth + 1):
        cands = []
        for r in np.nonzero(row_depth == d - 1)[0]:
            top = np.argsort(-logits[r], kind="stable")[:top_k]
            cands += [score[r] + logits[r][t] - lse[r] for t in top]
        level[d] = cands
        every += cands
        if d < depth:
            order = np.argsort(-np.asarray(cands), kind="stable")[:top_k]
            for j, c in enumerate(order):
                score[1 + (d - 1) * top_k + j] = cands[c]
    safe = 0
    for d in range(1, depth):
        rows_ok = all(_cut_clear(logits[r], top_k) for r in np.nonzero(row_depth == d - 1)[0])
        if not (rows_ok and _cut_clear(level[d], top_k)):
            break
        safe = d
    tree_ok = (safe == depth - 1 and all(_cut_clear(logits[r], top_k) for r in range(R))
               and _cut_clear(every, n_nodes - 1))
    return safe, tree_ok


def paths(tokens, parents):
    """Token path from the root of every entry of a parent-linked list."""
    out = []
    for i in range(len(tokens)):
        p, j = [], i
        while j >= 0:
            p.append(int(tokens[j]))
            j = int(parents[j])
        out.append(tuple(reversed(p)))
    return out


def run_case(seed, B, H, Hq, Hkv, D, I, V, P, top_k, depth, n_nodes):
    R = 1 + (depth - 1) * top_k
    bits, vals = draft_case(seed, 91, B, H, Hq, Hkv, D, I, V, P, cap=P + R + 3)
    scale, eps = D ** -0.5, 1e-5
    print(f"draft expand seed={seed} B={B} H={H} Hq={Hq} Hkv={Hkv} D={D} I={I} V={V} P={P} "
          f"k={top_k} depth={depth} n={n_nodes}", flush=True)
    head = device_head(bits)
    kc, vc = to_dev_bf16(bits["k_cache"]), to_dev_bf16(bits["v_cache"])
    got = sda.eagle_draft_expand(head, to_dev_bf16(bits["f0"]), to_dev(bits["root"]), kc, vc, P, Hq,
                                 top_k, depth, n_nodes, scale, eps)
    torch.cuda.synchronize()
    g = {k: v.cpu() for k, v in got.items()}
    w = draft_weights_for(vals)
    verified_rows, trees_checked = [], []
    for b in range(B):
        tree, logits, feats, prow, rtok = draft_expand(
            w, vals["f0"][b], int(vals["root"][b]), vals["k_cache"][b], vals["v_cache"][b], P, top_k,
            depth, n_nodes, scale, eps)
        sd, tree_clear = decided(logits, prow, top_k, depth, n_nodes)
        rows = 1 + sd * top_k   # rows of depths 0 .. sd
        verified_rows.append(rows)
        want = {pth: r for r, pth in enumerate(paths(rtok, prow)[:rows])}
        have = {pth: r for r, pth in enumerate(paths(g["row_token"][b].numpy(), g["parent_row"][b].numpy())[:rows])}
        assert set(have) == set(want), f"sequence {b}: rows of depth <= {sd} differ"
        order_w = [want[pth] for pth in want]
        order_h = [have[pth] for pth in want]
        assert_close_draft(g["draft_logits"][b].numpy()[order_h], logits[order_w])
        assert_close_draft(g["features"][b].float().numpy()[order_h], feats[order_w])
        np.testing.assert_allclose(g["draft_lse"][b].numpy()[order_h], tree["draft_lse"][order_w], atol=TAU)
        if tree_clear:
            trees_checked.append(b)
            tw = dict(zip(paths(tree["tokens"], tree["parents"]), zip(tree["depths"], tree["scores"])))
            th = dict(zip(paths(g["tokens"][b].numpy(), g["parents"][b].numpy()),
                          zip(g["depths"][b].numpy(), g["scores"][b].numpy())))
            assert set(th) == set(tw), f"sequence {b}: trees differ"
            for pth in tw:
                assert th[pth][0] == tw[pth][0]
                assert abs(th[pth][1] - tw[pth][1]) <= TAU
            # breadth-first output: depths never decrease, parents come first
            d_out = g["depths"][b].numpy()
            assert np.all(np.diff(d_out) >= 0) and np.all(g["parents"][b].numpy()[1:] < np.arange(1, n_nodes))
        # the cache rows the expansion wrote are the rows' keys and values: the
        # oracle's attention read them, so matching logits already vouch for them;
        # the prefix rows are left alone
        np.testing.assert_array_equal(kc[b, :, :P].cpu().view(torch.int16).numpy().view(np.uint16),
                                      bits["k_cache"][b, :, :P])
    print(f"   rows verified per sequence {verified_rows}, whole trees {trees_checked}", flush=True)
    return verified_rows, trees_checked


@pytest.mark.parametrize("seed,B,H,Hq,Hkv,D,I,V,P,top_k,depth,n_nodes,whole_tree", DRAFT_CASES)
def test_draft_expand_matches_oracle(gpu_lib, seed, B, H, Hq, Hkv, D, I, V, P, top_k, depth, n_nodes,
                                     whole_tree):
    rows, trees = run_case(seed, B, H, Hq, Hkv, D, I, V, P, top_k, depth, n_nodes)
    assert max(rows) > 1 + top_k   # rows of depth 2 or deeper were compared
    assert bool(trees) == whole_tree


def test_draft_expand_rejects_bad_sizes(gpu_lib):
    bits, _ = draft_case(1, 91, 1, 256, 4, 2, 64, 512, 1000, 10, cap=30)
    head = device_head(bits)
    kc, vc = to_dev_bf16(bits["k_cache"]), to_dev_bf16(bits["v_cache"])
    with pytest.raises(sda.EagleError):   # kv_cap < P + R
        sda.eagle_draft_expand(head, to_dev_bf16(bits["f0"]), to_dev(bits["root"]), kc, vc, 10, 4,
                               5, 5, 10, 0.125, 1e-5)
    with pytest.raises(sda.EagleError):   # 1 + (depth-1)*top_k > 64 rows
        sda.eagle_draft_expand(head, to_dev_bf16(bits["f0"]), to_dev(bits["root"]), kc, vc, 10, 4,
                               10, 8, 10, 0.125, 1e-5)


class _Rows:
    """Row access to a bf16 table without converting all of it (the embedding)."""

    def __init__(self, bits):
        self.bits = bits

    def __getitem__(self, i):
        return synth.bf16_bits_to_f64(self.bits[i])


def test_draft_expand_full_size_sampled(gpu_lib):
    """Llama-3-8B-shaped draft head (H 4096, 32/8 heads, MLP 14336, vocabulary 128256),
    draft prefix 4096, top-k 10, depth 6, 60 nodes.  Sampled against the oracle: the
    root row and the ten depth-1 rows, each computed by the oracle from its own
    choices (the root row's top 10), matched to the GPU's rows by token."""
    B, H, Hq, Hkv, D, I, V, P, k, depth, n = 1, 4096, 32, 8, 128, 14336, 128256, 4096, 10, 6, 60
    R = 1 + (depth - 1) * k
    bits, vals = draft_case(5, 93, B, H, Hq, Hkv, D, I, V, P, cap=P + R)
    scale, eps = D ** -0.5, 1e-5
    print(f"draft expand full size: H={H} I={I} V={V} P={P} k={k} depth={depth}", flush=True)
    head = device_head(bits)
    kc, vc = to_dev_bf16(bits["k_cache"]), to_dev_bf16(bits["v_cache"])
    got = sda.eagle_draft_expand(head, to_dev_bf16(bits["f0"]), to_dev(bits["root"]), kc, vc, P, Hq, k,
                                 depth, n, scale, eps)
    torch.cuda.synchronize()
    g = {key: v.cpu().numpy() if v.dtype != torch.bfloat16 else v.float().cpu().numpy()
         for key, v in got.items()}
    del head, kc, vc, got
    torch.cuda.empty_cache()
    w = {key: vals[key] for key in ("fc", "q", "k", "v", "o", "gate", "up", "down", "lm", "g1", "g2",
                                    "Hq", "Hkv", "D")}
    w["embed"] = _Rows(bits["embed"])
    kcache = np.zeros((Hkv, P + R, D))
    vcache = np.zeros((Hkv, P + R, D))
    kcache[:, :P] = vals["k_cache"][0, :, :P]
    vcache[:, :P] = vals["v_cache"][0, :, :P]
    y0, l0 = draft_layer_row(w, vals["f0"][0], int(vals["root"][0]), kcache, vcache, [0], 0, P, scale, eps)
    assert_close_draft(g["draft_logits"][0, 0], l0)
    assert_close_draft(g["features"][0, 0], y0)
    # the depth-1 rows: the oracle computes a row for every token that may rank in the
    # root row's top k within the logit tolerance (its own candidates); the GPU's k
    # choices must come from them, include every clearly chosen token, and match the
    # oracle's row for the same token
    s0 = np.sort(l0)[::-1]
    maybe = [int(t) for t in np.nonzero(l0 >= s0[k - 1] - TAU)[0]]
    sure = {int(t) for t in np.nonzero(l0 > s0[k] + TAU)[0]}
    gpu_row_of = {int(g["row_token"][0, r]): r for r in range(1, 1 + k)}
    assert len(gpu_row_of) == k and set(gpu_row_of) <= set(maybe) and sure <= set(gpu_row_of)
    assert all(g["parent_row"][0, r] == 0 for r in range(1, 1 + k))
    for t in maybe:
        if t not in gpu_row_of:
            continue
        kc1, vc1 = kcache.copy(), vcache.copy()
        y1, l1 = draft_layer_row(w, y0, t, kc1, vc1, [1, 0], 1, P, scale, eps)
        assert_close_draft(g["draft_logits"][0, gpu_row_of[t]], l1)
        assert_close_draft(g["features"][0, gpu_row_of[t]], y1)
    # properties of the whole result at this size: a breadth-first tree of n nodes
    # whose scores never grow down a path, every node's token is among the top k of
    # its proposing row, and the rows' normalisers match their logits
    par, tok, dep, sc = g["parents"][0], g["tokens"][0], g["depths"][0], g["scores"][0]
    assert par[0] == -1 and np.all(par[1:] < np.arange(1, n)) and np.all(np.diff(dep) >= 0)
    assert np.all(dep[1:] == dep[par[1:]] + 1) and np.all(sc[1:] <= sc[par[1:]] + 1e-4)
    lse = g["draft_lse"][0]
    logits = g["draft_logits"][0]
    for r in range(R):
        ref = logits[r].max() + np.log(np.exp(logits[r] - logits[r].max()).sum())
        assert abs(lse[r] - ref) < 1e-3
    for i in range(1, n):
        row = g["draft_row"][0, par[i]]
        kth = np.sort(logits[row])[::-1][k - 1]
        assert logits[row][tok[i]] >= kth - 1e-6
        assert abs(sc[i] - (sc[par[i]] + logits[row][tok[i]] - lse[row])) < 1e-3
