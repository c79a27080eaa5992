"""GPU parity of eagle_kv_commit against the oracle ([P3] section 4; a byte copy, so
bit-exact), on caches of several layers, in-place overlapping paths, failed and
root-only acceptances, path contents that name no cache row (the library skips
them; expected values written out by hand), and a greedy acceptance."""
import numpy as np
import pytest
import torch

import synth
from oracle.kv_commit import kv_commit

pytestmark = pytest.mark.gpu


def bf16_cache(shape, seed, tensor):
    return synth.normal_bf16_bits(shape, 1.0, seed, 70, tensor)


def run(gpu_lib, L, B, H, cap, D, P, alen, path):
    kb, vb = bf16_cache((L, B, H, cap, D), 3, 1), bf16_cache((L, B, H, cap, D), 3, 2)
    dev = torch.device("cuda:0")
    k = torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).to(dev)
    v = torch.from_numpy(vb.view(np.int16)).view(torch.bfloat16).to(dev)
    a = torch.tensor(alen, dtype=torch.int32, device=dev)
    p = torch.tensor(path, dtype=torch.int32, device=dev)
    gpu_lib.eagle_kv_commit(k, v, a, p, P)
    torch.cuda.synchronize()
    got_k = k.cpu().view(torch.int16).numpy().view(np.uint16)
    got_v = v.cpu().view(torch.int16).numpy().view(np.uint16)
    # the library caps alpha at path_len - 1; the oracle takes the capped value
    alpha = np.minimum(np.array(alen), len(path[0]) - 1)
    want_k = kv_commit(kb, alpha, np.array(path), P)
    want_v = kv_commit(vb, alpha, np.array(path), P)
    np.testing.assert_array_equal(got_k, want_k)
    np.testing.assert_array_equal(got_v, want_v)


@pytest.mark.parametrize("D", [64, 128])
def test_overlapping_paths_several_layers(gpu_lib, D):
    # path[i] >= i: the row written for entry i is the source of a later entry
    path = [[0, 2, 5, 9, 14, -1, -1], [0, 1, 3, 4, -1, -1, -1], [0, 3, 4, 5, 6, 7, 8]]
    run(gpu_lib, L=3, B=3, H=2, cap=70, D=D, P=37, alen=[4, 3, 6], path=path)


def test_failed_root_only_and_identity(gpu_lib):
    path = [[-1, -1, -1, -1], [0, -1, -1, -1], [0, 1, 2, 3]]
    run(gpu_lib, L=2, B=3, H=4, cap=40, D=128, P=20, alen=[-1, 0, 3], path=path)


def test_longest_path_and_capped_alpha(gpu_lib):
    rng = np.random.default_rng(5)
    nodes = np.sort(rng.choice(np.arange(1, 64), size=64, replace=True))
    path = [[0] + sorted(int(x) for x in nodes)[:64]]
    # alpha larger than the path capacity is capped at path_len - 1 = 64
    run(gpu_lib, L=1, B=1, H=1, cap=64 + 65 + 3, D=128, P=64, alen=[200], path=path)


def test_entries_outside_the_cache_are_skipped(gpu_lib):
    L, B, H, cap, D, P = 1, 1, 2, 30, 64, 20
    path = [[0, 3, 500, -7, 9]]
    kb = bf16_cache((L, B, H, cap, D), 4, 1)
    dev = torch.device("cuda:0")
    k = torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).to(dev)
    v = k.clone()
    gpu_lib.eagle_kv_commit(k, v, torch.tensor([4], dtype=torch.int32, device=dev),
                            torch.tensor(path, dtype=torch.int32, device=dev), P)
    got = k.cpu().view(torch.int16).numpy().view(np.uint16)
    want = kb.copy()
    want[0, 0, :, P + 1] = kb[0, 0, :, P + 3]     # entries 2 (row 520) and 3 (negative) skipped
    want[0, 0, :, P + 4] = kb[0, 0, :, P + 9]
    np.testing.assert_array_equal(got, want)


def test_after_a_greedy_acceptance(gpu_lib):
    # a whole step's acceptance feeding the commit: random trees with planted matches,
    # accepted by the oracle's greedy rule (the inputs never come from the HIP path)
    from oracle.accept import accept_greedy
    B, N, maxd = 2, 26, 6
    rng = np.random.default_rng(11)
    par = np.full((B, N), -1, dtype=np.int32)
    for b in range(B):
        for i in range(1, N):
            par[b, i] = rng.integers(0, i)
    tok = rng.integers(0, 50, size=(B, N)).astype(np.int32)
    amax = rng.integers(0, 50, size=(B, N)).astype(np.int32)
    for b in range(B):
        for i in range(1, N):
            if rng.random() < 0.8:
                tok[b, i] = amax[b, par[b, i]]
    alen, path = [], []
    for b in range(B):
        a, pth, _ = accept_greedy(tok[b], par[b], amax[b], maxd)
        alen.append(a)
        path.append(pth + [-1] * (maxd + 1 - len(pth)))
    assert max(alen) >= 1
    run(gpu_lib, L=2, B=B, H=2, cap=300 + N, D=128, P=300, alen=alen, path=path)
