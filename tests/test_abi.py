"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before launching anything."""
import ctypes
import os
import re

import numpy as np
import pytest

import speculative_decoding_attn_amd as sda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "eagle_mi355.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(eagle\w*)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return sda.load()


def test_header_declares_the_five_calls():
    names = _declared()
    for n in ("eagle_tree_verify_attn", "eagle_lm_head_argmax", "eagle_accept_greedy",
              "eagle_accept_spec", "eagle2_rerank"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_covers_every_symbol():
    assert set(_declared()) == set(sda._SIGNATURES)


def test_version_and_status_strings(lib):
    assert lib.eagle_abi_version() == 3
    assert lib.eagle_status_string(0) == b"ok"
    assert lib.eagle_status_string(99) == b"unknown status"


def _tree(arr):
    a = np.ascontiguousarray(np.asarray(arr, dtype=np.int32))
    return a, a.ctypes.data


def test_check_tree(lib):
    a, p = _tree([[-1, 0, 0, 1, 3], [-1, 0, 1, 1, 2]])
    assert lib.eagle_check_tree(p, 2, 5) == 0
    a, p = _tree([[-1, 0, 2]])
    assert lib.eagle_check_tree(p, 1, 3) == 5
    assert b"parents[2]" in lib.eagle_last_error()
    a, p = _tree([[0, 0]])
    assert lib.eagle_check_tree(p, 1, 2) == 5
    assert lib.eagle_check_tree(None, 1, 2) == 1
    assert lib.eagle_check_tree(p, 0, 2) == 2
    assert sda.eagle_check_tree([-1, 0, 1]) is True
    assert sda.eagle_check_tree([-1, 1, 1]) is False


FAKE = 1 << 20   # a non-NULL, 16-byte aligned address that is never dereferenced


def test_attention_argument_errors(lib):
    f = lib.eagle_tree_verify_attn
    ok = dict(B=1, N=10, Hq=2, Hkv=1, D=64, P=128, cap=138, scale=0.125)

    def call(q=FAKE, parents=FAKE, out=FAKE, B=1, N=10, Hq=2, Hkv=1, D=64, P=128, cap=138,
             scale=0.125, dtype=0, ws=None, wsb=0):
        return f(q, FAKE, FAKE, parents, B, N, Hq, Hkv, D, P, cap, scale, dtype, out, None, ws, wsb,
                 None)

    assert call(q=None) == 1
    assert call(dtype=1) == 3                  # EAGLE_F32: not implemented
    assert b"EAGLE_F32" in lib.eagle_last_error()
    assert call(dtype=7) == 2                  # not an eagle_dtype_t
    assert call(out=None) == 1
    assert call(B=0) == 2
    assert call(Hq=3, Hkv=2) == 2
    assert call(N=65, cap=200) == 3
    assert call(D=96) == 3
    assert call(cap=137) == 2
    assert call(scale=0.0) == 2
    assert call(scale=float("nan")) == 2
    assert call(q=FAKE + 2) == 2
    # a shape that needs split-KV partials, without workspace
    need = lib.eagle_tree_verify_attn_workspace(1, 60, 32, 8, 128, 4096)
    assert need > 0
    assert call(N=60, Hq=32, Hkv=8, D=128, P=4096, cap=4156) == 4
    assert call(N=60, Hq=32, Hkv=8, D=128, P=4096, cap=4156, ws=FAKE, wsb=need - 1) == 4
    assert b"need" in lib.eagle_last_error()


def test_workspace_queries_are_pure_and_consistent(lib):
    assert lib.eagle_tree_verify_attn_workspace(1, 10, 2, 1, 64, 128) == 0      # no split
    a = lib.eagle_tree_verify_attn_workspace(4, 60, 64, 8, 128, 32768)
    assert a > 0 and a == lib.eagle_tree_verify_attn_workspace(4, 60, 64, 8, 128, 32768)
    assert lib.eagle_tree_verify_attn_workspace(1, 65, 2, 1, 64, 128) == 0     # unsupported
    assert lib.eagle_lm_head_workspace(240, 8192, 128256) >= 240 * 16
    assert lib.eagle_lm_head_workspace(10, 100, 1000) == 0                     # H % 64 != 0
    assert lib.eagle_accept_spec_workspace(1, 60, 128256) >= 2 * 8 * 128256
    assert lib.eagle2_rerank_workspace(4, 128256, 10, 6) > 0


def test_lm_head_argument_errors(lib):
    f = lib.eagle_lm_head_argmax

    def call(hidden=FAKE, M=4, H=64, V=100, dtype=0, out=FAKE, ws=FAKE, wsb=1 << 20):
        return f(hidden, FAKE, M, H, V, dtype, out, FAKE, FAKE, None, None, ws, wsb, None)

    assert call(hidden=None) == 1
    assert call(dtype=1) == 3
    assert call(dtype=-1) == 2
    assert call(out=None) == 1
    assert call(M=0) == 2
    assert call(V=1) == 2
    assert call(H=100) == 3
    assert call(ws=None) == 4
    assert call(wsb=16) == 4


def test_accept_and_rerank_argument_errors(lib):
    g = lib.eagle_accept_greedy
    assert g(None, FAKE, FAKE, 1, 5, 4, FAKE, FAKE, FAKE, None) == 1
    assert g(FAKE, FAKE, FAKE, 1, 65, 4, FAKE, FAKE, FAKE, None) == 3
    assert g(FAKE, FAKE, FAKE, 1, 5, -1, FAKE, FAKE, FAKE, None) == 2
    s = lib.eagle_accept_spec

    def sp(tokens=FAKE, tl=FAKE, tlse=None, dl=FAKE, dlse=None, mode=0, ws=FAKE, wsb=1 << 20,
           B=1, N=5, V=8, max_depth=3, R=4):
        # tokens, parents, B, N, V, max_depth, target_logits, target_lse, draft_logits,
        # draft_lse, draft_row, draft_rows, u_accept, u_sample, mode, outputs, workspace
        return s(tokens, FAKE, B, N, V, max_depth, tl, tlse, dl, dlse, FAKE, R, FAKE, FAKE, mode,
                 FAKE, FAKE, FAKE, ws, wsb, None)

    assert sp(tokens=None) == 1
    assert sp(tl=None) == 1
    assert sp(dl=None, dlse=FAKE) == 1
    assert b"target_lse" in lib.eagle_last_error()   # the message names the nullable ones
    assert sp(ws=None, wsb=0) == 4
    # sibling model: EAGLE_SPEC_SAMPLED (0) or EAGLE_SPEC_POINT_MASS (1) only
    assert sp(mode=2) == 2
    assert sp(mode=-1) == 2
    assert sp(mode=1, ws=None, wsb=0) == 4
    assert sp(R=0) == 2
    assert sp(N=65) == 3
    r = lib.eagle2_rerank

    def rr(B=1, V=100, k=10, depth=3, n=20, ws=FAKE, wsb=1 << 24):
        return r(FAKE, FAKE, B, V, k, depth, n, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, wsb, None)

    assert rr(k=0) == 2
    assert rr(k=65, V=1000) == 3
    assert rr(k=10, V=5) == 2
    assert rr(n=65) == 3
    assert rr(k=2, depth=2, n=8) == 2          # only 2 + 4 = 6 candidates
    assert rr(k=64, depth=3, V=1000, n=10) == 3  # too many candidates
    assert rr(ws=None) == 4


def test_kv_commit_argument_errors(lib):
    c = lib.eagle_kv_commit

    def kc(k=FAKE, L=2, B=1, H=2, D=128, P=10, cap=80, path_len=7):
        return c(k, FAKE, FAKE, FAKE, L, B, H, D, P, cap, path_len, None)

    assert kc(k=None) == 1
    assert kc(L=0) == 2
    assert kc(P=-1) == 2
    assert kc(D=96) == 3
    assert kc(path_len=66, cap=200) == 3
    assert kc(P=75, cap=80, path_len=7) == 2   # rows P .. P+6 do not fit
    assert kc(k=FAKE + 8) == 2                 # misaligned cache
    assert b"aligned" in lib.eagle_last_error()


def test_ragged_argument_errors(lib):
    a = lib.eagle_tree_verify_attn_ragged
    # both per-sequence arrays NULL: the uniform call is the right one
    assert a(FAKE, FAKE, FAKE, FAKE, None, None, 1, 4, 2, 1, 64, 16, 64, 0.1, 0, FAKE, None, None, 0,
             None) == 1
    # layouts must hold the maxima
    assert a(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4, 2, 1, 64, 16, 19, 0.1, 0, FAKE, None, None, 0,
             None) == 2
    assert a(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4, 2, 1, 64, 16, 64, 0.1, 1, FAKE, None, None, 0,
             None) == 3
    g = lib.eagle_accept_greedy_ragged
    assert g(FAKE, FAKE, FAKE, None, 1, 5, 4, FAKE, FAKE, FAKE, None) == 1
    assert g(FAKE, FAKE, FAKE, FAKE, 1, 65, 4, FAKE, FAKE, FAKE, None) == 3
    s = lib.eagle_accept_spec_ragged
    # tokens, parents, tree_len, B, N, V, max_depth, target_logits, target_lse, draft_logits,
    # draft_lse, draft_row, draft_rows, u_accept, u_sample, mode, outputs, workspace
    assert s(FAKE, FAKE, None, 1, 5, 8, 3, FAKE, None, FAKE, None, FAKE, 4, FAKE, FAKE, 0, FAKE,
             FAKE, FAKE, FAKE, 1 << 20, None) == 1
    assert s(FAKE, FAKE, FAKE, 1, 5, 8, 3, FAKE, None, FAKE, None, FAKE, 4, FAKE, FAKE, 7, FAKE,
             FAKE, FAKE, FAKE, 1 << 20, None) == 2


def test_paged_argument_errors(lib):
    a = lib.eagle_tree_verify_attn_paged

    def pg(ps=16, max_pages=8, nblk=100, P=100, N=10, k=FAKE):
        return a(FAKE, k, FAKE, FAKE, FAKE, 1, N, 2, 1, 64, P, ps, max_pages, nblk, 0.1, 0, FAKE,
                 None, FAKE, 1 << 30, None)

    assert pg(k=None) == 1
    assert pg(ps=24) == 3                  # not a power of two
    assert pg(max_pages=6) == 2            # 6 * 16 < P + N
    assert pg(nblk=0) == 2
    assert lib.eagle_tree_verify_attn_paged_workspace(1, 10, 2, 1, 64, 100, 24) == 0
    # with one-row pages the plan splits a long prefix finely enough for the on-chip
    # slice of the block table, which then needs a split-KV workspace
    assert lib.eagle_tree_verify_attn_paged_workspace(1, 10, 2, 1, 64, 30000, 1) > 0


def test_draft_expand_argument_errors(lib):
    buf = ctypes.create_string_buffer(256)   # host memory: only its address is used
    base = (ctypes.addressof(buf) + 15) // 16 * 16
    head = sda.DraftHead(*([base] * 9))
    f = lib.eagle_draft_expand

    def dx(h=head, B=1, H=256, Hq=4, Hkv=2, D=64, I=512, V=1000, P=10, cap=40, k=4, depth=4, n=12,
           f0=base, ws=None, wsb=0):
        p = ctypes.byref(h) if h is not None else None
        return f(p, f0, base, base, base, B, H, Hq, Hkv, D, I, V, P, cap, k, depth, n, 0.125, 1e-5,
                 *([base] * 10), ws, wsb, None)

    assert dx(h=None) == 1
    assert dx(h=sda.DraftHead(*([base] * 8 + [0]))) == 1   # g2 NULL
    assert dx(f0=None) == 1
    assert dx(H=200) == 3          # H not a multiple of 64
    assert dx(I=100) == 3
    assert dx(D=96) == 3
    assert dx(Hq=3) == 2           # Hq % Hkv
    assert dx(k=10, depth=8, cap=200) == 3   # 71 expansion rows > 64
    assert dx(cap=20) == 2         # kv_cap < P + 13
    assert dx(f0=base + 8) == 2    # misaligned
    assert dx() == 4               # no workspace
    need = lib.eagle_draft_expand_workspace(1, 256, 4, 2, 64, 512, 1000, 10, 40, 4, 4)
    assert need > 0
    assert dx(ws=base, wsb=need - 1) == 4
    assert lib.eagle_draft_expand_workspace(1, 256, 4, 2, 96, 512, 1000, 10, 40, 4, 4) == 0
    assert lib.eagle_draft_expand_workspace(1, 256, 4, 2, 64, 512, 1000, 10, 5, 4, 4) == 0
