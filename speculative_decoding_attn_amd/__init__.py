"""Python binding of the EAGLE / EAGLE-2 tree-verification library for MI355X.

Thin ctypes wrappers with the C-ABI names (include/eagle_mi355.h).  They check
tensor device, dtype and contiguity, allocate outputs and workspace through
PyTorch (device memory only) and pass raw pointers plus the current HIP stream.
Every step of the computation runs in the HIP kernels of ``libeagle_mi355.so``;
there is no fallback: if the library is missing or a call fails, an exception is
raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libeagle_mi355.so")

_lib = None

EAGLE_OK = 0
SPEC_MODES = {"sampled": 0, "point_mass": 1}   # eagle_spec_mode_t
EAGLE_BF16 = 0                                 # eagle_dtype_t of bf16 operands
STATUS_NAMES = {0: "EAGLE_OK", 1: "EAGLE_ERR_NULL", 2: "EAGLE_ERR_INVALID_ARG",
                3: "EAGLE_ERR_UNSUPPORTED", 4: "EAGLE_ERR_WORKSPACE", 5: "EAGLE_ERR_TREE",
                6: "EAGLE_ERR_HIP"}


class EagleError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        super().__init__(f"{func}: {STATUS_NAMES.get(status, status)}: {detail}")
        self.status = status


_vp, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t

_SIGNATURES = {
    "eagle_abi_version": ([], ctypes.c_int),
    "eagle_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "eagle_last_error": ([], ctypes.c_char_p),
    "eagle_check_tree": ([_vp, _i32, _i32], ctypes.c_int),
    "eagle_tree_verify_attn_workspace": ([_i32] * 6, _sz),
    "eagle_tree_verify_attn": ([_vp, _vp, _vp, _vp] + [_i32] * 7 + [_f32, _i32, _vp, _vp, _vp, _sz,
                                                                    _vp], ctypes.c_int),
    "eagle_lm_head_workspace": ([_i32] * 3, _sz),
    "eagle_lm_head_argmax": ([_vp, _vp, _i32, _i32, _i32, _i32] + [_vp] * 6 + [_sz, _vp], ctypes.c_int),
    "eagle_lm_head_argmax_noalloc": ([_vp, _vp, _i32, _i32, _i32, _i32] + [_vp] * 6, ctypes.c_int),
    "eagle_accept_greedy": ([_vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp], ctypes.c_int),
    "eagle_kv_commit": ([_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp],
                        ctypes.c_int),
    "eagle_accept_spec_workspace": ([_i32] * 3, _sz),
    "eagle_accept_spec": ([_vp, _vp, _i32, _i32, _i32, _i32] + [_vp] * 5 + [_i32, _vp, _vp, _i32]
                          + [_vp] * 4 + [_sz, _vp], ctypes.c_int),
    "eagle_tree_verify_attn_ragged": ([_vp] * 6 + [_i32] * 7 + [_f32, _i32, _vp, _vp, _vp, _sz, _vp],
                                      ctypes.c_int),
    "eagle_tree_verify_attn_paged_workspace": ([_i32] * 7, _sz),
    "eagle_tree_verify_attn_paged": ([_vp] * 5 + [_i32] * 9 + [_f32, _i32, _vp, _vp, _vp, _sz, _vp],
                                     ctypes.c_int),
    "eagle_accept_greedy_ragged": ([_vp] * 4 + [_i32, _i32, _i32] + [_vp] * 4, ctypes.c_int),
    "eagle_accept_spec_ragged": ([_vp, _vp, _vp, _i32, _i32, _i32, _i32] + [_vp] * 5
                                 + [_i32, _vp, _vp, _i32] + [_vp] * 4 + [_sz, _vp], ctypes.c_int),
    "eagle2_rerank_workspace": ([_i32] * 4, _sz),
    "eagle2_rerank": ([_vp, _vp] + [_i32] * 5 + [_vp] * 7 + [_sz, _vp], ctypes.c_int),
    "eagle_draft_expand_workspace": ([_i32] * 11, _sz),
    "eagle_draft_expand": ([_vp] * 5 + [_i32] * 12 + [_f32, _f32] + [_vp] * 11 + [_sz, _vp],
                           ctypes.c_int),
    "eagle_calib_stream_read": ([_vp, _sz, _vp, _vp], ctypes.c_int),
    "eagle_calib_mfma_bf16_flops": ([_i32], ctypes.c_double),
    "eagle_calib_mfma_bf16": ([_i32, _vp, _sz, _vp], ctypes.c_int),
}


class DraftHead(ctypes.Structure):
    """The C struct eagle_draft_head: device pointers of the draft head's weights."""
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("embed", "w_fc", "w_qkv", "w_o", "w_gate_up", "w_down", "w_lm", "g1", "g2")]


def load(path: Optional[str] = None):
    """Load the shared library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m speculative_decoding_attn_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (args, res) in _SIGNATURES.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    lib.eagle_draft_expand.argtypes = [ctypes.POINTER(DraftHead)] + _SIGNATURES["eagle_draft_expand"][0][1:]
    _lib = lib
    return lib


def _check(status: int, func: str) -> None:
    if status != EAGLE_OK:
        raise EagleError(status, func, _lib.eagle_last_error().decode())


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype, device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def eagle_check_tree(parents) -> bool:
    """Host-side validation of a [B][N] parent array (any array-like of ints)."""
    lib = load()
    t = torch.as_tensor(parents, dtype=torch.int32).contiguous().cpu()
    if t.dim() == 1:
        t = t[None]
    st = lib.eagle_check_tree(t.data_ptr(), t.shape[0], t.shape[1])
    if st not in (EAGLE_OK, 5):
        _check(st, "eagle_check_tree")
    return st == EAGLE_OK


def eagle_tree_verify_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, parents: torch.Tensor,
                           P: int, scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                           lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                           workspace: Optional[torch.Tensor] = None,
                           prefix_len: Optional[torch.Tensor] = None,
                           tree_len: Optional[torch.Tensor] = None):
    """q [B][N][Hq][D] bf16; k, v [B][Hkv][kv_cap][D] bf16; parents [B][N] int32.

    With prefix_len / tree_len (int32 [B]) the batch is ragged (P and N are then the
    maxima) and eagle_tree_verify_attn_ragged is called.
    Returns (out [B][N][Hq][D] bf16, lse [B][N][Hq] fp32 or None)."""
    lib = load()
    dev = q.device
    _need(q, "q", torch.bfloat16, dev)
    _need(k, "k", torch.bfloat16, dev)
    _need(v, "v", torch.bfloat16, dev)
    _need(parents, "parents", torch.int32, dev)
    B, N, Hq, D = q.shape
    Hkv, kv_cap = k.shape[1], k.shape[2]
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != D or tuple(parents.shape) != (B, N):
        raise ValueError("inconsistent shapes")
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty((B, N, Hq, D), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, dev)
    if lse is None and want_lse:
        lse = torch.empty((B, N, Hq), dtype=torch.float32, device=dev)
    ws_bytes = lib.eagle_tree_verify_attn_workspace(B, N, Hq, Hkv, D, P)
    if workspace is None and ws_bytes:
        workspace = _workspace(ws_bytes, dev)
    wsb = 0 if workspace is None else workspace.numel()
    if prefix_len is None and tree_len is None:
        st = lib.eagle_tree_verify_attn(q.data_ptr(), k.data_ptr(), v.data_ptr(), parents.data_ptr(),
                                        B, N, Hq, Hkv, D, P, kv_cap, float(scale), EAGLE_BF16,
                                        out.data_ptr(), _ptr(lse), _ptr(workspace), wsb, _stream())
        _check(st, "eagle_tree_verify_attn")
        return out, lse
    for t, n in ((prefix_len, "prefix_len"), (tree_len, "tree_len")):
        if t is not None:
            _need(t, n, torch.int32, dev)
            if tuple(t.shape) != (B,):
                raise ValueError(f"{n} must be [B]")
    st = lib.eagle_tree_verify_attn_ragged(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                           parents.data_ptr(), _ptr(prefix_len), _ptr(tree_len),
                                           B, N, Hq, Hkv, D, P, kv_cap, float(scale), EAGLE_BF16,
                                           out.data_ptr(), _ptr(lse), _ptr(workspace), wsb,
                                           _stream())
    _check(st, "eagle_tree_verify_attn_ragged")
    return out, lse


def eagle_tree_verify_attn_paged(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                                 block_table: torch.Tensor, parents: torch.Tensor, P: int,
                                 scale: Optional[float] = None, want_lse: bool = True,
                                 workspace: Optional[torch.Tensor] = None):
    """q [B][N][Hq][D] bf16; k_pool, v_pool [num_blocks][Hkv][page_size][D] bf16;
    block_table [B][max_pages] int32; parents [B][N] int32.
    Returns (out [B][N][Hq][D] bf16, lse [B][N][Hq] fp32 or None)."""
    lib = load()
    dev = q.device
    _need(q, "q", torch.bfloat16, dev)
    _need(k_pool, "k_pool", torch.bfloat16, dev)
    _need(v_pool, "v_pool", torch.bfloat16, dev)
    _need(block_table, "block_table", torch.int32, dev)
    _need(parents, "parents", torch.int32, dev)
    B, N, Hq, D = q.shape
    nblk, Hkv, ps, Dk = k_pool.shape
    if v_pool.shape != k_pool.shape or Dk != D or block_table.dim() != 2 or block_table.shape[0] != B \
            or tuple(parents.shape) != (B, N):
        raise ValueError("inconsistent shapes")
    if scale is None:
        scale = D ** -0.5
    out = torch.empty((B, N, Hq, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, N, Hq), dtype=torch.float32, device=dev) if want_lse else None
    ws_bytes = lib.eagle_tree_verify_attn_paged_workspace(B, N, Hq, Hkv, D, P, ps)
    if workspace is None and ws_bytes:
        workspace = _workspace(ws_bytes, dev)
    st = lib.eagle_tree_verify_attn_paged(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                          block_table.data_ptr(), parents.data_ptr(), B, N, Hq, Hkv,
                                          D, P, ps, block_table.shape[1], nblk, float(scale),
                                          EAGLE_BF16, out.data_ptr(), _ptr(lse), _ptr(workspace),
                                          0 if workspace is None else workspace.numel(), _stream())
    _check(st, "eagle_tree_verify_attn_paged")
    return out, lse


def eagle_tree_verify_attn_ragged(q, k, v, parents, prefix_len, tree_len, P: int, **kw):
    """eagle_tree_verify_attn with per-sequence prefix_len / tree_len (int32 [B])."""
    return eagle_tree_verify_attn(q, k, v, parents, P, prefix_len=prefix_len, tree_len=tree_len, **kw)


def eagle_lm_head_argmax(hidden: torch.Tensor, weight: torch.Tensor, want_logits: bool = False,
                         want_second: bool = True, workspace: Optional[torch.Tensor] = None):
    """hidden [M][H] bf16, weight [V][H] bf16.

    Returns dict(max, argmax, lse, second, logits) (second/logits may be None)."""
    lib = load()
    dev = hidden.device
    _need(hidden, "hidden", torch.bfloat16, dev)
    _need(weight, "weight", torch.bfloat16, dev)
    M, H = hidden.shape
    V = weight.shape[0]
    if weight.shape[1] != H:
        raise ValueError("hidden and weight disagree on H")
    f = dict(device=dev)
    res = {"max": torch.empty(M, dtype=torch.float32, **f),
           "argmax": torch.empty(M, dtype=torch.int32, **f),
           "lse": torch.empty(M, dtype=torch.float32, **f),
           "second": torch.empty(M, dtype=torch.float32, **f) if want_second else None,
           "logits": torch.empty((M, V), dtype=torch.float32, **f) if want_logits else None}
    if workspace is None:
        workspace = _workspace(lib.eagle_lm_head_workspace(M, H, V), dev)
    st = lib.eagle_lm_head_argmax(hidden.data_ptr(), weight.data_ptr(), M, H, V, EAGLE_BF16,
                                  res["max"].data_ptr(), res["argmax"].data_ptr(),
                                  res["lse"].data_ptr(), _ptr(res["second"]), _ptr(res["logits"]),
                                  workspace.data_ptr(), workspace.numel(), _stream())
    _check(st, "eagle_lm_head_argmax")
    return res


def eagle_accept_greedy(tokens: torch.Tensor, parents: torch.Tensor, target_argmax: torch.Tensor,
                        max_depth: int, tree_len: Optional[torch.Tensor] = None):
    """tokens, parents, target_argmax [B][N] int32 -> (accept_len [B], accept_path, out_tokens
    [B][max_depth+1]).  With tree_len (int32 [B]) eagle_accept_greedy_ragged is called."""
    lib = load()
    dev = tokens.device
    for t, n in ((tokens, "tokens"), (parents, "parents"), (target_argmax, "target_argmax")):
        _need(t, n, torch.int32, dev)
    B, N = tokens.shape
    if tuple(parents.shape) != (B, N) or tuple(target_argmax.shape) != (B, N):
        raise ValueError("inconsistent shapes")
    alen = torch.empty(B, dtype=torch.int32, device=dev)
    path = torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev)
    out = torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev)
    if tree_len is None:
        st = lib.eagle_accept_greedy(tokens.data_ptr(), parents.data_ptr(), target_argmax.data_ptr(),
                                     B, N, max_depth, alen.data_ptr(), path.data_ptr(),
                                     out.data_ptr(), _stream())
        _check(st, "eagle_accept_greedy")
        return alen, path, out
    _need(tree_len, "tree_len", torch.int32, dev)
    if tuple(tree_len.shape) != (B,):
        raise ValueError("tree_len must be [B]")
    st = lib.eagle_accept_greedy_ragged(tokens.data_ptr(), parents.data_ptr(),
                                        target_argmax.data_ptr(), tree_len.data_ptr(), B, N,
                                        max_depth, alen.data_ptr(), path.data_ptr(), out.data_ptr(),
                                        _stream())
    _check(st, "eagle_accept_greedy_ragged")
    return alen, path, out


def eagle_accept_greedy_ragged(tokens, parents, target_argmax, tree_len, max_depth: int):
    """eagle_accept_greedy with per-sequence tree sizes tree_len (int32 [B])."""
    return eagle_accept_greedy(tokens, parents, target_argmax, max_depth, tree_len=tree_len)


def eagle_kv_commit(k_cache: torch.Tensor, v_cache: torch.Tensor, accept_len: torch.Tensor,
                    accept_path: torch.Tensor, P: int) -> None:
    """In place: the accepted path's tree rows P + path[b][i] -> P + i in every layer.

    k_cache, v_cache bf16 [L][B][Hkv][kv_cap][D]; accept_len int32 [B];
    accept_path int32 [B][path_len]."""
    lib = load()
    dev = k_cache.device
    _need(k_cache, "k_cache", torch.bfloat16, dev)
    _need(v_cache, "v_cache", torch.bfloat16, dev)
    _need(accept_len, "accept_len", torch.int32, dev)
    _need(accept_path, "accept_path", torch.int32, dev)
    if k_cache.dim() != 5 or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache and v_cache must both be [L][B][Hkv][kv_cap][D]")
    L, B, Hkv, cap, D = k_cache.shape
    if tuple(accept_len.shape) != (B,) or accept_path.dim() != 2 or accept_path.shape[0] != B:
        raise ValueError("accept_len must be [B] and accept_path [B][path_len]")
    st = lib.eagle_kv_commit(k_cache.data_ptr(), v_cache.data_ptr(), accept_len.data_ptr(),
                             accept_path.data_ptr(), L, B, Hkv, D, P, cap, accept_path.shape[1],
                             _stream())
    _check(st, "eagle_kv_commit")


def eagle_accept_spec(tokens: torch.Tensor, parents: torch.Tensor, draft_row: torch.Tensor,
                      target_logits: torch.Tensor, draft_logits: torch.Tensor,
                      u_accept: torch.Tensor, u_sample: torch.Tensor, max_depth: int,
                      workspace: Optional[torch.Tensor] = None,
                      tree_len: Optional[torch.Tensor] = None, mode: str = "sampled",
                      target_lse: Optional[torch.Tensor] = None,
                      draft_lse: Optional[torch.Tensor] = None):
    """tokens, parents, draft_row [B][N] int32; target_logits [B][N][V] fp32;
    draft_logits [B][R][V] fp32; u_accept, u_sample [B][N] fp32; optional normalisers
    target_lse [B][N] and draft_lse [B][R] fp32 (the LM head's out_lse and the rerank's
    draft_lse).  With tree_len (int32 [B]) eagle_accept_spec_ragged is called.  mode:
    "sampled" (siblings drawn from the draft distribution) or "point_mass"
    (deterministic siblings)."""
    lib = load()
    if mode not in SPEC_MODES:
        raise ValueError(f"mode must be one of {sorted(SPEC_MODES)}")
    m = SPEC_MODES[mode]
    dev = tokens.device
    for t, n in ((tokens, "tokens"), (parents, "parents"), (draft_row, "draft_row")):
        _need(t, n, torch.int32, dev)
    for t, n in ((target_logits, "target_logits"), (draft_logits, "draft_logits"),
                 (u_accept, "u_accept"), (u_sample, "u_sample")):
        _need(t, n, torch.float32, dev)
    B, N = tokens.shape
    V = target_logits.shape[-1]
    R = draft_logits.shape[1]
    if tuple(target_logits.shape) != (B, N, V) or tuple(draft_logits.shape) != (B, R, V):
        raise ValueError("inconsistent logits shapes")
    for t, n, shape in ((target_lse, "target_lse", (B, N)), (draft_lse, "draft_lse", (B, R))):
        if t is not None:
            _need(t, n, torch.float32, dev)
            if tuple(t.shape) != shape:
                raise ValueError(f"{n} must be {list(shape)}")
    alen = torch.empty(B, dtype=torch.int32, device=dev)
    path = torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev)
    out = torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = _workspace(lib.eagle_accept_spec_workspace(B, N, V), dev)
    tail = (_ptr(target_logits), _ptr(target_lse), _ptr(draft_logits), _ptr(draft_lse),
            draft_row.data_ptr(), R, u_accept.data_ptr(), u_sample.data_ptr(), m,
            alen.data_ptr(), path.data_ptr(), out.data_ptr(), workspace.data_ptr(),
            workspace.numel(), _stream())
    if tree_len is None:
        st = lib.eagle_accept_spec(tokens.data_ptr(), parents.data_ptr(), B, N, V, max_depth, *tail)
        _check(st, "eagle_accept_spec")
        return alen, path, out
    _need(tree_len, "tree_len", torch.int32, dev)
    if tuple(tree_len.shape) != (B,):
        raise ValueError("tree_len must be [B]")
    st = lib.eagle_accept_spec_ragged(tokens.data_ptr(), parents.data_ptr(), tree_len.data_ptr(),
                                      B, N, V, max_depth, *tail)
    _check(st, "eagle_accept_spec_ragged")
    return alen, path, out


def eagle_accept_spec_ragged(tokens, parents, draft_row, target_logits, draft_logits, u_accept,
                             u_sample, tree_len, max_depth: int, workspace=None,
                             mode: str = "sampled", target_lse=None, draft_lse=None):
    """eagle_accept_spec with per-sequence tree sizes tree_len (int32 [B])."""
    return eagle_accept_spec(tokens, parents, draft_row, target_logits, draft_logits, u_accept,
                             u_sample, max_depth, workspace=workspace, tree_len=tree_len, mode=mode,
                             target_lse=target_lse, draft_lse=draft_lse)


def eagle2_rerank(draft_logits: torch.Tensor, root_token: torch.Tensor, top_k: int, depth: int,
                  n_nodes: int, workspace: Optional[torch.Tensor] = None):
    """draft_logits [B][R][V] fp32 (R = 1 + (depth-1)*top_k); root_token [B] int32.

    Returns dict(tokens, parents, depths, scores, draft_row, draft_lse)."""
    lib = load()
    dev = draft_logits.device
    _need(draft_logits, "draft_logits", torch.float32, dev)
    _need(root_token, "root_token", torch.int32, dev)
    B, R, V = draft_logits.shape
    if R != 1 + (depth - 1) * top_k:
        raise ValueError(f"draft_logits has {R} rows, expected {1 + (depth - 1) * top_k}")
    f = dict(device=dev)
    res = {"tokens": torch.empty((B, n_nodes), dtype=torch.int32, **f),
           "parents": torch.empty((B, n_nodes), dtype=torch.int32, **f),
           "depths": torch.empty((B, n_nodes), dtype=torch.int32, **f),
           "scores": torch.empty((B, n_nodes), dtype=torch.float32, **f),
           "draft_row": torch.empty((B, n_nodes), dtype=torch.int32, **f),
           "draft_lse": torch.empty((B, R), dtype=torch.float32, **f)}
    if workspace is None:
        workspace = _workspace(lib.eagle2_rerank_workspace(B, V, top_k, depth), dev)
    st = lib.eagle2_rerank(draft_logits.data_ptr(), root_token.data_ptr(), B, V, top_k, depth,
                           n_nodes, res["tokens"].data_ptr(), res["parents"].data_ptr(),
                           res["depths"].data_ptr(), res["scores"].data_ptr(),
                           res["draft_row"].data_ptr(), res["draft_lse"].data_ptr(),
                           workspace.data_ptr(), workspace.numel(), _stream())
    _check(st, "eagle2_rerank")
    return res


DRAFT_HEAD_KEYS = ("embed", "w_fc", "w_qkv", "w_o", "w_gate_up", "w_down", "w_lm")


def eagle_draft_expand_workspace(B, H, Hq, Hkv, D, I, V, P, kv_cap, top_k, depth) -> int:
    return load().eagle_draft_expand_workspace(B, H, Hq, Hkv, D, I, V, P, kv_cap, top_k, depth)


def eagle_draft_expand(head: dict, f0: torch.Tensor, root_token: torch.Tensor, k_cache: torch.Tensor,
                       v_cache: torch.Tensor, P: int, Hq: int, top_k: int, depth: int, n_nodes: int,
                       scale: float, eps: float, workspace: Optional[torch.Tensor] = None,
                       out: Optional[dict] = None):
    """Per-depth EAGLE-2 draft expansion with a one-layer draft head.

    head: dict of device tensors embed [V][H], w_fc [H][2H], w_qkv [(Hq+2Hkv)D][H],
    w_o [H][Hq D], w_gate_up [2I][H], w_down [H][I], w_lm [V][H] (bf16) and g1, g2 [H]
    (fp32).  f0 [B][H] bf16; root_token [B] int32; k_cache, v_cache [B][Hkv][kv_cap][D]
    bf16 (rows P.. are overwritten).  Returns dict(tokens, parents, depths, scores,
    draft_row, draft_logits, draft_lse, features, row_token, parent_row)."""
    lib = load()
    dev = f0.device
    for name in DRAFT_HEAD_KEYS:
        _need(head[name], name, torch.bfloat16, dev)
    for name in ("g1", "g2"):
        _need(head[name], name, torch.float32, dev)
    _need(f0, "f0", torch.bfloat16, dev)
    _need(root_token, "root_token", torch.int32, dev)
    _need(k_cache, "k_cache", torch.bfloat16, dev)
    _need(v_cache, "v_cache", torch.bfloat16, dev)
    B, H = f0.shape
    V = head["embed"].shape[0]
    I = head["w_down"].shape[1]
    _, Hkv, kv_cap, D = k_cache.shape
    R = 1 + (depth - 1) * top_k
    f = dict(device=dev)
    res = out if out is not None else {
        "tokens": torch.empty((B, n_nodes), dtype=torch.int32, **f),
        "parents": torch.empty((B, n_nodes), dtype=torch.int32, **f),
        "depths": torch.empty((B, n_nodes), dtype=torch.int32, **f),
        "scores": torch.empty((B, n_nodes), dtype=torch.float32, **f),
        "draft_row": torch.empty((B, n_nodes), dtype=torch.int32, **f),
        "draft_logits": torch.empty((B, R, V), dtype=torch.float32, **f),
        "draft_lse": torch.empty((B, R), dtype=torch.float32, **f),
        "features": torch.empty((B, R, H), dtype=torch.bfloat16, **f),
        "row_token": torch.empty((B, R), dtype=torch.int32, **f),
        "parent_row": torch.empty((B, R), dtype=torch.int32, **f)}
    if workspace is None:
        workspace = _workspace(lib.eagle_draft_expand_workspace(B, H, Hq, Hkv, D, I, V, P, kv_cap,
                                                                top_k, depth), dev)
    hd = DraftHead(*[head[k].data_ptr() for k in DRAFT_HEAD_KEYS + ("g1", "g2")])
    st = lib.eagle_draft_expand(ctypes.byref(hd), f0.data_ptr(), root_token.data_ptr(),
                                k_cache.data_ptr(), v_cache.data_ptr(), B, H, Hq, Hkv, D, I, V, P,
                                kv_cap, top_k, depth, n_nodes, scale, eps, res["tokens"].data_ptr(),
                                res["parents"].data_ptr(), res["depths"].data_ptr(),
                                res["scores"].data_ptr(), res["draft_row"].data_ptr(),
                                res["draft_logits"].data_ptr(), res["draft_lse"].data_ptr(),
                                res["features"].data_ptr(), res["row_token"].data_ptr(),
                                res["parent_row"].data_ptr(), workspace.data_ptr(),
                                workspace.numel(), _stream())
    _check(st, "eagle_draft_expand")
    return res


def eagle_calib_stream_read(src: torch.Tensor) -> None:
    """Read the device tensor `src` once (streaming-read bandwidth probe)."""
    lib = load()
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    sink = torch.empty(4096, dtype=torch.int32, device=src.device)
    nbytes = src.numel() * src.element_size() // 16 * 16
    _check(lib.eagle_calib_stream_read(src.data_ptr(), nbytes, sink.data_ptr(), _stream()),
           "eagle_calib_stream_read")


def eagle_calib_mfma_bf16(iters: int, out: Optional[torch.Tensor] = None) -> float:
    """Run the bf16 matrix-core loop once; returns its flop count."""
    lib = load()
    if out is None:
        out = torch.empty(2048 * 256, dtype=torch.float32, device="cuda")
    _check(lib.eagle_calib_mfma_bf16(iters, out.data_ptr(), out.numel(), _stream()),
           "eagle_calib_mfma_bf16")
    return lib.eagle_calib_mfma_bf16_flops(iters)
