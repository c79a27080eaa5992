"""Chunked, order-independent seeded generators (see package docstring)."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22  # elements per independently seeded chunk


def _rng(seed: int, cfg: int, tensor: int, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cfg, tensor, chunk])))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _fill_chunked(out: np.ndarray, seed: int, cfg: int, tensor: int, fill) -> np.ndarray:
    flat = out.reshape(-1)
    n_chunks = (flat.size + CHUNK - 1) // CHUNK

    def work(i: int) -> None:
        seg = flat[i * CHUNK:(i + 1) * CHUNK]
        fill(_rng(seed, cfg, tensor, i), seg)

    if n_chunks <= 1:
        for i in range(n_chunks):
            work(i)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(n_chunks)))
    return out


def round_f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = b + (((b >> 16) & np.uint32(1)) + np.uint32(0x7FFF))
    return (r >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


def normal_bf16_bits(shape, std: float, seed: int, cfg: int, tensor: int) -> np.ndarray:
    """N(0, std^2) drawn in fp32, rounded once to bf16; returned as uint16 bits."""
    out = np.empty(shape, dtype=np.uint16)
    flat_out = out.reshape(-1)
    n_chunks = (flat_out.size + CHUNK - 1) // CHUNK
    s = np.float32(std)

    def work(i: int) -> None:
        seg_out = flat_out[i * CHUNK:(i + 1) * CHUNK]
        seg = np.empty(seg_out.size, dtype=np.float32)
        _rng(seed, cfg, tensor, i).standard_normal(out=seg, dtype=np.float32)
        if std != 1.0:
            seg *= s
        seg_out[...] = round_f32_to_bf16_bits(seg)

    if n_chunks <= 1:
        for i in range(n_chunks):
            work(i)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(n_chunks)))
    return out


def normal_f32(shape, std: float, seed: int, cfg: int, tensor: int) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    s = np.float32(std)

    def fill(g, seg):
        g.standard_normal(out=seg, dtype=np.float32)
        if std != 1.0:
            seg *= s

    return _fill_chunked(out, seed, cfg, tensor, fill)


def uniform_f32(shape, seed: int, cfg: int, tensor: int) -> np.ndarray:
    """U[0, 1) in fp32."""
    out = np.empty(shape, dtype=np.float32)

    def fill(g, seg):
        g.random(out=seg, dtype=np.float32)

    return _fill_chunked(out, seed, cfg, tensor, fill)


def integers(shape, low: int, high: int, seed: int, cfg: int, tensor: int) -> np.ndarray:
    """Uniform int32 in [low, high)."""
    out = np.empty(shape, dtype=np.int32)

    def fill(g, seg):
        seg[...] = g.integers(low, high, size=seg.size, dtype=np.int32)

    return _fill_chunked(out, seed, cfg, tensor, fill)


def plant_tokens(parents: np.ndarray, parent_argmax: np.ndarray, prob: float, vocab: int,
                 seed: int, cfg: int, tensor: int) -> np.ndarray:
    """Draft tokens for a fixed tree: node i gets ``parent_argmax[b, parents[b, i]]``
    with probability ``prob``, else a uniform token; node 0 (the root) gets a uniform
    token.  ``parent_argmax`` is supplied by the caller (it is the target's top-1 per
    node); this function only mixes it with noise.
    """
    parents = np.asarray(parents, dtype=np.int64)
    B, N = parents.shape
    u = uniform_f32((B, N), seed, cfg, tensor)
    rnd = integers((B, N), 0, vocab, seed, cfg, tensor + 1000)
    tok = rnd.copy()
    for b in range(B):
        for i in range(1, N):
            if u[b, i] < prob:
                tok[b, i] = parent_argmax[b, parents[b, i]]
    return tok.astype(np.int32)


def random_parents(B: int, N: int, seed: int, cfg: int, tensor: int) -> np.ndarray:
    """B random trees of N nodes: parents[b][0] = -1, parents[b][i] uniform in [0, i)."""
    u = uniform_f32((B, N), seed, cfg, tensor).astype(np.float64)
    par = np.floor(u * np.arange(N)[None, :]).astype(np.int32)
    par = np.minimum(par, np.maximum(np.arange(N)[None, :] - 1, 0)).astype(np.int32)
    par[:, 0] = -1
    return par


def chain_parents(B: int, N: int) -> np.ndarray:
    return np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
