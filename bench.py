#!/usr/bin/env python3
"""Benchmark of one EAGLE-2 tree-verification step on one MI355X.

A step is the whole hot path over one batch of synthetic input at the
Llama-3-70B-shaped workload (4 sequences, 60-node EAGLE-2 trees, 64 query / 8 KV
heads, head dim 128, 32768-token KV prefix, hidden 8192, vocabulary 128256, bf16):

    eagle2_rerank          -> tree (tokens, parents, draft rows) from draft logits
    eagle_tree_verify_attn -> one layer of tree attention over prefix + tree
    eagle_lm_head_argmax   -> LM head + per-node max/argmax/lse over the tree's hidden states
    eagle_accept_greedy    -> accepted path and emitted tokens

Inputs are resident in HBM before timing.  Every step streams 2.1 GB of LM-head
weights, 538 MB of KV and 105 MB of draft logits, more than the 256 MB Infinity
Cache, so nothing is served warm from one step to the next.

Prints ONE JSON line.  `value` is tree-verify tokens/s = B*N tree tokens verified
per step / step time.  The per-kernel breakdown, the roofline of the dominant
kernel (LM head, HBM-bound) and of the attention kernel, the speculative-sampling
acceptance latency at the Llama-3-8B-shaped workload and the timed CPU oracle
baseline are added as extra fields.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
METRIC = "tree-verify tokens/s + HBM GB/s (% peak) at 8B/70B shapes; accept+rerank µs"
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "lm_head": "speculative_decoding_attn_amd/csrc/lm_head.hip",
    "tree_attn": "speculative_decoding_attn_amd/csrc/tree_attn.hip",
}


COMMON_HEADER = "speculative_decoding_attn_amd/csrc/common.h"


def _src_hash(rel: str) -> str:
    """Hash of a kernel source together with the device header it includes."""
    h = hashlib.sha256()
    for path in (rel, COMMON_HEADER):
        with open(os.path.join(ROOT, path), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None if
    the summary is missing or was taken on a different kernel source."""
    path = os.path.join(PROFILE_DIR, f"{kernel}_C5_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256_16") != _src_hash(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("bytes_per_launch")


def make_inputs(cfg, torch, dev):
    """Synthetic C5 inputs as device tensors (bf16 where the GPU reads bf16)."""
    B, N, Hq, Hkv, D, P, H, V = cfg.B, cfg.N, cfg.Hq, cfg.Hkv, cfg.D, cfg.P, cfg.H, cfg.V

    def dbf(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    x = {}
    x["q"] = dbf(synth.normal_bf16_bits((B, N, Hq, D), 1.0, 0, cfg.index, 1))
    x["k"] = dbf(synth.normal_bf16_bits((B, Hkv, P + N, D), 1.0, 0, cfg.index, 2))
    x["v"] = dbf(synth.normal_bf16_bits((B, Hkv, P + N, D), 1.0, 0, cfg.index, 3))
    x["hidden"] = dbf(synth.normal_bf16_bits((B * N, H), 1.0, 0, cfg.index, 4))
    x["W"] = dbf(synth.normal_bf16_bits((V, H), cfg.w_std, 0, cfg.index, 5))
    if cfg.rows:
        x["draft_logits"] = torch.from_numpy(
            synth.normal_f32((B, cfg.rows, V), cfg.draft_std, 0, cfg.index, 6)).to(dev)
    x["root"] = torch.from_numpy(synth.integers((B,), 0, V, 0, cfg.index, 7)).to(dev)
    return x


def attn_bytes(cfg) -> int:
    """Algorithmic HBM bytes of one tree-attention call: K and V of every (sequence, KV
    head) over prefix + tree once, q and out (bf16), lse (fp32)."""
    B, N, Hq, Hkv, D, P = cfg.B, cfg.N, cfg.Hq, cfg.Hkv, cfg.D, cfg.P
    return 2 * B * Hkv * (P + N) * D * 2 + 2 * B * N * Hq * D * 2 + B * N * Hq * 4


def lm_bytes(M, H, V, logits=False) -> int:
    """Algorithmic HBM bytes of one LM-head call: W and the hidden rows once, 16 bytes of
    row statistics per row, plus the fp32 logits when they are written."""
    return V * H * 2 + M * H * 2 + M * 16 + (M * V * 4 if logits else 0)


def roof(us, nbytes, nflops=None):
    """HBM and bf16-MFMA fractions of nominal peak for `nbytes` / `nflops` in `us`."""
    out = {"us": round(us, 2), "hbm_gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
           "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    if nflops is not None:
        tf = nflops / (us * 1e-6) / 1e12
        out.update({"mfma_tflops": round(tf, 1), "mfma_frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4)})
    return out


def attn_flops(parents_np, cfg) -> float:
    """Algorithmic flops of tree attention: 2*D for q.k and 2*D for p*v per (query, key);
    node i of depth d sees P + d + 1 keys."""
    total_keys = 0
    for b in range(parents_np.shape[0]):
        depth = [0] * cfg.N
        for i in range(1, cfg.N):
            depth[i] = depth[parents_np[b, i]] + 1
        total_keys += sum(cfg.P + d + 1 for d in depth)
    return 4.0 * cfg.D * cfg.Hq * total_keys


def _host_info():
    """The host the CPU baseline ran on: CPU model, cores this process may use, cores
    in the machine."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return {"cpu_model": model, "usable_cores": usable, "machine_cores": os.cpu_count()}


def cpu_baseline(cfg, n_pairs=6, n_slices=24, n_rerank=2):
    """Time the fp64 oracle on a bounded sample of the C5 step and scale to one step."""
    import oracle
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:  # pragma: no cover
        threads = 1
    B, N, Hq, Hkv, D, P, H, V = cfg.B, cfg.N, cfg.Hq, cfg.Hkv, cfg.D, cfg.P, cfg.H, cfg.V
    G = Hq // Hkv
    f64 = synth.bf16_bits_to_f64
    slice_rows = (V + 63) // 64

    # attention: n_pairs of the B*Hkv (sequence, KV head) pairs, all nodes and heads
    parents = synth.random_parents(B, N, 0, cfg.index, 20)
    t_attn = 0.0
    for j in range(n_pairs):
        b, g = j % B, (j * 3) % Hkv
        qb = synth.normal_bf16_bits((N, G, D), 1.0, 0, cfg.index, 1001 + j)
        kb = synth.normal_bf16_bits((P + N, D), 1.0, 0, cfg.index, 1101 + j)
        vb = synth.normal_bf16_bits((P + N, D), 1.0, 0, cfg.index, 1201 + j)
        q, k, v = f64(qb), f64(kb), f64(vb)
        anc = oracle.ancestor_sets(parents[b])
        t0 = time.perf_counter()
        for i in range(N):
            oracle.tree_verify_attention_node(q[i], k, v, anc[i], P, D ** -0.5)
        t_attn += time.perf_counter() - t0
    t_attn *= (B * Hkv) / n_pairs

    # LM head: n_slices vocabulary slices of 1/64 of the vocabulary, all rows
    hidden = f64(synth.normal_bf16_bits((B * N, H), 1.0, 0, cfg.index, 4))
    t_lm = 0.0
    for j in range(n_slices):
        wb = synth.normal_bf16_bits((slice_rows, H), cfg.w_std, 0, cfg.index, 1301 + j)
        t0 = time.perf_counter()
        lg = oracle.lm_head_logits(hidden, wb, to_f64=f64)
        oracle.lm_head_row_stats(lg)
        t_lm += time.perf_counter() - t0
    t_lm *= 64.0 / n_slices

    # rerank: n_rerank sequences
    t_rr = 0.0
    for j in range(n_rerank):
        dl = synth.normal_f32((cfg.rows, V), cfg.draft_std, 0, cfg.index, 1401 + j)
        t0 = time.perf_counter()
        oracle.eagle2_rerank(dl, 1, cfg.top_k, cfg.depth, N)
        t_rr += time.perf_counter() - t0
    t_rr *= B / n_rerank

    # greedy acceptance: all sequences
    t0 = time.perf_counter()
    for b in range(B):
        oracle.accept_greedy(np.zeros(N, np.int64), parents[b], np.zeros(N, np.int64), cfg.max_depth)
    t_acc = time.perf_counter() - t0

    step = t_attn + t_lm + t_rr + t_acc
    return {"value": round(B * N / step, 3), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "host": _host_info(),
            "sample": (f"fp64 numpy oracle on {n_pairs}/{B * Hkv} attention (sequence, KV head) "
                       f"pairs, {n_slices}/64 LM-head vocabulary slices, {n_rerank}/{B} rerank "
                       f"sequences and all {B} greedy acceptances of the C5 step, each scaled "
                       f"to the full step"),
            "step_seconds": round(step, 3),
            "parts_seconds": {"tree_attn": round(t_attn, 3), "lm_head": round(t_lm, 3),
                              "rerank": round(t_rr, 3), "accept_greedy": round(t_acc, 4)}}


def cpu_baseline_single_thread(cfg):
    """The same oracle sample, smaller (1 of 32 attention pairs, 4 of 64 LM-head slices,
    1 rerank sequence), with the BLAS pool limited to one thread."""
    try:
        import threadpoolctl
    except Exception:  # pragma: no cover
        return None
    with threadpoolctl.threadpool_limits(limits=1):
        r = cpu_baseline(cfg, n_pairs=1, n_slices=4, n_rerank=1)
    r["cores"] = 1
    return r


def copy_calibration(torch, dev, nbytes=1 << 30, reps=5):
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters;
    also prints the copy's rate (bytes read + written per second)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(s)
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1000.0 / reps
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps,
                      "copy_gbs_read_plus_write": round(2 * nbytes / sec / 1e9, 1)}))


def _window_ms(torch, fn, n):
    """Mean event time (ms) of n back-to-back calls of fn, with one event before the
    first and one after the last (nothing recorded in between)."""
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(n):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def _warm(torch, fn, seconds=0.25, min_calls=3):
    """Untimed calls of fn until the GPU has run this workload for about `seconds`.  The
    chip's power management runs a fresh load fast for its first milliseconds, then
    throttles hard and settles over the next few tens of milliseconds (a C5 step: 0.91 ms
    over its first 50 steps, then 0.79-0.81 ms, flat over 10 s), so every timed window
    starts in the settled state."""
    n = 0
    t0 = time.perf_counter()
    while n < min_calls or time.perf_counter() - t0 < seconds:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def measured_ceilings(torch, sda, dev, read_bytes=4 << 30, reps=10, mfma_iters=20000):
    """What this GPU reaches, next to the nominal peaks: a streaming HBM read of a 4 GiB
    buffer (the library's read probe, 16-byte non-temporal loads), a 1 GiB device copy
    (torch), and the bf16 matrix-core loop (the library's probe: 8192 waves, four
    independent 32x32x16 MFMA chains each).  Event-timed on the launch stream."""
    s = torch.cuda.current_stream()

    def timed(fn, n):
        _warm(torch, fn, seconds=0.15, min_calls=1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(n):
            fn()
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1000.0 / n

    buf = torch.ones(read_bytes // 2, dtype=torch.bfloat16, device=dev)
    t_read = timed(lambda: sda.eagle_calib_stream_read(buf), reps)
    del buf
    src = torch.ones(1 << 29, dtype=torch.int16, device=dev)
    dst = torch.empty_like(src)
    t_copy = timed(lambda: dst.copy_(src), reps)
    del src, dst
    out = torch.empty(2048 * 256, dtype=torch.float32, device=dev)
    flops = sda.eagle_calib_mfma_bf16(mfma_iters, out)
    t_mfma = timed(lambda: sda.eagle_calib_mfma_bf16(mfma_iters, out), 3)
    torch.cuda.empty_cache()
    rd = read_bytes / t_read / 1e9
    cp = 2 * (1 << 30) / t_copy / 1e9
    mf = flops / t_mfma / 1e12
    return {"stream_read_gbs": round(rd, 1), "stream_read_frac_of_peak": round(rd / HBM_PEAK_GBS, 4),
            "copy_gbs_read_plus_write": round(cp, 1),
            "mfma_bf16_tflops": round(mf, 1), "mfma_bf16_frac_of_peak": round(mf / BF16_MFMA_PEAK_TFLOPS, 4),
            "how": "4 GiB streaming read (eagle_calib_stream_read), 1 GiB device copy, "
                   f"{mfma_iters}-step bf16 MFMA loop (eagle_calib_mfma_bf16); mean of {reps} / 3 runs"}


def lm_head_back_to_back(torch, sda, dev, x, iters=20):
    """The C5 LM head alone, launched back to back (nothing in between): W (2.1 GB)
    streams from HBM on every call, as inside the step."""
    cfg = synth.CONFIGS["C5"]
    M, H, V = cfg.B * cfg.N, cfg.H, cfg.V
    ws = torch.empty(sda.load().eagle_lm_head_workspace(M, H, V), dtype=torch.uint8, device=dev)
    _warm(torch, lambda: sda.eagle_lm_head_argmax(x["hidden"], x["W"], want_logits=False, workspace=ws))
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(iters):
        sda.eagle_lm_head_argmax(x["hidden"], x["W"], want_logits=False, workspace=ws)
    e1.record(s)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / iters
    return dict(roof(us, lm_bytes(M, H, V), 2.0 * M * H * V), calls=iters)


def config_step(torch, sda, dev, name, steps=50):
    """One verification step at another of the five workloads, each call timed with HIP
    events on the launch stream:
      C2  static EAGLE-1 tree: attention -> LM head -> greedy acceptance
      C3  eagle2_rerank -> attention -> LM head -> greedy acceptance
      C4  eagle2_rerank -> attention -> LM head (fp32 logits written) -> speculative
          acceptance (sampled siblings) fed the LM head's out_lse and the rerank's
          draft_lse
    tokens/s = B*N tree tokens / step time; per kernel the HBM and bf16-MFMA fractions
    of the nominal peaks (algorithmic bytes and flops)."""
    cfg = synth.CONFIGS[name]
    B, N, Hq, Hkv, D, P, H, V = cfg.B, cfg.N, cfg.Hq, cfg.Hkv, cfg.D, cfg.P, cfg.H, cfg.V
    x = make_inputs(cfg, torch, dev)
    lib = sda.load()
    spec = cfg.accept == "spec"
    ws_attn = torch.empty(max(1, lib.eagle_tree_verify_attn_workspace(B, N, Hq, Hkv, D, P)),
                          dtype=torch.uint8, device=dev)
    ws_lm = torch.empty(lib.eagle_lm_head_workspace(B * N, H, V), dtype=torch.uint8, device=dev)
    attn_out = torch.empty((B, N, Hq, D), dtype=torch.bfloat16, device=dev)
    attn_lse = torch.empty((B, N, Hq), dtype=torch.float32, device=dev)
    static = None
    if cfg.parents is not None:
        static = {"parents": torch.tensor([cfg.parents] * B, dtype=torch.int32, device=dev),
                  "tokens": torch.from_numpy(synth.integers((B, N), 0, V, 0, cfg.index, 21)).to(dev)}
    else:
        ws_rr = torch.empty(lib.eagle2_rerank_workspace(B, V, cfg.top_k, cfg.depth), dtype=torch.uint8,
                            device=dev)
    if spec:
        ua = torch.from_numpy(synth.uniform_f32((B, N), 0, cfg.index, 8)).to(dev)
        us = torch.from_numpy(synth.uniform_f32((B, N), 0, cfg.index, 9)).to(dev)
        ws_sp = torch.empty(lib.eagle_accept_spec_workspace(B, N, V), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    names = (["rerank"] if static is None else []) + ["tree_attn", "lm_head",
                                                      "accept_spec" if spec else "accept_greedy"]

    def step(ev=None):
        k = 0
        if ev:
            ev[k].record(stream)
        if static is None:
            tree = sda.eagle2_rerank(x["draft_logits"], x["root"], cfg.top_k, cfg.depth, N,
                                     workspace=ws_rr)
            k += 1
            if ev:
                ev[k].record(stream)
        else:
            tree = static
        sda.eagle_tree_verify_attn(x["q"], x["k"], x["v"], tree["parents"], P, D ** -0.5,
                                   out=attn_out, lse=attn_lse, workspace=ws_attn)
        k += 1
        if ev:
            ev[k].record(stream)
        res = sda.eagle_lm_head_argmax(x["hidden"], x["W"], want_logits=spec, workspace=ws_lm)
        k += 1
        if ev:
            ev[k].record(stream)
        if spec:
            acc = sda.eagle_accept_spec(tree["tokens"], tree["parents"], tree["draft_row"],
                                        res["logits"].view(B, N, V), x["draft_logits"], ua, us,
                                        cfg.max_depth, workspace=ws_sp,
                                        target_lse=res["lse"].view(B, N), draft_lse=tree["draft_lse"])
        else:
            acc = sda.eagle_accept_greedy(tree["tokens"], tree["parents"], res["argmax"].view(B, N),
                                          cfg.max_depth)
        k += 1
        if ev:
            ev[k].record(stream)
        return tree, acc

    last = {}
    _warm(torch, lambda: last.update(r=step()))
    tree, acc = last["r"]
    parents_np = tree["parents"].cpu().numpy()
    alen = acc[0].cpu().numpy()
    # step time from a window with no events inside; the per-call times from a second
    # window with an event between the calls
    ms = _window_ms(torch, step, steps)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    per = {n: 1000.0 * sum(e[j].elapsed_time(e[j + 1]) for e in evs) / steps
           for j, n in enumerate(names)}
    kern = {"tree_attn": roof(per["tree_attn"], attn_bytes(cfg), attn_flops(parents_np, cfg)),
            "lm_head": roof(per["lm_head"], lm_bytes(B * N, H, V, logits=spec), 2.0 * B * N * H * V)}
    if static is None:
        kern["rerank"] = roof(per["rerank"], B * cfg.rows * V * 4)
    del x
    torch.cuda.empty_cache()
    return {"workload": (f"{name}: B={B} Hq={Hq} Hkv={Hkv} D={D} P={P} N={N} H={H} V={V}, "
                         + ("static EAGLE-1 tree" if static is not None else
                            f"EAGLE-2 tree (top-k {cfg.top_k}, depth {cfg.depth})")
                         + (", speculative sampling" if spec else ", greedy")),
            "tokens_per_s": round(B * N / (ms / 1000.0), 1), "ms_per_step": round(ms, 4),
            "breakdown_us": {k: round(v, 2) for k, v in per.items()}, "kernels": kern,
            "accept_len": [int(a) for a in alen]}


def spec_latency(torch, sda, dev, iters=100, mode="sampled", with_lse=True):
    """eagle_accept_spec at the Llama-3-8B-shaped speculative-sampling workload (C4): a
    60-node tree from eagle2_rerank, target logits N(0,1) over 128256 tokens.  mode
    "sampled" runs the pages' rule with the draft distribution (10 residual rounds at
    the root), "point_mass" the rule for deterministic top-k siblings.  with_lse hands
    the rows' normalisers over (as the LM head and the rerank produce them); without,
    the kernel forms them itself."""
    cfg = synth.CONFIGS["C4"]
    dl = torch.from_numpy(synth.normal_f32((1, cfg.rows, cfg.V), cfg.draft_std, 0, cfg.index, 6)).to(dev)
    root = torch.from_numpy(synth.integers((1,), 0, cfg.V, 0, cfg.index, 7)).to(dev)
    tree = sda.eagle2_rerank(dl, root, cfg.top_k, cfg.depth, cfg.N)
    tl = torch.from_numpy(synth.normal_f32((1, cfg.N, cfg.V), 1.0, 0, cfg.index, 10)).to(dev)
    ua = torch.from_numpy(synth.uniform_f32((1, cfg.N), 0, cfg.index, 8)).to(dev)
    us = torch.from_numpy(synth.uniform_f32((1, cfg.N), 0, cfg.index, 9)).to(dev)
    ws = torch.empty(sda.load().eagle_accept_spec_workspace(1, cfg.N, cfg.V), dtype=torch.uint8,
                     device=dev)
    lse = {}
    if with_lse:
        lse = {"target_lse": torch.logsumexp(tl.double(), dim=-1).float().contiguous(),
               "draft_lse": tree["draft_lse"]}

    def call():
        sda.eagle_accept_spec(tree["tokens"], tree["parents"], tree["draft_row"], tl, dl, ua, us,
                              cfg.max_depth, workspace=ws, mode=mode, **lse)

    _warm(torch, call)
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(iters):
        call()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1000.0 / iters


def kv_commit_latency(torch, sda, dev, parents, iters=50, layers=80):
    """eagle_kv_commit over the caches of every layer of a Llama-3-70B-shaped model
    (80 layers x 4 sequences x 8 KV heads x head dim 128) after accepting, in each
    sequence, the root path of the tree's deepest node.  The commit only touches rows
    P .. P+N, so the caches hold a short prefix (P = 64) plus the 60 tree rows."""
    cfg = synth.CONFIGS["C5"]
    B, N, Hkv, D, P = cfg.B, cfg.N, cfg.Hkv, cfg.D, 64
    par = parents.cpu().numpy()
    maxd = cfg.max_depth
    alen = np.zeros(B, dtype=np.int32)
    path = np.full((B, maxd + 1), -1, dtype=np.int32)
    for b in range(B):
        depth = [0] * N
        for i in range(1, N):
            depth[i] = depth[par[b, i]] + 1
        node = max(range(N), key=lambda i: (min(depth[i], maxd), -i) if depth[i] <= maxd else (-1, 0))
        chain = [node]
        while chain[-1] != 0:
            chain.append(int(par[b, chain[-1]]))
        chain.reverse()
        alen[b] = len(chain) - 1
        path[b, :len(chain)] = chain
    shape = (layers, B, Hkv, P + N, D)
    k = torch.empty(shape, dtype=torch.bfloat16, device=dev).normal_()
    v = torch.empty(shape, dtype=torch.bfloat16, device=dev).normal_()
    a = torch.from_numpy(alen).to(dev)
    p = torch.from_numpy(path).to(dev)
    _warm(torch, lambda: sda.eagle_kv_commit(k, v, a, p, P))
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(iters):
        sda.eagle_kv_commit(k, v, a, p, P)
    e1.record(s)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / iters
    moved = 2 * 2 * layers * Hkv * D * 2 * int((alen + 1).sum())   # K and V, read + write
    return {"us": round(us, 2), "layers": layers, "accepted_rows_per_seq": [int(x) + 1 for x in alen],
            "bytes": moved, "gbs": round(moved / (us * 1e-6) / 1e9, 1)}


def paged_attention(torch, sda, dev, x, parents, page_size=16, iters=20):
    """Tree attention at C5 with the KV cache in pages of `page_size` rows scattered
    over a pool by a seeded permutation (the same rows as the contiguous cache)."""
    cfg = synth.CONFIGS["C5"]
    B, N, Hkv, D, P = cfg.B, cfg.N, cfg.Hkv, cfg.D, cfg.P
    L = P + N
    pages = (L + page_size - 1) // page_size
    nblk = B * pages
    perm = torch.from_numpy(np.random.default_rng(5).permutation(nblk).astype(np.int64)).to(dev)
    table = perm.view(B, pages).to(torch.int32).contiguous()

    def pool_of(c):
        pad = torch.zeros((B, Hkv, pages * page_size - L, D), dtype=c.dtype, device=dev)
        blocks = torch.cat([c, pad], dim=2).view(B, Hkv, pages, page_size, D).permute(0, 2, 1, 3, 4)
        pool = torch.empty((nblk, Hkv, page_size, D), dtype=c.dtype, device=dev)
        pool[perm] = blocks.reshape(nblk, Hkv, page_size, D)
        return pool

    kp, vp = pool_of(x["k"]), pool_of(x["v"])
    ws = torch.empty(max(1, sda.load().eagle_tree_verify_attn_paged_workspace(
        B, N, cfg.Hq, Hkv, D, P, page_size)), dtype=torch.uint8, device=dev)
    _warm(torch, lambda: sda.eagle_tree_verify_attn_paged(x["q"], kp, vp, table, parents, P, workspace=ws))
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(iters):
        sda.eagle_tree_verify_attn_paged(x["q"], kp, vp, table, parents, P, workspace=ws)
    e1.record(s)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / iters
    del kp, vp
    return {"page_size": page_size, "us": round(us, 2)}


# untimed expansions after the first (about 0.2 s of work at C5: past the power
# transient, see _warm)
DRAFT_WARMUP = 40

DRAFT_SHAPES = {
    # name: (B, H, Hq, Hkv, D, I, V, P)  draft head = one decoder layer of the target family
    "C3": (1, 4096, 32, 8, 128, 14336, 128256, 4096),
    "C5": (4, 8192, 64, 8, 128, 28672, 128256, 32768),
}


def draft_expansion(torch, sda, dev, name="C5", top_k=10, depth=6, n_nodes=60, iters=3):
    """Per-depth EAGLE-2 draft expansion (eagle_draft_expand) with a one-layer draft head
    of the target family's shape (random bf16 weights drawn on the device, seeded) over
    a draft prefix of P rows.  Reports the time of one whole expansion and the weight
    bytes it streams: every depth reads W_fc, W_qkv, W_o, W_gate_up, W_down and the LM
    head once."""
    B, H, Hq, Hkv, D, I, V, P = DRAFT_SHAPES[name]
    R = 1 + (depth - 1) * top_k
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)

    def w(rows, cols, std):
        return (torch.randn((rows, cols), generator=gen, device=dev) * std).to(torch.bfloat16)

    qkvn = (Hq + 2 * Hkv) * D
    head = {"embed": w(V, H, 1.0), "w_fc": w(H, 2 * H, (2 * H) ** -0.5), "w_qkv": w(qkvn, H, H ** -0.5),
            "w_o": w(H, Hq * D, (Hq * D) ** -0.5), "w_gate_up": w(2 * I, H, H ** -0.5),
            "w_down": w(H, I, I ** -0.5), "w_lm": w(V, H, H ** -0.5),
            "g1": torch.ones(H, device=dev), "g2": torch.ones(H, device=dev)}
    f0 = w(B, H, 1.0)
    root = torch.randint(0, V, (B,), generator=gen, device=dev, dtype=torch.int32)
    kc = torch.randn((B, Hkv, P + R, D), generator=gen, device=dev).to(torch.bfloat16)
    vc = torch.randn((B, Hkv, P + R, D), generator=gen, device=dev).to(torch.bfloat16)
    ws = torch.empty(max(1, sda.eagle_draft_expand_workspace(B, H, Hq, Hkv, D, I, V, P, P + R, top_k,
                                                             depth)), dtype=torch.uint8, device=dev)
    out = sda.eagle_draft_expand(head, f0, root, kc, vc, P, Hq, top_k, depth, n_nodes, D ** -0.5, 1e-5,
                                 workspace=ws)
    for i in range(DRAFT_WARMUP):
        sda.eagle_draft_expand(head, f0, root, kc, vc, P, Hq, top_k, depth, n_nodes, D ** -0.5, 1e-5,
                               workspace=ws, out=out)
        if i % 4 == 3:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(iters):
        sda.eagle_draft_expand(head, f0, root, kc, vc, P, Hq, top_k, depth, n_nodes, D ** -0.5, 1e-5,
                               workspace=ws, out=out)
    e1.record(s)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / iters
    weights = sum(head[k].numel() * 2 for k in ("w_fc", "w_qkv", "w_o", "w_gate_up", "w_down", "w_lm"))
    streamed = depth * weights
    del head, kc, vc, ws, out
    torch.cuda.empty_cache()
    return {"shape": f"B={B} H={H} Hq={Hq} Hkv={Hkv} D={D} I={I} V={V} draft prefix {P}",
            "top_k": top_k, "depth": depth, "n_nodes": n_nodes, "us": round(us, 1),
            "weight_bytes_per_expansion": streamed,
            "weight_stream_gbs": round(streamed / us / 1e3, 1),
            "weight_stream_frac_of_hbm_peak": round(streamed / us / 1e3 / HBM_PEAK_GBS, 4)}


RAGGED_PREFIX = [32768, 8192, 24576, 2048]
RAGGED_TREE = [60, 40, 60, 25]


def ragged_step(torch, sda, dev, x, steps=50):
    """The verification step (attention, LM head, greedy acceptance) on a ragged C5
    batch: the four sequences keep C5's shapes but have prefixes of RAGGED_PREFIX
    tokens and trees of RAGGED_TREE nodes (rows of the C5 tensors past them are
    padding).  The LM head takes only the real rows, packed."""
    cfg = synth.CONFIGS["C5"]
    B, N, P, D, H, V = cfg.B, cfg.N, cfg.P, cfg.D, cfg.H, cfg.V
    plen = torch.tensor(RAGGED_PREFIX, dtype=torch.int32, device=dev)
    tlen = torch.tensor(RAGGED_TREE, dtype=torch.int32, device=dev)
    M = sum(RAGGED_TREE)
    lib = sda.load()
    ws_attn = torch.empty(max(1, lib.eagle_tree_verify_attn_workspace(B, N, cfg.Hq, cfg.Hkv, D, P)),
                          dtype=torch.uint8, device=dev)
    ws_lm = torch.empty(lib.eagle_lm_head_workspace(M, H, V), dtype=torch.uint8, device=dev)
    attn_out = torch.empty((B, N, cfg.Hq, D), dtype=torch.bfloat16, device=dev)
    attn_lse = torch.empty((B, N, cfg.Hq), dtype=torch.float32, device=dev)
    hidden = x["hidden"][:M]
    amax = torch.zeros((B, N), dtype=torch.int32, device=dev)
    rows = []
    for b, n in enumerate(RAGGED_TREE):
        rows += [b * N + i for i in range(n)]
    idx = torch.tensor(rows, dtype=torch.long, device=dev)
    parents = torch.from_numpy(synth.random_parents(B, N, 0, cfg.index, 20)).to(dev)
    tokens = torch.from_numpy(synth.integers((B, N), 0, V, 0, cfg.index, 21)).to(dev)
    stream = torch.cuda.current_stream()

    def one(ev=None):
        if ev:
            ev[0].record(stream)
        sda.eagle_tree_verify_attn(x["q"], x["k"], x["v"], parents, P, D ** -0.5, out=attn_out,
                                   lse=attn_lse, workspace=ws_attn, prefix_len=plen, tree_len=tlen)
        if ev:
            ev[1].record(stream)
        res = sda.eagle_lm_head_argmax(hidden, x["W"], want_logits=False, workspace=ws_lm)
        if ev:
            ev[2].record(stream)
        amax.view(-1).index_copy_(0, idx, res["argmax"])
        sda.eagle_accept_greedy(tokens, parents, amax, cfg.max_depth, tree_len=tlen)
        if ev:
            ev[3].record(stream)

    _warm(torch, one)
    ms = _window_ms(torch, one, steps)   # no events inside the window
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        one(evs[i])
    torch.cuda.synchronize()
    per = {n: 1000.0 * sum(e[j].elapsed_time(e[j + 1]) for e in evs) / steps
           for j, n in enumerate(["tree_attn", "lm_head", "accept_greedy"])}
    return {"prefix_len": RAGGED_PREFIX, "tree_len": RAGGED_TREE,
            "tokens_per_s": round(M / (ms / 1000.0), 1), "ms_per_step": round(ms, 4),
            "breakdown_us": {k: round(v, 2) for k, v in per.items()}}


# rocprofv3 runs behind the committed summaries; {out} is the directory they write to
# (the same directory is then passed to --summarize-profiles)
PROFILE_RUNS = {
    "prof": "rocprofv3 --kernel-trace --stats -T -d {out}/prof -o run --output-format csv "
            "-- python -u bench.py --steps 200 --warmup 250 --no-cpu-baseline --no-spec",
    "prof_draft": "rocprofv3 --kernel-trace --stats -T -d {out}/prof_draft -o run --output-format csv "
                  "-- python -u bench.py --only-draft",
    "pmc_fetch": "rocprofv3 --pmc FETCH_SIZE -T -d {out}/pmc_fetch -o run --output-format csv "
                 "-- python -u bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-spec",
    "pmc_write": "rocprofv3 --pmc WRITE_SIZE -T -d {out}/pmc_write -o run --output-format csv "
                 "-- python -u bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-spec",
    "pmc_copy_fetch": "rocprofv3 --pmc FETCH_SIZE -T -d {out}/pmc_copy_fetch -o run "
                      "--output-format csv -- python -u bench.py --copy-calib",
    "pmc_copy_write": "rocprofv3 --pmc WRITE_SIZE -T -d {out}/pmc_copy_write -o run "
                      "--output-format csv -- python -u bench.py --copy-calib",
    "pmc_mfma": "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_BUSY_CU_CYCLES "
                "SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS GRBM_GUI_ACTIVE GRBM_COUNT -T "
                "-d {out}/pmc_mfma -o run --output-format csv -- python -u bench.py --steps 2 "
                "--warmup 1 --no-cpu-baseline --no-spec",
}
TRACE_MD = "c5_step_kernel_trace.md"
DRAFT_TRACE_MD = "c5_draft_expand_kernel_trace.md"
TRAFFIC_MD = "c5_step_hbm_traffic.md"
MFMA_MD = "c5_step_mfma_counters.md"
SIMDS = 1024   # 256 CUs x 4 SIMDs
XCCS = 8


def _run_cmd(name, root):
    """The command of PROFILE_RUNS[name] as run with output directory `root`."""
    return PROFILE_RUNS[name].replace("{out}", os.path.normpath(root))


def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def step_kernel_stats(trace_csv, n_warm, n_timed):
    """(name, calls, avg us, min us, max us, total us) per kernel of a rocprofv3 kernel
    trace, from its dispatches in launch order.  A kernel dispatched once per step keeps
    only the dispatches of the timed steps: bench.py runs n_warm warm-up steps, then
    n_timed steps timed as a whole, then n_timed more with an event between the calls
    (n_warm + 2 n_timed dispatches).  Any other kernel keeps all of its dispatches."""
    runs = {}
    for r in sorted(_read_csv(trace_csv), key=lambda r: int(r["Start_Timestamp"])):
        runs.setdefault(r["Kernel_Name"], []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    stats = []
    for name, d in runs.items():
        if len(d) == n_warm + 2 * n_timed:
            d = d[n_warm:]
        stats.append((name, len(d), sum(d) / len(d), min(d), max(d), sum(d)))
    return stats


def summarize_profiles(root):
    """Turn the five rocprofv3 runs of PROFILE_RUNS (under `root`) into the committed
    text summaries under profiles/ and the per-kernel traffic records bench.py reads."""
    cfg = synth.CONFIGS["C5"]
    B, N, Hq, Hkv, D, P, H, V = cfg.B, cfg.N, cfg.Hq, cfg.Hkv, cfg.D, cfg.P, cfg.H, cfg.V
    cmd = _run_cmd("prof", root)
    flags = cmd.split()
    n_warm = int(flags[flags.index("--warmup") + 1])
    n_timed = int(flags[flags.index("--steps") + 1])
    stats = step_kernel_stats(os.path.join(root, "prof", "run_kernel_trace.csv"), n_warm, n_timed)
    total = sum(st[5] for st in stats)
    lines = ["# rocprofv3 kernel trace: C5 verification step", "",
             "Command (repository root, one MI355X):", "", "    " + cmd, "",
             f"Workload: C5 (B={B}, N={N}, Hq={Hq}, Hkv={Hkv}, D={D}, P={P}, H={H}, V={V}); "
             f"{n_warm + 2 * n_timed} steps ({n_warm} warmup, {n_timed} timed as a whole, {n_timed} "
             "timed call by call, as bench.py runs them), nothing else.  Per-step kernels: the "
             f"{2 * n_timed} timed steps' dispatches only (from the kernel trace).", "",
             "| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for name, n, avg, lo, hi, tot in sorted(stats, key=lambda st: -st[5]):
        lines.append(f"| {name} | {n} | {avg:.2f} | {lo:.2f} | {hi:.2f} | {100.0 * tot / total:.1f} |")
    with open(os.path.join(PROFILE_DIR, TRACE_MD), "w") as f:
        f.write("\n".join(lines) + "\n")
    dpath = os.path.join(root, "prof_draft", "run_kernel_stats.csv")
    if os.path.exists(dpath):
        # the library's kernels only (torch's weight initialisation is left out)
        ours = ("lm_head_", "gemm_splitk", "tree_attn_", "draft_", "rerank_")
        calls = 1 + DRAFT_WARMUP + 3   # first call, warm-up calls, timed calls
        druns = {}
        for r in sorted(_read_csv(os.path.join(root, "prof_draft", "run_kernel_trace.csv")),
                        key=lambda r: int(r["Start_Timestamp"])):
            if r["Kernel_Name"].startswith(ours):
                druns.setdefault(r["Kernel_Name"], []).append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        dstats = []
        for name, d in druns.items():
            if len(d) % calls == 0:
                d = d[len(d) - 3 * (len(d) // calls):]   # the three timed expansions
            dstats.append((name, len(d), sum(d) / len(d), sum(d)))
        dtotal = sum(st[3] for st in dstats)
        B_, H_, Hq_, Hkv_, D_, I_, V_, P_ = DRAFT_SHAPES["C5"]
        dl = ["# rocprofv3 kernel trace: per-depth draft expansion, C5 shapes", "",
              "Command (repository root, one MI355X):", "", "    " + _run_cmd("prof_draft", root), "",
              f"Workload: eagle_draft_expand with a one-layer draft head (B={B_}, H={H_}, Hq={Hq_}, "
              f"Hkv={Hkv_}, D={D_}, MLP {I_}, V={V_}, draft prefix {P_}), top-k 10, depth 6, 60 nodes; "
              f"{calls} expansions ({calls - 3} warmup + 3 timed), the 3 timed ones summarised.  "
              "lm_head_gemm runs every projection and the LM head (6 GEMMs per depth); the library's "
              "kernels only (torch's weight initialisation is left out).", "",
              "| kernel | calls | avg us | total ms | share % |", "|---|---|---|---|---|"]
        for name, n, avg, tot in sorted(dstats, key=lambda st: -st[3]):
            dl.append(f"| {name} | {n} | {avg:.2f} | {tot / 1e3:.3f} | {100.0 * tot / dtotal:.1f} |")
        with open(os.path.join(PROFILE_DIR, DRAFT_TRACE_MD), "w") as f:
            f.write("\n".join(dl) + "\n")
        lines += ["", *dl]

    def per_kernel(run, counter):
        acc = {}
        for r in _read_csv(os.path.join(root, run, "run_counter_collection.csv")):
            if r["Counter_Name"] == counter:
                acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in acc.items()}

    copy_bytes = 1 << 30
    cf = per_kernel("pmc_copy_fetch", "FETCH_SIZE")
    cw = per_kernel("pmc_copy_write", "WRITE_SIZE")
    copy_name = max(cf, key=cf.get)
    f_fac = copy_bytes / 1024.0 / cf[copy_name]
    w_fac = copy_bytes / 1024.0 / cw[copy_name]
    fetch = per_kernel("pmc_fetch", "FETCH_SIZE")
    write = per_kernel("pmc_write", "WRITE_SIZE")
    # the C5 attention kernel (the D = 128 eight-wave kernel at these shapes)
    attn_name = next(k for k in fetch if k.startswith("tree_attn_") and "merge" not in k)
    algo = {attn_name: 2 * B * Hkv * (P + N) * D * 2 + 2 * B * N * Hq * D * 2 + B * N * Hq * 4,
            "lm_head_gemm": V * H * 2 + B * N * H * 2 + B * N * 16}
    cmds = [_run_cmd(k, root) for k in ("pmc_fetch", "pmc_write", "pmc_copy_fetch", "pmc_copy_write")]
    rows = ["# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE), C5 verification step", "",
            "Commands (repository root, one MI355X; each counter in a run of its own):", ""]
    rows += ["    " + c for c in cmds]
    rows += ["", f"Calibration: a plain 1 GiB device copy (`bench.py --copy-calib`, `{copy_name}`) reads",
             f"FETCH_SIZE = {cf[copy_name]:.0f} KiB and WRITE_SIZE = {cw[copy_name]:.0f} KiB per dispatch,",
             f"so HBM bytes = FETCH_SIZE x 1024 x {f_fac:.3f} + WRITE_SIZE x 1024 x {w_fac:.3f}.", "",
             "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (calibrated) | algorithmic bytes | ratio |",
             "|---|---|---|---|---|---|"]
    for k in fetch:
        if k.startswith("__amd"):
            continue
        hbm = fetch[k] * 1024 * f_fac + write.get(k, 0.0) * 1024 * w_fac
        a = algo.get(k)
        rows.append(f"| {k} | {fetch[k]:.0f} | {write.get(k, 0.0):.0f} | {hbm / 1e6:.1f} MB | "
                    + (f"{a / 1e6:.1f} MB | {hbm / a:.3f} |" if a else " |  |"))
    with open(os.path.join(PROFILE_DIR, TRAFFIC_MD), "w") as f:
        f.write("\n".join(rows) + "\n")
    for short, kname in (("lm_head", "lm_head_gemm"), ("tree_attn", attn_name)):
        hbm = fetch[kname] * 1024 * f_fac + write[kname] * 1024 * w_fac
        rec = {"kernel": kname, "workload": "C5", "fetch_kib": fetch[kname], "write_kib": write[kname],
               "fetch_factor": f_fac, "write_factor": w_fac, "bytes_per_launch": int(round(hbm)),
               "algorithmic_bytes": algo[kname], "source": KERNEL_SOURCES[short],
               "source_sha256_16": _src_hash(KERNEL_SOURCES[short]), "commands": cmds}
        with open(os.path.join(PROFILE_DIR, f"{short}_C5_traffic.json"), "w") as f:
            json.dump(rec, f, indent=1)
    print("\n".join(lines + [""] + rows))
    mpath = os.path.join(root, "pmc_mfma", "run_counter_collection.csv")
    if os.path.exists(mpath):
        print(summarize_mfma(mpath, root))


def summarize_mfma(path, root=None):
    """Per-kernel matrix-core and LDS counters of the C5 step (the PROFILE_RUNS
    "pmc_mfma" run): the clock the kernel ran at (GRBM_GUI_ACTIVE cycles per XCC over
    the dispatch time), MFMA busy cycles per SIMD over those cycles, bf16 MFMA flops
    (512 per MOPS unit, padding included) over the dispatch time, LDS activity."""
    import collections
    if root is None:   # <root>/pmc_mfma/run_counter_collection.csv
        root = os.path.dirname(os.path.dirname(os.path.abspath(path)))
    per = collections.defaultdict(dict)
    span = {}
    import re
    for r in _read_csv(path):
        # plain ("lm_head_gemm") or demangled ("void eagle::(anonymous namespace)::lm_head_gemm<...>(...)")
        m = re.search(r"(?<![A-Za-z0-9_])(lm_head_gemm|tree_attn_d128)(?![A-Za-z0-9_])", r["Kernel_Name"])
        if not m:
            continue
        key = (int(r["Dispatch_Id"]), m.group(1))
        per[key][r["Counter_Name"]] = float(r["Counter_Value"])
        span[key] = (int(r["Start_Timestamp"]), int(r["End_Timestamp"]))
    agg = collections.defaultdict(list)
    for key, c in per.items():
        name = key[1]
        t0, t1 = span[key]
        dur_s = (t1 - t0) * 1e-9
        cycles = c["GRBM_GUI_ACTIVE"] / XCCS
        agg[name].append({"us": dur_s * 1e6, "mhz": cycles / dur_s / 1e6,
                          "busy": c["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * SIMDS),
                          "tflops": c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / dur_s / 1e12,
                          "lds_active": c["SQ_LDS_IDX_ACTIVE"] / (cycles * SIMDS / 4),
                          "conflicts": c["SQ_LDS_BANK_CONFLICT"]})
    lines = ["# rocprofv3 matrix-core and LDS counters: C5 verification step", "",
             "Command (repository root, one MI355X):", "", "    " + _run_cmd("pmc_mfma", root), "",
             "Per kernel, the mean over the run's dispatches (3 steps).  clock = GRBM_GUI_ACTIVE / 8 XCCs",
             "over the dispatch time; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (clock cycles x 1024 SIMDs);",
             "bf16 MFMA rate = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 flop over the dispatch time (padded",
             "tiles included); LDS active = SQ_LDS_IDX_ACTIVE / (clock cycles x 256 CUs).  Peak bf16",
             "MFMA at the measured clock = 1024 flop/clk/SIMD x 1024 SIMDs x clock.", "",
             "| kernel | dispatches | avg us | clock MHz | MFMA busy % | bf16 MFMA TFLOP/s | peak at clock TFLOP/s | LDS active % | LDS bank conflicts |",
             "|---|---|---|---|---|---|---|---|---|"]
    for name, v in sorted(agg.items()):
        m = {k: sum(x[k] for x in v) / len(v) for k in v[0]}
        lines.append(f"| {name} | {len(v)} | {m['us']:.1f} | {m['mhz']:.0f} | {100 * m['busy']:.1f} | "
                     f"{m['tflops']:.0f} | {1024 * SIMDS * m['mhz'] * 1e6 / 1e12:.0f} | "
                     f"{100 * m['lds_active']:.1f} | {m['conflicts']:.0f} |")
    text = "\n".join(lines) + "\n"
    with open(os.path.join(PROFILE_DIR, MFMA_MD), "w") as f:
        f.write(text)
    return text


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # about 0.2 s of steps: the chip's power management throttles a fresh load hard
    # over its first few tens of milliseconds and then settles (see _warm); the timed
    # steps measure the settled rate, and the warmup steps' own rate is reported too
    ap.add_argument("--warmup", type=int, default=250)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-spec", action="store_true",
                    help="only the C5 step: skip the other workloads' steps, the measured "
                         "ceilings, the back-to-back LM head, the spec latency, KV commit, "
                         "ragged, paged and draft-expansion measurements")
    ap.add_argument("--only-draft", action="store_true",
                    help="only the C5-shaped draft expansion (eagle_draft_expand)")
    ap.add_argument("--only-ragged", action="store_true",
                    help="only the ragged C5 step (attention, LM head, greedy acceptance)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write profiles/ summaries from the rocprofv3 runs listed in "
                         "PROFILE_RUNS, found under DIR (no GPU needed)")
    args = ap.parse_args(argv)
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return 0
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding is described in DESIGN.md, not implemented)", file=sys.stderr)
        return 2

    import torch

    import speculative_decoding_attn_amd as sda
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    sda.load()
    dev = torch.device("cuda:0")
    if args.copy_calib:
        copy_calibration(torch, dev)
        return 0
    if args.only_draft:
        print(json.dumps({"draft_expand_C5": draft_expansion(torch, sda, dev, "C5")}))
        return 0
    if args.only_ragged:
        x = make_inputs(synth.CONFIGS["C5"], torch, dev)
        print(json.dumps({"ragged_C5": ragged_step(torch, sda, dev, x)}))
        return 0

    cfg = synth.CONFIGS["C5"]
    B, N, Hq, Hkv, D, P, H, V = cfg.B, cfg.N, cfg.Hq, cfg.Hkv, cfg.D, cfg.P, cfg.H, cfg.V
    t_gen = time.perf_counter()
    x = make_inputs(cfg, torch, dev)
    torch.cuda.synchronize()
    print(f"# inputs resident in HBM ({time.perf_counter() - t_gen:.1f} s)", file=sys.stderr,
          flush=True)
    lib = sda.load()
    ws_attn = torch.empty(max(1, lib.eagle_tree_verify_attn_workspace(B, N, Hq, Hkv, D, P)),
                          dtype=torch.uint8, device=dev)
    ws_lm = torch.empty(lib.eagle_lm_head_workspace(B * N, H, V), dtype=torch.uint8, device=dev)
    ws_rr = torch.empty(lib.eagle2_rerank_workspace(B, V, cfg.top_k, cfg.depth), dtype=torch.uint8,
                        device=dev)
    attn_out = torch.empty((B, N, Hq, D), dtype=torch.bfloat16, device=dev)
    attn_lse = torch.empty((B, N, Hq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        tree = sda.eagle2_rerank(x["draft_logits"], x["root"], cfg.top_k, cfg.depth, N, workspace=ws_rr)
        if ev:
            ev[1].record(stream)
        sda.eagle_tree_verify_attn(x["q"], x["k"], x["v"], tree["parents"], P, D ** -0.5,
                                   out=attn_out, lse=attn_lse, workspace=ws_attn)
        if ev:
            ev[2].record(stream)
        res = sda.eagle_lm_head_argmax(x["hidden"], x["W"], want_logits=False, workspace=ws_lm)
        if ev:
            ev[3].record(stream)
        acc = sda.eagle_accept_greedy(tree["tokens"], tree["parents"], res["argmax"].view(B, N),
                                      cfg.max_depth)
        if ev:
            ev[4].record(stream)
        return tree, acc

    ew = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ew[0].record(stream)
    for i in range(args.warmup):
        tree, _ = step()
        if i % 8 == 7:
            torch.cuda.synchronize()
    ew[1].record(stream)
    torch.cuda.synchronize()
    warmup_ms = ew[0].elapsed_time(ew[1]) / args.warmup if args.warmup > 0 else None
    parents_np = tree["parents"].cpu().numpy()

    # the timed steps: one event before and one after, nothing recorded in between (an
    # event between the calls of a step costs the step about 11 us)
    ew = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ew[0].record(stream)
    for i in range(args.steps):
        step()
    ew[1].record(stream)
    torch.cuda.synchronize()
    total_ms = ew[0].elapsed_time(ew[1])
    ms_per_step = total_ms / args.steps
    # the per-call breakdown: as many steps again, with an event between the calls
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    names = ["rerank", "tree_attn", "lm_head", "accept_greedy"]
    per = {n: 1000.0 * sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps
           for j, n in enumerate(names)}
    breakdown_ms = evs[0][0].elapsed_time(evs[-1][4]) / args.steps
    value = B * N / (ms_per_step / 1000.0)

    # rooflines
    lm_b = lm_bytes(B * N, H, V)
    lm_gbs = lm_b / (per["lm_head"] * 1e-6) / 1e9
    attn_b = attn_bytes(cfg)
    a_flops = attn_flops(parents_np, cfg)
    attn_tflops = a_flops / (per["tree_attn"] * 1e-6) / 1e12
    attn_gbs = attn_b / (per["tree_attn"] * 1e-6) / 1e9
    rr_bytes = B * cfg.rows * V * 4
    dominant = max(("lm_head", "tree_attn"), key=lambda n: per[n])
    roof_lm = {"kernel": "lm_head (eagle_lm_head_argmax)", "bound": "hbm",
               "achieved": round(lm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
               "frac": round(lm_gbs / HBM_PEAK_GBS, 4), "traffic": _traffic("lm_head"),
               "algorithmic_bytes": lm_b, "avg_us": round(per["lm_head"], 2),
               "mfma_frac": round(2.0 * B * N * H * V / (per["lm_head"] * 1e-6) / 1e12
                                  / BF16_MFMA_PEAK_TFLOPS, 4)}
    roof_attn = {"kernel": "tree_attn (eagle_tree_verify_attn)", "bound": "mfma",
                 "achieved": round(attn_tflops, 1), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(attn_tflops / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": _traffic("tree_attn"),
                 "algorithmic_flops": a_flops, "algorithmic_bytes": attn_b,
                 "hbm_gbs": round(attn_gbs, 1), "hbm_frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                 "avg_us": round(per["tree_attn"], 2)}
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "warmup_ms_per_step": None if warmup_ms is None else round(warmup_ms, 4),
        "breakdown_ms_per_step": round(breakdown_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "C5 Llama-3-70B-shaped tree verification: 4 sequences x 60-node "
                               "EAGLE-2 trees (top-k 10, depth 6), GQA 64/8 heads, head dim 128, "
                               "KV prefix 32768, hidden 8192, vocab 128256, greedy acceptance",
                   "B": B, "N": N, "Hq": Hq, "Hkv": Hkv, "D": D, "P": P, "H": H, "V": V,
                   "top_k": cfg.top_k, "depth": cfg.depth, "parallelism": "single GPU"},
        "roofline": roof_lm if dominant == "lm_head" else roof_attn,
        "roofline_attn": roof_attn,
        "roofline_lm_head": roof_lm,
        "breakdown_us": {k: round(v, 2) for k, v in per.items()},
        "rerank_hbm_gbs": round(rr_bytes / (per["rerank"] * 1e-6) / 1e9, 1),
    }
    if not args.no_spec:
        out["lm_head_back_to_back_C5"] = lm_head_back_to_back(torch, sda, dev, x)
        del x
        torch.cuda.empty_cache()
        out["configs"] = {}
        for name in ("C2", "C3", "C4"):
            print(f"# {name} step", file=sys.stderr, flush=True)
            out["configs"][name] = config_step(torch, sda, dev, name)
        out["measured_ceilings"] = measured_ceilings(torch, sda, dev)
        x = make_inputs(cfg, torch, dev)
        out["accept_spec_us_C4"] = round(spec_latency(torch, sda, dev), 2)
        out["accept_spec_no_lse_us_C4"] = round(spec_latency(torch, sda, dev, with_lse=False), 2)
        out["accept_spec_point_mass_us_C4"] = round(spec_latency(torch, sda, dev, mode="point_mass"), 2)
        out["kv_commit_80_layers"] = kv_commit_latency(torch, sda, dev, tree["parents"])
        out["ragged_C5"] = ragged_step(torch, sda, dev, x)
        out["paged_attention_C5"] = paged_attention(torch, sda, dev, x, tree["parents"])
        out["draft_expand_C5"] = draft_expansion(torch, sda, dev, "C5")
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg)
        print("# timing the CPU oracle baseline on one thread", file=sys.stderr, flush=True)
        out["cpu_baseline"]["single_thread"] = cpu_baseline_single_thread(cfg)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
