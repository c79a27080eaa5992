"""Test-side glue: seeded inputs from `synth` as numpy (oracle side) and torch
(device side) views of the same values.  No method arithmetic here."""
import numpy as np

import synth


def bf16(shape, std, seed, cfg, tensor):
    """Returns (bits uint16, fp64 values)."""
    bits = synth.normal_bf16_bits(shape, std, seed, cfg, tensor)
    return bits, synth.bf16_bits_to_f64(bits)


def to_dev_bf16(bits, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def to_dev(a, dtype=None, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device)


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def assert_close_attn(got, ref, max_abs=2e-2, max_rel_l2=5e-3):
    """Tolerance for bf16 inputs with fp32 accumulation and bf16 output."""
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref).max() if got.size else 0.0
    rl = rel_l2(got, ref) if got.size else 0.0
    assert err <= max_abs and rl <= max_rel_l2, f"max-abs {err:.3g}, rel-L2 {rl:.3g}"


# ---- one-layer draft head (per-depth draft expansion): shapes and seeded values
DRAFT_STD = {  # tensor -> (shape builder, std builder, generator tensor id)
    "embed": (lambda H, Hq, Hkv, D, I, V: (V, H), lambda H, Hq, Hkv, D, I: 1.0, 40),
    "fc": (lambda H, Hq, Hkv, D, I, V: (H, 2 * H), lambda H, Hq, Hkv, D, I: (2 * H) ** -0.5, 41),
    "q": (lambda H, Hq, Hkv, D, I, V: (Hq * D, H), lambda H, Hq, Hkv, D, I: H ** -0.5, 42),
    "k": (lambda H, Hq, Hkv, D, I, V: (Hkv * D, H), lambda H, Hq, Hkv, D, I: H ** -0.5, 43),
    "v": (lambda H, Hq, Hkv, D, I, V: (Hkv * D, H), lambda H, Hq, Hkv, D, I: H ** -0.5, 44),
    "o": (lambda H, Hq, Hkv, D, I, V: (H, Hq * D), lambda H, Hq, Hkv, D, I: (Hq * D) ** -0.5, 45),
    "gate": (lambda H, Hq, Hkv, D, I, V: (I, H), lambda H, Hq, Hkv, D, I: H ** -0.5, 46),
    "up": (lambda H, Hq, Hkv, D, I, V: (I, H), lambda H, Hq, Hkv, D, I: H ** -0.5, 47),
    "down": (lambda H, Hq, Hkv, D, I, V: (H, I), lambda H, Hq, Hkv, D, I: I ** -0.5, 48),
    "lm": (lambda H, Hq, Hkv, D, I, V: (V, H), lambda H, Hq, Hkv, D, I: H ** -0.5, 49),
}


def draft_case(seed, cfg, B, H, Hq, Hkv, D, I, V, P, cap=None):
    """Synthetic draft head weights and inputs.

    Returns (bits, vals): bits holds uint16 bf16 bits for the device (weights, f0
    [B][H], k_cache / v_cache [B][Hkv][cap][D] with rows 0..P-1 filled) and float32
    gains g1, g2 [H]; vals holds the same values as fp64 for the oracle, plus the
    ints Hq, Hkv, D.  Root tokens [B] are in both.
    """
    cap = cap if cap is not None else P
    bits, vals = {}, {"Hq": Hq, "Hkv": Hkv, "D": D}
    for name, (shape, std, tid) in DRAFT_STD.items():
        b_, v_ = bf16(shape(H, Hq, Hkv, D, I, V), std(H, Hq, Hkv, D, I), seed, cfg, tid)
        bits[name], vals[name] = b_, v_
    for gname, tid in (("g1", 50), ("g2", 51)):
        g = (1.0 + 0.1 * synth.normal_f32((H,), 1.0, seed, cfg, tid)).astype(np.float32)
        bits[gname], vals[gname] = g, g.astype(np.float64)
    bits["f0"], vals["f0"] = bf16((B, H), 1.0, seed, cfg, 52)
    kc = np.zeros((B, Hkv, cap, D), dtype=np.uint16)
    vc = np.zeros((B, Hkv, cap, D), dtype=np.uint16)
    if P > 0:
        kc[:, :, :P] = synth.normal_bf16_bits((B, Hkv, P, D), 1.0, seed, cfg, 53)
        vc[:, :, :P] = synth.normal_bf16_bits((B, Hkv, P, D), 1.0, seed, cfg, 54)
    bits["k_cache"], bits["v_cache"] = kc, vc
    vals["k_cache"], vals["v_cache"] = synth.bf16_bits_to_f64(kc), synth.bf16_bits_to_f64(vc)
    root = synth.integers((B,), 0, V, seed, cfg, 55)
    bits["root"], vals["root"] = root, root.astype(np.int64)
    return bits, vals


def draft_weights_for(vals, b=None):
    """The oracle's weight dict (shared by all sequences)."""
    keys = list(DRAFT_STD) + ["g1", "g2", "Hq", "Hkv", "D"]
    return {k: vals[k] for k in keys}


# ---- per-depth draft expansion: the GPU parity cases and their float tolerance.
# (seed, B, H, Hq, Hkv, D, I, V, P, top_k, depth, n_nodes, whole_tree): seeds chosen
# with the oracle alone so that deep rows, and in the first two cases whole trees, are
# decided clearly; V spans one to eight LM-head vocabulary tiles.
DRAFT_CASES = [
    (23, 4, 128, 8, 2, 128, 192, 128, 0, 3, 5, 14, True),
    (26, 3, 192, 2, 1, 64, 320, 96, 37, 5, 3, 16, True),
    (7, 4, 256, 4, 2, 64, 512, 200, 100, 4, 4, 12, False),
    (4, 2, 256, 4, 2, 64, 512, 1000, 100, 4, 4, 12, False),
    # 225 rows per depth (45 x 5): the GEMMs' 256-row tile with one real row in its
    # last 32-row tile (the 16x16x32 path), split over K in W_down (I = 2048)
    (31, 45, 128, 4, 2, 64, 2048, 300, 40, 5, 3, 12, False),
]
# Float tolerance (max-abs, logits and bf16 features) of the draft expansion: at least
# 1.5 x the largest deviation from the fp64 oracle that a CPU model of the kernels'
# arithmetic (bf16 storage at the oracle's rounding points, fp32 accumulation, softmax
# weights rounded to bf16 before the value product) shows on DRAFT_CASES;
# tests/test_oracle_draft.py checks that bound.
DRAFT_TAU = 0.05
