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
