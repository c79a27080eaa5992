"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module draws random numbers and rounds them to the storage type; it holds
none of the method's arithmetic (no attention, no softmax, no acceptance rule,
no tree search).  Both `oracle/` and the HIP binding's callers take their inputs
from here, and nothing here imports either of them.

Every tensor ``t`` of workload ``c`` is drawn from
``numpy.random.Generator(PCG64(SeedSequence([seed, c, t, chunk])))`` over fixed
chunks of its flattened elements, so the values do not depend on the order in
which tensors (or chunks) are produced, and large tensors are filled by several
threads.  Floating-point tensors that the GPU reads as bf16 are drawn in fp32
and rounded to bf16 once, round-to-nearest-even; both sides see those rounded
values (the oracle widens them to fp64).
"""
from .gen import (  # noqa: F401
    CHUNK,
    bf16_bits_to_f32,
    chain_parents,
    random_parents,
    bf16_bits_to_f64,
    integers,
    normal_bf16_bits,
    normal_f32,
    plant_tokens,
    round_f32_to_bf16_bits,
    uniform_f32,
)
from .configs import CONFIGS, Config, TENSOR_IDS  # noqa: F401
