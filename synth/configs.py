"""The five synthetic workloads (shapes, tree topologies, value distributions).

C1 tiny CPU-scale case; C2 Vicuna-7B-shaped layer with a static EAGLE-1 tree;
C3 Llama-3-8B-shaped layer with an EAGLE-2 dynamic tree, greedy; C4 the same with
multi-round speculative sampling; C5 Llama-3-70B-shaped, 32K prefix, batch 4.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple

# tensor ids used in the seed sequence [seed, config, tensor, chunk]
TENSOR_IDS = {
    "q": 1, "k": 2, "v": 3, "hidden": 4, "W": 5, "draft_logits": 6, "root_token": 7,
    "u_accept": 8, "u_sample": 9, "target_logits": 10, "plant": 11,
}


@dataclass(frozen=True)
class Config:
    name: str
    index: int            # config number used in the seed sequence
    B: int                # sequences
    Hq: int
    Hkv: int
    D: int
    P: int                # KV prefix length
    N: int                # tree nodes per sequence, root included
    H: int                # hidden size
    V: int                # vocabulary
    w_std: float          # LM-head weight std
    accept: str           # "greedy" or "spec"
    parents: Optional[Tuple[int, ...]] = None   # static tree, else built by rerank
    plant_prob: float = 0.0
    top_k: int = 0        # rerank expansion width
    depth: int = 0        # rerank draft levels
    draft_std: float = 3.0
    max_depth: int = field(default=0)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def M(self) -> int:
        return self.B * self.N

    @property
    def rows(self) -> int:
        """Draft-logit rows per sequence for rerank: root + (depth-1) frontier levels."""
        return 1 + (self.depth - 1) * self.top_k if self.depth else 0

    @property
    def kv_len(self) -> int:
        return self.P + self.N


C2_TREE = (-1, 0, 0, 0, 0, 1, 1, 1, 2, 2, 3, 4, 5, 5, 6, 7, 8, 8, 9, 10, 12, 13, 14, 16, 20, 21)

CONFIGS = {
    "C1": Config("C1", 1, B=1, Hq=2, Hkv=1, D=64, P=128, N=10, H=256, V=1000, w_std=1 / 16,
                 accept="greedy", parents=(-1, 0, 0, 0, 1, 1, 2, 2, 3, 3), plant_prob=0.7,
                 max_depth=2),
    "C2": Config("C2", 2, B=1, Hq=32, Hkv=32, D=128, P=1024, N=26, H=4096, V=32000, w_std=1 / 64,
                 accept="greedy", parents=C2_TREE, plant_prob=0.75, max_depth=5),
    "C3": Config("C3", 3, B=1, Hq=32, Hkv=8, D=128, P=4096, N=60, H=4096, V=128256, w_std=1 / 64,
                 accept="greedy", top_k=10, depth=6, max_depth=6),
    "C4": Config("C4", 4, B=1, Hq=32, Hkv=8, D=128, P=4096, N=60, H=4096, V=128256, w_std=1 / 64,
                 accept="spec", top_k=10, depth=6, max_depth=6),
    "C5": Config("C5", 5, B=4, Hq=64, Hkv=8, D=128, P=32768, N=60, H=8192, V=128256,
                 w_std=8192 ** -0.5, accept="greedy", top_k=10, depth=6, max_depth=6),
}
