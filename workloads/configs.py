"""The five synthetic workloads the layer is checked and measured on.

Shapes follow the Kimi K2 pages: hidden size d = 7168 ("Input features" page,
tensor x), expert intermediate size 2048 ("Element-wise product" page, operand
shapes), 384 routed experts with 8 selected per position ("Mixture of experts"
page, experts inspector header), one shared expert of the same intermediate
size ("Mixture of experts" page, Direct evidence "moe-init").
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Config:
    name: str
    N: int          # tokens (B * T)
    d: int          # hidden size
    d_ff: int       # expert intermediate size
    E: int          # routed experts
    K: int          # experts per token
    x_mode: str     # "normal": N(0,1) rows; "rmsnorm": N(0,1) rows normalised (fp32, eps 1e-6, gain 1)
    ids_mode: str   # "uniform": K distinct uniform experts; "zipf": Zipf(1.2) without replacement
    w_mode: str     # "softmax": softmax of N(0,1) logits; "uniform": U(0,1) normalised; "dirichlet": Dirichlet(1)
    shared: bool    # one always-on shared expert
    seed: int = 0
    weight_std: float = 0.02

    @property
    def slots(self) -> int:
        return self.N * self.K


CONFIGS = [
    Config("toy", 64, 256, 128, 8, 2, "normal", "uniform", "softmax", False),
    Config("k2_decode_16", 16, 7168, 2048, 384, 8, "rmsnorm", "uniform", "uniform", False),
    Config("k2_decode_256", 256, 7168, 2048, 384, 8, "rmsnorm", "uniform", "uniform", False),
    Config("k2_prefill_8192", 8192, 7168, 2048, 384, 8, "rmsnorm", "uniform", "uniform", False),
    Config("k2_skewed_shared_4096", 4096, 7168, 2048, 384, 8, "rmsnorm", "zipf", "dirichlet", True),
]


def config_by_name(name: str) -> Config:
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)
