"""The synthetic workloads the layer is checked and measured on.

Shapes follow the Kimi K2 pages: hidden size d = 7168 ("Input features" page,
tensor x), expert intermediate size 2048 ("Element-wise product" page, operand
shapes), 384 routed experts with 8 selected per position ("Mixture of experts"
page, experts inspector header), one shared expert of the same intermediate
size ("Mixture of experts" page, Direct evidence "moe-init").

The sixth workload is what one GPU of an 8-way expert-parallel group runs at 8192
tokens per GPU. The same page's moe-init evidence gives each rank a contiguous
range of 384 / 8 = 48 experts, and its Code (moe_infer) sends every (token,
choice) row to the rank that owns the chosen expert. That rank then runs its
experts on the rows it received and returns them unweighted; the sender does the
weighting. With uniform top-8 routing a rank receives 8 x 8192 x 8 / 8 = 65536
rows on average, and each lands on a given local expert with probability 1/48,
so each local expert gets about 1365 rows. Here the count is fixed at 65536. Each
row's local expert is uniform over the 48, which is the marginal of the routing.
Rows are drawn independently: a token that picks two experts of the rank
contributes two rows, and whether those rows hold equal values changes no work.
The layer call on such a shard (K = 1, unit weights) is the receiving rank's whole
part: sort the rows by local expert, run the experts, and put the outputs back in
arrival order (the combine of one unit-weight choice is that inverse permutation).

The seventh workload is the dense block's SwiGLU MLP ("SwiGLU output" page: one dense
block whose feed-forward network is the same down(silu(gate x) * up x) with the model's
intermediate_size) at 8192 tokens: one expert that every token visits with weight 1.
The pages print no value for that intermediate size. The workload takes 18432 (9 x 2048,
the size of the public configs of this architecture family, an assumption); the kernels
take any multiple of 128.
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
    w_mode: str     # "softmax": softmax of N(0,1) logits; "uniform": U(0,1) normalised; "dirichlet": Dirichlet(1);
                    # "ones": every weight 1 (unweighted rows)
    shared: bool    # one always-on shared expert
    seed: int = 0
    weight_std: float = 0.02
    # > 0: the workload is one GPU's shard of an expert-parallel layer whose router picks
    # this many experts per token; its N rows are received token choices, E the local experts
    shard_topk: int = 0
    # the dense block's MLP (E = 1, K = 1, unit weights) rather than a routed layer
    dense: bool = False

    @property
    def slots(self) -> int:
        return self.N * self.K

    @property
    def layer_tokens(self) -> int:
        """Tokens of the layer that one step covers (for a shard: its GPU's own tokens)."""
        return self.N * self.K // self.shard_topk if self.shard_topk else self.N


CONFIGS = [
    Config("toy", 64, 256, 128, 8, 2, "normal", "uniform", "softmax", False),
    Config("k2_decode_16", 16, 7168, 2048, 384, 8, "rmsnorm", "uniform", "uniform", False),
    Config("k2_decode_256", 256, 7168, 2048, 384, 8, "rmsnorm", "uniform", "uniform", False),
    Config("k2_prefill_8192", 8192, 7168, 2048, 384, 8, "rmsnorm", "uniform", "uniform", False),
    Config("k2_skewed_shared_4096", 4096, 7168, 2048, 384, 8, "rmsnorm", "zipf", "dirichlet", True),
    Config("k2_ep8_shard_8192", 65536, 7168, 2048, 48, 1, "rmsnorm", "uniform", "ones", False, shard_topk=8),
    Config("k2_dense_8192", 8192, 7168, 18432, 1, 1, "rmsnorm", "uniform", "ones", False, dense=True),
]


def config_by_name(name: str) -> Config:
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)
