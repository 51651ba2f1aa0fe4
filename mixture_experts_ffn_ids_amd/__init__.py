"""MI355X-native routed-expert MoE layer (Kimi-K2 shapes): Python binding of libmoe.

The layer runs entirely in the HIP kernels of libmoe.so (include/moe.h):
dispatch -> grouped FP8 SwiGLU experts -> deterministic weighted combine; moe_block_ffn
adds the block's RMSNorm (fused with the activation quantisation) and residual addition
(fused with the combine) around it. dense_swiglu and dense_block_ffn run the dense block's
SwiGLU MLP through the same kernels as a single expert that every token visits.
"""
from .api import (Dispatch, combine, dense_block_ffn, dense_swiglu, dispatch, grouped_swiglu,  # noqa: F401
                  grouped_swiglu_noalloc, grouped_swiglu_q, grouped_swiglu_top1, identity_dispatch, moe_block_ffn, moe_layer,
                  profile_enable, profile_read, profile_reset, quantize_rows, rmsnorm_quantize)
from ._lib import (FLAG_CHECKED, FLAG_TILE_16, FLAG_TILE_128, FLAG_TILE_192, FLAG_TILE_224,  # noqa: F401
                   FLAG_TILE_256, KERNEL_COMBINE, KERNEL_DISPATCH, KERNEL_DOWN, KERNEL_GATE_UP, KERNEL_QUANT,
                   LIB_PATH, MoeError)

__all__ = ["Dispatch", "combine", "dense_block_ffn", "dense_swiglu", "dispatch", "grouped_swiglu",
           "grouped_swiglu_noalloc", "grouped_swiglu_q", "grouped_swiglu_top1", "identity_dispatch", "moe_block_ffn", "moe_layer",
           "quantize_rows", "rmsnorm_quantize", "profile_enable", "profile_read", "profile_reset", "MoeError",
           "LIB_PATH", "FLAG_CHECKED", "FLAG_TILE_16", "FLAG_TILE_128", "FLAG_TILE_192", "FLAG_TILE_224",
           "FLAG_TILE_256"]
