"""CPU oracle for GLM-5.2's DSA lightning indexer + IndexShare + sparse MLA.

TEST INFRASTRUCTURE. This package is a plain, slow, obviously-correct numpy
(float64) statement of what the hot path computes. It exists to check the HIP
library against. Only the tests, the smoke check and the benchmark's CPU
baseline leg may import it; the product path never does, and this package
imports nothing from the product (it shares no code, constants generator,
table or helper with it).

Sources (page titles as published):
  * "GLM-5.2 总览" (t6page), table tbl-glm52-config: 32-head x 128-dim indexer,
    top-K 2048, 64 heads, QK dim 256 = 192 + 64, MLA latent 512 + RoPE 64 in
    BF16 = 1152 B per token per layer (~656 B in FP8 with per-group scales);
    glossary (FP8 is E4M3, also for the latent cache).
  * "GLM-5.2 架构深度拆解" (pillumina), CH2 §2.1 (indexer_types pattern),
    §2.2 (F layer: score all history, take top-2048, attend; S layer: skip the
    indexer, reuse the nearest full layer's indices), §2.4 (F writes / S reads
    the shared top-k buffer), §7.3 (all-"full" degrades to per-layer DSA).
  * "GLM-5→5.1→5.2：稀疏索引、Agent 后训练与 1M 上下文服务" (papers-3lj),
    §10 (operator order: indexer once per group, write shared buffer, each
    layer gathers its own K/V, sparse attention).

Readings where the pages are silent are listed with each function.

Every function is pinned by `-m "not gpu"` tests against brute force, closed
forms, invariants or an independent library routine; none is "parity
unpinned".
"""
from .e4m3 import e4m3_decode, e4m3_encode, quantize_blocks, dequantize_blocks
from .indexer import indexer_score
from .topk import group_max, topk_select
from .mla import paged_cache_view, sparse_mla
from .latent_fp8 import dequantize_latent, quantize_latent
from .hadamard import hadamard, indexer_inputs_fp8_hadamard, quantize_blocks_hadamard, rotate_blocks
from .pattern import layer_pattern, shared_source
from .group import indexer_inputs_fp8, indexshare_group, layer_stack

__all__ = [
    "e4m3_decode", "e4m3_encode", "quantize_blocks", "dequantize_blocks",
    "indexer_score", "topk_select", "sparse_mla", "layer_pattern",
    "shared_source", "indexshare_group", "layer_stack", "indexer_inputs_fp8",
    "paged_cache_view", "group_max", "quantize_latent", "dequantize_latent",
    "hadamard", "rotate_blocks", "quantize_blocks_hadamard", "indexer_inputs_fp8_hadamard",
]
