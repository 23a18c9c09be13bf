"""IndexShare composition: one F layer's indices serve it and its S layers. Oracle only.

Pages: "GLM-5.2 架构深度拆解" CH2 §2.2 (an S layer skips the indexer and reuses
the indices of the nearest full layer), §2.4 (the full layer writes an outer
shared top-k buffer, shared layers read it), §7.3 (with no shared layers the
model is per-layer DSA); "GLM-5→5.1→5.2…" §10 (indexer once per group, shared
buffer written once, each layer gathers from its own cache, then sparse
attention).
"""
from __future__ import annotations

import numpy as np

from .e4m3 import dequantize_blocks, quantize_blocks
from .indexer import indexer_score
from .mla import sparse_mla
from .pattern import layer_pattern, shared_source
from .topk import topk_select


def indexer_inputs_fp8(q_idx, k_idx):
    """The fp8 variant scores the dequantised per-128-block E4M3 values of q and k."""
    qc, qs = quantize_blocks(q_idx)
    kc, ks = quantize_blocks(k_idx)
    return dequantize_blocks(qc, qs), dequantize_blocks(kc, ks)


def indexshare_group(q_idx, w, k_idx, q_seq, q_pos, layers, k=2048, scale=1.0 / 16.0):
    """layers: [(q_lat, q_rope, kv), ...] — the F layer first, then its S layers.

    Returns (scores, idx, [(out, lse) per layer]); every layer uses the same idx."""
    scores = indexer_score(q_idx, w, k_idx, q_seq, q_pos)
    idx = topk_select(scores, q_pos, k)
    outs = [sparse_mla(ql, qr, kv, q_seq, idx, scale) for (ql, qr, kv) in layers]
    return scores, idx, outs


def layer_stack(indexer_by_f, mla_by_layer, q_seq, q_pos, n_layers=78, k=2048,
                scale=1.0 / 16.0):
    """indexer_by_f[f] = (q_idx, w, k_idx) for every full layer f;
    mla_by_layer[l] = (q_lat, q_rope, kv). Returns ({f: idx}, [(out, lse)])."""
    pattern = layer_pattern(n_layers)
    src = shared_source(pattern)
    idx_of = {}
    outs = []
    for l in range(n_layers):
        if pattern[l] == "full":
            q_idx, w, k_idx = indexer_by_f[l]
            idx_of[l] = topk_select(indexer_score(q_idx, w, k_idx, q_seq, q_pos), q_pos, k)
        ql, qr, kv = mla_by_layer[l]
        outs.append(sparse_mla(ql, qr, kv, q_seq, idx_of[src[l]], scale))
    return idx_of, outs


__all__ = ["indexshare_group", "layer_stack", "indexer_inputs_fp8"]
