"""The 78-layer indexer_types pattern of IndexShare. Oracle only.

Pages: "GLM-5.2 架构深度拆解" CH2 §2.1 table — layers 0, 1, 2 are full; then
3 shared; then one full every 4 layers (6, 10, ..., 74), each followed by 3
shared; 21 full + 57 shared in all; layers 3-5 reuse layer 2's indices;
§1.2 (index_topk_freq = 4).

Reading: §1.3's diagram says layer 77 reuses "L76", but §2.1's table makes
layer 76 shared and 74 full, so an S layer reuses the latest full layer
before it (77 -> 74).
"""
from __future__ import annotations


def layer_pattern(n_layers: int = 78, n_lead_full: int = 3, freq: int = 4):
    """List of "full"/"shared" per layer."""
    out = []
    for i in range(n_layers):
        if i < n_lead_full or (i - (n_lead_full - 1)) % freq == 0:
            out.append("full")
        else:
            out.append("shared")
    return out


def shared_source(pattern):
    """For every layer, the full layer whose indices it uses (itself if full)."""
    src = []
    last = None
    for i, t in enumerate(pattern):
        if t == "full":
            last = i
        if last is None:
            raise ValueError("the first layer must be full")
        src.append(last)
    return src
