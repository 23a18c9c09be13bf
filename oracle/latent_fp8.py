"""The FP8 latent cache row. Oracle only.

Pages: "GLM-5.2 总览" tbl-glm52-config (per token and layer the cache holds
1152 bytes in BF16, about 640 bytes in FP8 with one scale per tensor, about
656 bytes with per-group scales) and its glossary (KV FP8 is E4M3, applied to
the 512-dim MLA latent).

Reading (the pages give the byte counts, not the layout): a 656-byte row is
  [512 E4M3 codes of the latent | 4 float32 scales | 64 bf16 RoPE dims]
with the latent quantised in four 128-dim groups by the same block rule as the
indexer's FP8 variant (power-of-two scale, round to nearest even, saturating at
448; see e4m3.py) and the RoPE key kept in bf16 (512 + 16 + 128 = 656).
Attention over such a cache is attention over the dequantised rows.
"""
from __future__ import annotations

import numpy as np

from .e4m3 import dequantize_blocks, quantize_blocks

ROW_BYTES = 656


def _bf16_bits(x) -> np.ndarray:
    """float values that bf16 holds exactly -> their 16-bit patterns."""
    f = np.asarray(x, dtype=np.float32)
    bits = f.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "value is not a bf16"
    return (bits >> 16).astype(np.uint16)


def quantize_latent(rows) -> np.ndarray:
    """rows [..., 576] (bf16 values) -> uint8 [..., 656]."""
    rows = np.asarray(rows, dtype=np.float64)
    lead = rows.shape[:-1]
    codes, scales = quantize_blocks(rows[..., :512])                 # [..., 512], [..., 4]
    out = np.zeros(lead + (ROW_BYTES,), dtype=np.uint8)
    out[..., :512] = codes
    out[..., 512:528] = scales.astype("<f4").view(np.uint8).reshape(lead + (16,))
    out[..., 528:] = _bf16_bits(rows[..., 512:]).astype("<u2").view(np.uint8).reshape(lead + (128,))
    return out


def dequantize_latent(packed) -> np.ndarray:
    """uint8 [..., 656] -> float64 [..., 576]: codes x group scale, then RoPE."""
    p = np.ascontiguousarray(np.asarray(packed, dtype=np.uint8))
    lead = p.shape[:-1]
    scales = p[..., 512:528].copy().view("<f4").astype(np.float64).reshape(lead + (4,))
    lat = dequantize_blocks(p[..., :512], scales)
    rope = (p[..., 528:].copy().view("<u2").astype(np.uint32) << 16).view(np.float32)
    return np.concatenate([lat, rope.astype(np.float64).reshape(lead + (64,))], axis=-1)
