"""Hadamard rotation before per-block FP8. Oracle only.

Pages: "GLM-5.2 总览" sub-document index (row 02) lists, among the lightning
indexer's steps, FP8 per-block quantisation together with a Hadamard rotation;
the pages give no further detail.

Reading: each 128-element block x (a key row, or one (query, head) vector) is
replaced by y = H x / sqrt(128) before quantisation, H the Sylvester-ordered
Hadamard matrix (H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]), which is
orthogonal up to the factor 128, so rotating both q and k keeps every q . k in
exact arithmetic. Precision (the pages are silent; the decision of each FP8
code is taken in the GPU's precision): the +-1 sum is rounded once to float32
and multiplied, in float32, by the float32 value of 1/sqrt(128). The rotated
block is then quantised by the rule of e4m3.py.
"""
from __future__ import annotations

import numpy as np

from .e4m3 import dequantize_blocks, quantize_blocks


def hadamard(n: int) -> np.ndarray:
    """Sylvester-ordered n x n Hadamard matrix (n a power of two), int64."""
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    assert h.shape[0] == n, "n must be a power of two"
    return h


def rotate_blocks(x, block: int = 128) -> np.ndarray:
    """H x / sqrt(block) over the last axis in blocks, float32 as described."""
    x = np.asarray(x, dtype=np.float64)
    h = hadamard(block).astype(np.float64)
    xb = x.reshape(x.shape[:-1] + (x.shape[-1] // block, block))
    sums = np.einsum("ij,...j->...i", h, xb).astype(np.float32)      # exact sum, rounded once
    y = sums * np.float32(1.0 / np.sqrt(block))                      # one float32 multiply
    return y.reshape(x.shape)


def quantize_blocks_hadamard(x, block: int = 128):
    """Rotate, then quantise: (codes uint8, scales float64), as quantize_blocks."""
    return quantize_blocks(rotate_blocks(x, block).astype(np.float64), block)


def indexer_inputs_fp8_hadamard(q_idx, k_idx):
    """What the rotated FP8 indexer scores: the dequantised rotated q and k."""
    qc, qs = quantize_blocks_hadamard(q_idx)
    kc, ks = quantize_blocks_hadamard(k_idx)
    return dequantize_blocks(qc, qs), dequantize_blocks(kc, ks)
