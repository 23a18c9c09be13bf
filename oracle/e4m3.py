"""FP8 E4M3 (OCP "fn" variant) codec and per-block quantisation. Oracle only.

Pages: the indexer's q/k are quantised to FP8 per block ("GLM-5.2 总览",
sub-document index row 02: FP8 per-block), and the glossary states that the
FP8 in use is E4M3, not INT8.

Reading (the pages give the format, not the block or scale rule):
  * A block is one 128-element vector: one indexer key row, or one (query,
    head) query vector.
  * The scale is a power of two, 2**e with e the smallest integer such that
    amax <= 448 * 2**e, clamped to [-126, 127]; e = 0 for an all-zero block.
  * Codes are x / scale rounded to nearest, ties to even, in E4M3FN
    (bias 7, no infinities, 0x7F/0xFF are NaN, max finite 448), saturating at
    +-448. Power-of-two scales keep integer inputs exact.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_BIAS = 7


def e4m3_decode(codes) -> np.ndarray:
    """uint8 codes -> float64 values, straight from the bit fields."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    sub = man.astype(np.float64) * 2.0 ** (1 - _BIAS - 3)           # E = 0
    nor = (1.0 + man / 8.0) * np.power(2.0, exp.astype(np.float64) - _BIAS)
    val = np.where(exp == 0, sub, nor)
    val = np.where((exp == 0xF) & (man == 0x7), np.nan, val)
    return sign * val


def e4m3_encode(x) -> np.ndarray:
    """float -> uint8 E4M3FN code, round to nearest even, saturating at 448."""
    x = np.asarray(x, dtype=np.float64)
    nan = np.isnan(x)
    sign = np.where(np.signbit(x), 0x80, 0x00).astype(np.int64)
    a = np.where(nan, 0.0, np.abs(x))
    # subnormal range a < 2^-6: multiples of 2^-9; a rounded count of 8 is
    # exactly the smallest normal's code, so the formula carries over by itself
    sub_code = np.round(a / 2.0 ** (1 - _BIAS - 3)).astype(np.int64)   # half to even
    # normal range: a = 2^e * (1 + f), keep 3 fraction bits
    _, ex = np.frexp(np.where(a > 0.0, a, 1.0))
    e = ex.astype(np.int64) - 1                                        # a in [2^e, 2^(e+1))
    r = np.round(a / np.exp2((e - 3).astype(np.float64))).astype(np.int64)   # in [8, 16]
    carry = r == 16
    e = e + carry
    r = np.where(carry, 8, r)
    nor_code = ((e + _BIAS) << 3) | (r - 8)
    code = np.where(a < 2.0 ** (1 - _BIAS), sub_code, nor_code)
    code = np.where(a >= E4M3_MAX, 0x7E, np.minimum(code, 0x7E))
    out = (sign | code).astype(np.uint8)
    return np.where(nan, np.uint8(0x7F), out).astype(np.uint8)


def block_exponent(amax) -> np.ndarray:
    """Smallest e with amax <= 448 * 2**e, clamped to [-126, 127] (0 where amax == 0)."""
    amax = np.asarray(amax, dtype=np.float64)
    safe = np.where(amax > 0.0, amax, E4M3_MAX)
    e = np.ceil(np.log2(safe / E4M3_MAX))
    e = np.where(safe > E4M3_MAX * np.exp2(e), e + 1, e)        # repair log2 rounding
    e = np.where(safe <= E4M3_MAX * np.exp2(e - 1), e - 1, e)
    e = np.clip(e, -126, 127)
    return np.where(amax > 0.0, e, 0.0).astype(np.int64)


def quantize_blocks(x, block: int = 128):
    """Quantise the last axis of x in blocks of `block` elements.

    Returns (codes uint8, same shape as x; scales float64 [..., n_blocks])."""
    x = np.asarray(x, dtype=np.float64)
    assert x.shape[-1] % block == 0
    nb = x.shape[-1] // block
    xb = x.reshape(x.shape[:-1] + (nb, block))
    e = block_exponent(np.max(np.abs(xb), axis=-1))
    scales = np.exp2(e.astype(np.float64))
    codes = e4m3_encode(xb / scales[..., None])
    return codes.reshape(x.shape), scales


def dequantize_blocks(codes, scales, block: int = 128) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.float64)
    nb = codes.shape[-1] // block
    vals = e4m3_decode(codes).reshape(codes.shape[:-1] + (nb, block))
    return (vals * scales[..., None]).reshape(codes.shape)
