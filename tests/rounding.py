"""Exact checks of FP8 codes whose inputs were rounded in stages (test
infrastructure, not part of the library).

The rotated quantiser adds the 128 elements of a block in seven butterfly
stages of float32 adds and subtracts, then multiplies by the float32 value of
1/sqrt(128); the oracle rounds the exact +-1 sum once and multiplies the same
way. Standard floating-point error analysis bounds the difference of the two
rotated values: each stage rounds a partial sum whose magnitude is at most
sum|x| of the block, so the staged sum is within 7 u sum|x| of the exact one
(u = 2^-24), the oracle's single rounding adds u sum|x|, and the two final
multiplies add u |y| each, with |y| <= c sum|x| (c = fl(1/sqrt(128))). So

    |y_staged - y_oracle| <= (7 + 1 + 2) u c sum|x|   (taken with a 10% margin).

An FP8 decision (a code, or a block's power-of-two scale) taken from y_staged
must then equal the oracle's wherever the whole interval y_oracle +- delta
falls on one side of every rounding boundary; where it straddles one, any
code between those of the interval's two ends is correct (rounding is
monotone).
"""
from __future__ import annotations

import numpy as np

import oracle
from oracle.e4m3 import block_exponent, e4m3_encode

U32 = 2.0 ** -24


def staged_rotation_bound(x, block: int = 128, stages: int = 7) -> np.ndarray:
    """delta per block (shape x.shape[:-1] + (n_blocks,)) for the bound above."""
    xb = np.abs(np.asarray(x, np.float64)).reshape(np.shape(x)[:-1] + (-1, block))
    c = float(np.float32(1.0 / np.sqrt(block)))
    return 1.1 * (stages + 3) * U32 * c * xb.sum(axis=-1)


def check_rotated_codes(got_codes, got_scales, x, block: int = 128):
    """Assert that (got_codes, got_scales) are the oracle's rotated FP8 codes and
    scales of x, exactly, except where the bound leaves the decision open.
    Returns (codes compared, codes at an open boundary, blocks with an open scale)."""
    y = oracle.rotate_blocks(x, block).astype(np.float64)
    oc, osc = oracle.quantize_blocks(y, block)
    lead = y.shape[:-1]
    yb = y.reshape(lead + (-1, block))
    ocb = oc.reshape(yb.shape).astype(np.int64)
    gotb = np.asarray(got_codes).reshape(yb.shape).astype(np.int64)
    gs = np.asarray(got_scales, np.float64).reshape(osc.shape)
    delta = staged_rotation_bound(x, block)

    # scales: the oracle's block maximum within delta of a power-of-two step
    # leaves the exponent open
    amax = np.max(np.abs(yb), axis=-1)
    scale_open = block_exponent(np.maximum(amax - delta, 0.0)) != block_exponent(amax + delta)
    same_scale = gs == osc
    assert np.all(same_scale | scale_open), "a block scale differs where the bound fixes it"

    # codes of the blocks that took the oracle's scale
    s = osc[..., None]
    lo = e4m3_encode((yb - delta[..., None]) / s).astype(np.int64)
    hi = e4m3_encode((yb + delta[..., None]) / s).astype(np.int64)
    fixed = lo == hi
    rows = same_scale[..., None] & np.ones_like(fixed)
    exact = rows & fixed
    assert np.array_equal(gotb[exact], ocb[exact]), (
        f"{int(np.count_nonzero(gotb[exact] != ocb[exact]))} codes differ where the bound fixes them")
    # rounding is monotone, so a value in [y - delta, y + delta] takes a code
    # whose value lies between those of the interval's two ends
    open_ = rows & ~fixed
    gv = oracle.e4m3_decode(gotb[open_].astype(np.uint8))
    assert np.all((gv >= oracle.e4m3_decode(lo[open_].astype(np.uint8)))
                  & (gv <= oracle.e4m3_decode(hi[open_].astype(np.uint8)))), \
        "a code at an open boundary lies outside the interval's codes"
    return int(np.count_nonzero(rows)), int(np.count_nonzero(open_)), int(np.count_nonzero(scale_open))


def staged_rotation_fp32(x, block: int = 128) -> np.ndarray:
    """A staged float32 rotation (the standard in-place fast Walsh-Hadamard
    transform, butterfly distances 1, 2, ..., block/2, every add and subtract
    rounded to float32, then one float32 multiply by fl(1/sqrt(block))): a
    second computation with the staging the bound is about, for checking the
    bound itself on the CPU."""
    v = np.asarray(x, np.float32).reshape(np.shape(x)[:-1] + (-1, block)).copy()
    h = 1
    while h < block:
        w = v.reshape(v.shape[:-1] + (block // (2 * h), 2, h))
        a, b = w[..., 0, :].copy(), w[..., 1, :].copy()
        w[..., 0, :] = a + b
        w[..., 1, :] = a - b
        v = w.reshape(v.shape)
        h *= 2
    return (v * np.float32(1.0 / np.sqrt(block))).reshape(np.shape(x))


def check_selection_within_bound(have, want, k: int, tau: float) -> int:
    """have: the positions a kernel selected from its own scores of one row;
    want: the oracle's scores of that row (float64, -inf where masked), every
    kernel score lying within tau (1 + |want|) of the oracle's. With T the
    oracle's k-th largest score, and lo(w) = w - tau (1 + |w|), up(w) = w +
    tau (1 + |w|) (both increasing in w): at most k - 1 positions score above
    T, and no position at or below T can score above up(T) on the kernel's
    side, so every position with lo(w) > up(T) is selected; at least k
    positions score at T or above, all at lo(T) or above on the kernel's side,
    so no position with up(w) < lo(T) is selected. Asserts both; returns the
    number of positions in the band between, where either choice is correct."""
    want = np.asarray(want, np.float64)
    fin = np.isfinite(want)
    sel = np.array(sorted(set(int(v) for v in np.asarray(have).ravel()) - {-1}), np.int64)
    n_fin = int(np.count_nonzero(fin))
    if n_fin <= k:
        assert np.array_equal(sel, np.nonzero(fin)[0]), "every causal position is selected"
        return 0
    assert sel.size == k, f"{sel.size} positions selected, {k} expected"
    t = np.sort(want[fin])[-k]
    up = lambda w: w + tau * (1.0 + np.abs(w))
    lo = lambda w: w - tau * (1.0 + np.abs(w))
    must = np.nonzero(fin & (lo(np.where(fin, want, 0.0)) > up(t)))[0]
    assert np.all(np.isin(must, sel)), "a position clearly above the k-th score is not selected"
    assert np.all(fin[sel]) and np.all(up(want[sel]) >= lo(t)), "a position clearly below the k-th score is selected"
    band = fin & (up(np.where(fin, want, 0.0)) >= lo(t)) & (lo(np.where(fin, want, 0.0)) <= up(t))
    return int(np.count_nonzero(band))
