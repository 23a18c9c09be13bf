"""Helpers shared by the GPU parity tests (marshalling between torch and numpy)."""
import os
import sys

import numpy as np
import torch

# Attention tolerance: bf16 inputs, fp32 accumulation, P rounded to bf16 before
# P.V (relative error <= 2^-8 per weight, the bf16 unit roundoff); on unit-scale
# caches the outputs are O(0.1) and the rounding errors of many weights average
# out, so the expected max-abs error is ~1e-3. The bar is 1e-2 max-abs (a test
# whose data make the softmax peaked states its own bound).
ATOL_OUT = 1e-2
ATOL_LSE = 1e-2


def np32(t):
    """torch (any device) -> numpy float32 (bf16 widens exactly); ints stay ints."""
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.float()
    return t.numpy()


def dev():
    return torch.device("cuda", 0)


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def assert_scores_equal(gpu_row, oracle_row, label=""):
    g = np.asarray(gpu_row, dtype=np.float64)
    o = np.asarray(oracle_row, dtype=np.float64)
    bad = np.nonzero(~((g == o) | (np.isneginf(g) & np.isneginf(o))))[0]
    assert bad.size == 0, f"{label}: {bad.size} mismatches, first at {bad[:5]}: gpu {g[bad[:5]]} oracle {o[bad[:5]]}"


def max_abs(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):                  # inf - inf where both_inf masks it
        d = np.where(both_inf, 0.0, np.abs(a - b))
    return float(np.max(d)) if d.size else 0.0


# Largest attention errors against the oracle per test (printed at the end of the
# run by conftest.py, so that a run's log records the margin under the bar).
ERRORS = {}


def note(eo, el=0.0, bar=ATOL_OUT):
    """Record the max-abs output and lse errors of an attention check for the
    running test, with the output bar it was held to."""
    label = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    a, b, c = ERRORS.get(label, (0.0, 0.0, float(bar)))
    ERRORS[label] = (max(a, float(eo)), max(b, float(el)), min(c, float(bar)))
