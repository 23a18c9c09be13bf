"""The Hadamard-rotated FP8 indexer on the GPU: the rotated quantiser writes
the oracle's codes and scales (bit-exact on integer inputs, where every sum is
exact in fp32), and the fp8 score kernel on rotated codes matches the oracle's
score of the dequantised rotated q and k."""
import numpy as np
import pytest
import torch

import long_context_sparse_02_amd as gsa
import oracle
import workloads as W
from gpu_util import dev, np32, say

pytestmark = pytest.mark.gpu


def test_rotated_quantiser_bit_exact_on_integer_inputs():
    wl = W.Workload("had", 2, 3000, 5, 1, "fp8")
    q, _ = W.indexer_queries(wl, 3, 0)
    k = W.indexer_keys(wl, 3, 0)
    for name, x in (("q", q), ("k", k)):
        codes, scales = gsa.quantize_e4m3(x.to(dev()), hadamard=True)
        oc, osc = oracle.quantize_blocks_hadamard(np32(x))
        assert np.array_equal(np32(scales).astype(np.float64), osc[..., 0]), f"{name} scales"
        assert np.array_equal(np32(codes), oc), f"{name} codes"


def test_rotated_quantiser_on_float_inputs():
    # bf16 N(0,1) blocks with spread exponents: the kernel's staged float32
    # butterflies may differ from the oracle's once-rounded sums in the last
    # bits, within the bound of tests/rounding.py; every code and scale whose
    # decision that bound fixes must be the oracle's exactly
    import rounding
    g = torch.Generator().manual_seed(8)
    x = (torch.randn((4096, 128), generator=g) * torch.exp2(torch.randint(-6, 6, (4096, 1), generator=g).float()))
    x = x.to(torch.bfloat16)
    codes, scales = gsa.quantize_e4m3(x.to(dev()), hadamard=True)
    n, n_open, n_scale_open = rounding.check_rotated_codes(np32(codes), np32(scales), np32(x))
    say(f"rotated codes: {n} compared, {n_open} at an open boundary, {n_scale_open} blocks with an open scale")
    assert n >= x.numel() - 128 * n_scale_open          # only blocks with an open scale may be skipped


def test_rotated_fp8_score_and_topk():
    wl = W.Workload("had_score", 2, 5000, 3, 1, "fp8")
    q, w = W.indexer_queries(wl, 4, 0)
    k = W.indexer_keys(wl, 4, 0)
    q_seq, q_pos = W.query_layout(wl)
    d = dev()
    qc, qs = gsa.quantize_e4m3(q.to(d), hadamard=True)
    kc, ks = gsa.quantize_e4m3(k.to(d), hadamard=True)
    scores = gsa.indexer_score(qc, w.to(d), kc, q_seq.to(d), q_pos.to(d), q_scale=qs, k_scale=ks)
    idx = gsa.topk(scores, q_pos.to(d))
    torch.cuda.synchronize()
    qr, kr = oracle.indexer_inputs_fp8_hadamard(np32(q), np32(k))
    want = oracle.indexer_score(qr, np32(w), kr, np32(q_seq), np32(q_pos))
    got = np32(scores)[:, :wl.n_ctx].astype(np.float64)
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin)
    # fp32 accumulation of exact e4m3 products; a ReLU argument within rounding of
    # zero can land on either side
    err = np.abs(got[fin] - want[fin])
    assert np.all(err <= 1e-4 * (1.0 + np.abs(want[fin]))), err.max()
    # the selection is exact for the scores it was given
    assert np.array_equal(np32(idx), oracle.topk_select(np32(scores), np32(q_pos), 2048))
    # and it differs from the oracle's own selection only among positions whose
    # oracle scores the 1e-4 bound leaves at the threshold
    import rounding
    for i in range(wl.n_q):
        rounding.check_selection_within_bound(np32(idx)[i], want[i], 2048, 1e-4)
