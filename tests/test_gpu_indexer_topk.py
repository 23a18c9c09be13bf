"""Selection without a score buffer (gsa_indexer_topk and the group call with no
score buffer) on the GPU, through the C ABI: indices bit-exact against the CPU
oracle on integer inputs, and bit-identical to the buffered path
(gsa_indexer_score + gsa_topk) on any inputs, since the rescored scores are the
score kernels' own arithmetic."""
import numpy as np
import pytest
import torch

import long_context_sparse_02_amd as gsa
import oracle
import workloads as W
from gpu_util import dev, np32, say

pytestmark = pytest.mark.gpu


def _inputs(wl, seed, dtype, q=None, k=None):
    q0, w = W.indexer_queries(wl, seed, 0)
    k0 = W.indexer_keys(wl, seed, 0)
    q = q0 if q is None else q
    k = k0 if k is None else k
    d = dev()
    if dtype == "fp8":
        qc, qs = gsa.quantize_e4m3(q.to(d))
        kc, ks = gsa.quantize_e4m3(k.to(d))
        return q, w, k, dict(q=qc, w=w.to(d), k=kc, q_scale=qs, k_scale=ks)
    return q, w, k, dict(q=q.to(d), w=w.to(d), k=k.to(d))


def _fused_and_buffered(args, q_seq, q_pos):
    d = dev()
    qs, qp = q_seq.to(d), q_pos.to(d)
    fused = gsa.indexer_topk(args["q"], args["w"], args["k"], qs, qp,
                             q_scale=args.get("q_scale"), k_scale=args.get("k_scale"))
    ld = (args["k"].shape[1] + 3) // 4 * 4
    gm = torch.empty((q_seq.numel(), gsa.group_max_ld(ld)), dtype=torch.float32, device=d)
    s = gsa.indexer_score(args["q"], args["w"], args["k"], qs, qp, q_scale=args.get("q_scale"),
                          k_scale=args.get("k_scale"), group_max=gm)
    buffered = gsa.topk(s, qp, group_max=gm)
    torch.cuda.synchronize()
    return np32(fused), np32(buffered)


@pytest.mark.parametrize("q_per_seq", [1, 2, 8, 16])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_indexer_topk_matches_oracle(dtype, q_per_seq):
    # rows of 70,001 positions (ragged, 5 chunks): the last queries of each
    # sequence have a bound (>= 2048 full groups); every kernel shape of the
    # score pass (1, 2, 8, 16 queries per sequence) writes the group maxima
    wl = W.Workload("fused", 2, 70_001, q_per_seq, 1, dtype)
    q, w, k, args = _inputs(wl, 11 + q_per_seq, dtype)
    q_seq, q_pos = W.query_layout(wl)
    fused, buffered = _fused_and_buffered(args, q_seq, q_pos)
    want = oracle.topk_select(oracle.indexer_score(np32(q), np32(w), np32(k), np32(q_seq), np32(q_pos)),
                              np32(q_pos), 2048)
    for i in range(wl.n_q):
        assert np.array_equal(fused[i], want[i]), f"{dtype} q/seq {q_per_seq} row {i}"
        assert np.array_equal(fused[i], buffered[i]), f"{dtype} q/seq {q_per_seq} row {i} vs buffered"
    say(f"indexer_topk {dtype}, {q_per_seq}/seq: {wl.n_q} rows match the oracle and the buffered path")


def test_indexer_topk_mixed_positions_and_short_rows():
    # unsorted sequences, positions below and above the bound threshold
    # (65,536), single-chunk rows (< 16,384 positions: final indices written
    # directly), a row of one position, chunk edges
    wl = W.Workload("mixed", 3, 100_000, 4, 1, "bf16")
    q, w, k, args = _inputs(wl, 5, "bf16")
    q_seq = torch.tensor([2, 0, 1, 2, 0, 1, 1, 0, 2, 0, 1, 2], dtype=torch.int32)
    q_pos = torch.tensor([99_999, 0, 16_383, 16_384, 65_534, 65_535, 65_536, 70_000, 2047, 2048,
                          31, 81_919], dtype=torch.int32)
    fused, buffered = _fused_and_buffered(args, q_seq, q_pos)
    want = oracle.topk_select(oracle.indexer_score(np32(q), np32(w), np32(k), np32(q_seq), np32(q_pos)),
                              np32(q_pos), 2048)
    for i in range(wl.n_q):
        assert np.array_equal(fused[i], want[i]), f"row {i} (pos {int(q_pos[i])})"
        assert np.array_equal(fused[i], buffered[i]), f"row {i} vs buffered"


def test_indexer_topk_all_ties():
    # q = 0: every score is 0, every group reaches the bound; the lowest 2048
    # positions win (ties to the lower position)
    wl = W.Workload("ties", 1, 90_000, 2, 1, "bf16")
    q0, _ = W.indexer_queries(wl, 3, 0)
    _, _, _, args = _inputs(wl, 3, "bf16", q=torch.zeros_like(q0))
    q_seq, q_pos = W.query_layout(wl)
    fused, buffered = _fused_and_buffered(args, q_seq, q_pos)
    assert np.array_equal(fused, np.tile(np.arange(2048, dtype=np.int32), (wl.n_q, 1)))
    assert np.array_equal(fused, buffered)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_indexer_topk_float_inputs_identical_to_buffered(dtype):
    # non-integer q, k and signed weights: the rescored scores are the score
    # kernel's bits, so both paths select the same positions
    wl = W.Workload("float", 2, 80_003, 3, 1, dtype)
    g = torch.Generator().manual_seed(17)
    q = torch.randn((wl.n_q, 32, 128), generator=g).to(torch.bfloat16)
    k = torch.randn((wl.batch, wl.n_ctx, 128), generator=g).to(torch.bfloat16)
    _, _, _, args = _inputs(wl, 17, dtype, q=q, k=k)
    args["w"] = (torch.rand((wl.n_q, 32), generator=g) * 2 - 0.5).to(dev())
    q_seq, q_pos = W.query_layout(wl)
    fused, buffered = _fused_and_buffered(args, q_seq, q_pos)
    assert np.array_equal(fused, buffered)


def test_indexer_topk_million_positions_fp8():
    # the 1M-position decode shape (2 sequences, one query each at the last
    # position): about 6% of the groups reach the bound
    wl = W.Workload("long", 2, 1 << 20, 1, 1, "fp8")
    q, w, k, args = _inputs(wl, 23, "fp8")
    q_seq, q_pos = W.query_layout(wl)
    fused, buffered = _fused_and_buffered(args, q_seq, q_pos)
    want = oracle.topk_select(oracle.indexer_score(np32(q), np32(w), np32(k), np32(q_seq), np32(q_pos)),
                              np32(q_pos), 2048)
    assert np.array_equal(fused, want)
    assert np.array_equal(fused, buffered)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_group_without_score_buffer(dtype):
    # the group call with no score buffer: indices as the buffered group's, and
    # attention over them as the oracle's
    wl = W.Workload("group_nobuf", 2, 70_001, 2, 2, dtype)
    g = W.group_inputs(wl, seed=31, n_layers=2)
    d = dev()
    layers = [tuple(t.to(d) for t in L) for L in g.layers]
    kw = dict(q_pos=g.q_pos.to(d), w=g.w.to(d))
    if dtype == "fp8":
        qc, qs = gsa.quantize_e4m3(g.q_idx.to(d))
        kc, ks = gsa.quantize_e4m3(g.k_idx.to(d))
        kw.update(q_idx=qc, k_idx=kc, q_scale=qs, k_scale=ks)
    else:
        kw.update(q_idx=g.q_idx.to(d), k_idx=g.k_idx.to(d))
    idx_f = torch.empty((wl.n_q, 2048), dtype=torch.int32, device=d)
    idx_b = torch.empty_like(idx_f)
    outs_f = gsa.indexshare_group(layers, g.q_seq.to(d), idx_f, score_buffer=False, **kw)
    outs_b = gsa.indexshare_group(layers, g.q_seq.to(d), idx_b, **kw)
    torch.cuda.synchronize()
    assert np.array_equal(np32(idx_f), np32(idx_b))

    def f(t):
        return t.float().numpy() if t.dtype == torch.bfloat16 else t.numpy()

    _, oidx, oouts = oracle.indexshare_group(f(g.q_idx), f(g.w), f(g.k_idx), f(g.q_seq), f(g.q_pos),
                                             [tuple(f(t) for t in L) for L in g.layers])
    assert np.array_equal(np32(idx_f), oidx)
    for (o, s), (ob, sb), (wo, ws) in zip(outs_f, outs_b, oouts):
        assert np.array_equal(np32(o), np32(ob))
        assert float(np.max(np.abs(np32(o) - wo))) <= 1e-2


@pytest.mark.parametrize("name", ["decode_b8_n1048576_fp8", "prefill_q4096_n131072_fp8", "decode_b64_n131072"])
def test_indexer_topk_full_size_identical_to_buffered(name):
    # the measured workloads at full size, from bench.py's own inputs: every
    # row's indices without a score buffer equal the buffered path's
    import bench
    wl = W.WORKLOADS[name]
    d = dev()
    inp = bench.build_inputs(wl, 0, d)
    q, w, k, qs, ks = inp["indexers"][0]
    fused = gsa.indexer_topk(q, w, k, inp["q_seq"], inp["q_pos"], q_scale=qs, k_scale=ks)
    ld = (wl.n_ctx + 3) // 4 * 4
    gm = torch.empty((wl.n_q, gsa.group_max_ld(ld)), dtype=torch.float32, device=d)
    s = gsa.indexer_score(q, w, k, inp["q_seq"], inp["q_pos"], q_scale=qs, k_scale=ks, group_max=gm)
    buffered = gsa.topk(s, inp["q_pos"], group_max=gm)
    torch.cuda.synchronize()
    assert torch.equal(fused, buffered)
    say(f"indexer_topk {name}: {wl.n_q} full-size rows identical to the buffered path")
