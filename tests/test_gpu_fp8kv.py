"""FP8 latent caches on the GPU: rows of [512 E4M3 | 4 fp32 scales | 64 bf16
RoPE] (656 bytes). The library's quantiser must write the oracle's bytes, and
attention over such a cache must be attention over the dequantised rows: bit
for bit where the result is a single row, within the attention tolerance
otherwise."""
import numpy as np
import pytest
import torch

import long_context_sparse_02_amd as gsa
import oracle
import workloads as W
from gpu_util import ATOL_LSE, ATOL_OUT, dev, max_abs, np32, say, note

pytestmark = pytest.mark.gpu


def _rows(n, seed):
    g = torch.Generator().manual_seed(seed)
    r = torch.randn((n, 576), generator=g) * torch.exp2(torch.randint(-12, 9, (n, 1), generator=g).float())
    r[0] = 0.0                                             # an all-zero row: scales 2^0, codes 0
    r[1, :128] = 448.0 * 2.0 ** -20                        # a group that hits 448 exactly
    r[2, 5] = 1e30                                         # a huge value in one group
    return r.to(torch.bfloat16)


def test_quantize_latent_matches_oracle():
    rows = _rows(1000, 1)
    got = gsa.quantize_latent_fp8(rows.to(dev())).cpu().numpy()
    want = oracle.quantize_latent(rows.float().numpy())
    bad = np.nonzero(np.any(got != want, axis=1))[0]
    assert bad.size == 0, f"rows {bad[:5]} differ"
    # a 3-D cache goes through unchanged in shape
    assert gsa.quantize_latent_fp8(rows.view(10, 100, 576).to(dev())).shape == (10, 100, 656)


def _attn_case(n_q, batch, n_ctx, n_layers, seed, one_row=False):
    g = torch.Generator().manual_seed(seed)
    q_seq = torch.arange(n_q, dtype=torch.int32) % batch
    if one_row:
        idx = torch.full((n_q, 2048), -1, dtype=torch.int32)
        idx[:, 0] = torch.randint(0, n_ctx, (n_q,), generator=g, dtype=torch.int32)
    else:
        idx = torch.stack([torch.sort(torch.randperm(n_ctx, generator=g)[:2048])[0] for _ in range(n_q)]).to(torch.int32)
        idx[0, 1500:] = -1
    wl = W.Workload("fp8kv", batch, n_ctx, 1, 1, "bf16")
    layers_cpu = []
    for l in range(n_layers):
        ql, qr = W.mla_queries(wl, seed, l)
        ql = ql[:1].repeat(n_q, 1, 1) + 0.25 * torch.randn((n_q, 64, 512), generator=g).to(torch.bfloat16)
        qr = qr[:1].repeat(n_q, 1, 1)
        kv = W.mla_cache(wl, seed, l)
        layers_cpu.append((ql, qr, kv))
    d = dev()
    layers = [(ql.to(d), qr.to(d), gsa.quantize_latent_fp8(kv.to(d))) for ql, qr, kv in layers_cpu]
    outs = gsa.sparse_mla_attn_layers(layers, q_seq.to(d), idx.to(d), 1 / 16)
    torch.cuda.synchronize()
    return q_seq, idx, layers_cpu, layers, outs


def test_fp8kv_one_row_is_the_dequantised_latent():
    # one valid index per query: the output is that row's dequantised latent,
    # which the widening must reproduce exactly
    q_seq, idx, layers_cpu, layers, outs = _attn_case(8, 2, 3000, 2, seed=3, one_row=True)
    for (o, s), (_, _, kv8) in zip(outs, layers):
        deq = oracle.dequantize_latent(kv8.cpu().numpy())
        for i in range(8):
            want = deq[int(q_seq[i]), int(idx[i, 0]), :512].astype(np.float32)
            assert np.array_equal(np32(o[i]), np.broadcast_to(want, (64, 512))), f"query {i}"


@pytest.mark.parametrize("n_q,batch,n_layers", [(4, 1, 1), (8, 2, 4), (64, 4, 2), (5, 5, 9)])
def test_fp8kv_attention_matches_oracle(n_q, batch, n_layers):
    q_seq, idx, layers_cpu, layers, outs = _attn_case(n_q, batch, 2500, n_layers, seed=n_q + n_layers)
    say(f"fp8 latent attention: n_q={n_q} batch={batch} layers={n_layers}")
    for l, ((o, s), (ql, qr, _), (_, _, kv8)) in enumerate(zip(outs, layers_cpu, layers)):
        deq = oracle.dequantize_latent(kv8.cpu().numpy())
        wo, ws = oracle.sparse_mla(np32(ql), np32(qr), deq, np32(q_seq), np32(idx), 1 / 16)
        eo, el = max_abs(np32(o), wo), max_abs(np32(s), ws)
        say(f"  layer {l}: out err {eo:.2e} lse err {el:.2e}")
        note(eo, el)
        assert eo <= ATOL_OUT and el <= ATOL_LSE


@pytest.mark.parametrize("n_q,batch,n_layers", [(64, 4, 2), (8, 2, 4)])
def test_fp8kv_attention_equals_bf16_attention_on_dequantised_rows(n_q, batch, n_layers):
    # 64 x 2: 1024-row slices, the row-pair layout, which computes on the FP8
    # rows in place (codes converted with their group scale for Q.K; V unscaled,
    # the scales carried by P); 8 x 4: 256-row slices, the dim-pair layout, which
    # widens each block first. Either way the MFMAs see the products of the
    # dequantised rows, so attention over the bf16 rows that dequantisation gives
    # (exact: a 4-bit significand times a power of two) is the same, bit for bit.
    q_seq, idx, layers_cpu, layers, outs = _attn_case(n_q, batch, 2500, n_layers, seed=40 + n_q)
    d = dev()
    deq_layers = []
    for (ql, qr, kv8) in layers:
        deq = torch.from_numpy(oracle.dequantize_latent(kv8.cpu().numpy()).astype(np.float32))
        assert torch.equal(deq.to(torch.bfloat16).float(), deq)          # exact in bf16
        deq_layers.append((ql, qr, deq.to(torch.bfloat16).to(d)))
    ref = gsa.sparse_mla_attn_layers(deq_layers, q_seq.to(d), idx.to(d), 1 / 16)
    torch.cuda.synchronize()
    for l, ((o, s), (ro, rs)) in enumerate(zip(outs, ref)):
        assert torch.equal(o, ro) and torch.equal(s, rs), f"layer {l}: max |diff| {float((o - ro).abs().max()):.3e}"


def test_fp8kv_paged_matches_contiguous():
    q_seq, idx, layers_cpu, layers, outs = _attn_case(6, 3, 2500, 2, seed=11)
    ps = 32
    mp = -(-2500 // ps)
    n_pages = 3 * mp + 4
    bt = torch.randperm(n_pages, generator=torch.Generator().manual_seed(12))[:3 * mp].reshape(3, mp).to(torch.int32)
    d = dev()
    paged = []
    for ql, qr, kv8 in layers:
        pool = torch.zeros((n_pages, ps, 656), dtype=torch.uint8, device=d)
        padded = torch.zeros((3, mp * ps, 656), dtype=torch.uint8, device=d)
        padded[:, :2500] = kv8
        pool[bt.reshape(-1).long().to(d)] = padded.reshape(3 * mp, ps, 656)
        paged.append((ql, qr, pool))
    o_p = gsa.sparse_mla_attn_paged(paged, bt.to(d), q_seq.to(d), idx.to(d), 1 / 16)
    torch.cuda.synchronize()
    for (oc, sc), (op, sp) in zip(outs, o_p):
        assert torch.equal(oc, op) and torch.equal(sc, sp)


def test_fp8kv_group_and_stack_match_oracle():
    wl = W.Workload("fp8kv_group", 2, 3000, 3, 4, "bf16")
    gi = W.group_inputs(wl, 6, n_layers=4)
    d = dev()
    layers = [(ql.to(d), qr.to(d), gsa.quantize_latent_fp8(kv.to(d))) for ql, qr, kv in gi.layers]
    idx = torch.full((wl.n_q, 2048), -7, dtype=torch.int32, device=d)
    outs = gsa.indexshare_group(layers, gi.q_seq.to(d), idx, q_pos=gi.q_pos.to(d), q_idx=gi.q_idx.to(d),
                                w=gi.w.to(d), k_idx=gi.k_idx.to(d))
    torch.cuda.synchronize()
    deq = [(np32(ql), np32(qr), oracle.dequantize_latent(kv8.cpu().numpy())) for (ql, qr, _), (_, _, kv8)
           in zip(gi.layers, layers)]
    _, oidx, oouts = oracle.indexshare_group(np32(gi.q_idx), np32(gi.w), np32(gi.k_idx), np32(gi.q_seq),
                                             np32(gi.q_pos), deq)
    assert np.array_equal(np32(idx), oidx)
    for (o, s), (wo, ws) in zip(outs, oouts):
        eo, el = max_abs(np32(o), wo), max_abs(np32(s), ws)
        note(eo, el)
        assert eo <= ATOL_OUT and el <= ATOL_LSE


def test_fp8kv_row_pair_layout_rescales_and_edge_rows():
    # The row-pair layout on FP8 rows in place, under the conditions that stress
    # it: 4 layers x 32 queries split into two 1024-row slices; RoPE keys that
    # grow with the position (the running max moves block after block, in one or
    # both row halves at once), one query in descending order; edge rows (every
    # index -1, a single valid index, one row half of every block empty). The
    # result must be bf16 attention over the dequantised rows, bit for bit, with
    # the empty query's output zero and its lse -inf.
    n_layers, n_q, batch, n_ctx = 4, 32, 2, 5000
    wl = W.Workload("fp8kv_rp", batch, n_ctx, n_q // batch, n_layers, "bf16")
    q_seq = torch.arange(n_q, dtype=torch.int32) % batch
    g = torch.Generator().manual_seed(93)
    idx = torch.stack([torch.sort(torch.randperm(n_ctx, generator=g)[:2048])[0] for _ in range(n_q)]).to(torch.int32)
    idx[1] = torch.flip(idx[1], [0])
    idx[2] = -1
    idx[3] = -1
    idx[3, 700] = 4321
    second_half = (torch.arange(2048) // 16) % 2 == 1
    idx[4, second_half] = -1
    idx[5, ~second_half] = -1
    grow = 1.0 + torch.arange(n_ctx, dtype=torch.float32) / 500.0
    d = dev()
    layers, deq_layers = [], []
    for l in range(n_layers):
        ql, qr = W.mla_queries(wl, 11, l)
        kv = W.mla_cache(wl, 11, l).float()
        kv[..., 512:] *= grow[None, :, None]
        kv8 = oracle.quantize_latent(kv.to(torch.bfloat16).float().numpy())
        deq = torch.from_numpy(oracle.dequantize_latent(kv8).astype(np.float32))
        assert torch.equal(deq.to(torch.bfloat16).float(), deq)          # exact in bf16
        layers.append((ql.to(d), qr.to(d), torch.from_numpy(kv8).to(d)))
        deq_layers.append((ql.to(d), qr.to(d), deq.to(torch.bfloat16).to(d)))
    outs = gsa.sparse_mla_attn_layers(layers, q_seq.to(d), idx.to(d), 1 / 16)
    ref = gsa.sparse_mla_attn_layers(deq_layers, q_seq.to(d), idx.to(d), 1 / 16)
    torch.cuda.synchronize()
    for l, ((o, s), (ro, rs)) in enumerate(zip(outs, ref)):
        assert torch.equal(o, ro) and torch.equal(s, rs), f"layer {l}: max |diff| {float((o - ro).abs().max()):.3e}"
        assert torch.all(o[2] == 0) and torch.all(torch.isneginf(s[2]))
    say("FP8 row-pair layout: 4 layers bit-identical to bf16 attention on the dequantised rows")
