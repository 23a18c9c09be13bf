"""Paged latent caches on the GPU: the layers' caches live in pools of
fixed-size pages named by a per-sequence block table. Attention over a paged
cache must give the same bits as over the contiguous cache it was scattered
from (the kernel reads the same rows in the same order), and match the oracle
over the pool's logical view within the attention tolerance."""
import numpy as np
import pytest
import torch

import long_context_sparse_02_amd as gsa
import oracle
import workloads as W
from gpu_util import ATOL_LSE, ATOL_OUT, dev, max_abs, np32, say, note

pytestmark = pytest.mark.gpu


def _block_table(batch, max_pages, n_pages, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randperm(n_pages, generator=g)[:batch * max_pages].reshape(batch, max_pages).to(torch.int32)


def _to_pool(cache, page_size, bt, n_pages, seed):
    """Scatter a contiguous cache [B, N, 576] into a pool [n_pages, page_size, 576]
    at the pages bt names; the tail past N and unused pages hold noise."""
    B, N, D = cache.shape
    mp = bt.shape[1]
    g = torch.Generator().manual_seed(seed)
    padded = torch.randn((B, mp * page_size, D), generator=g).to(cache.dtype)
    padded[:, :N] = cache
    pool = torch.randn((n_pages, page_size, D), generator=g).to(cache.dtype)
    pool[bt.reshape(-1).long()] = padded.reshape(B * mp, page_size, D)
    return pool


@pytest.mark.parametrize("page_size,n_layers,n_q,batch", [(1, 2, 4, 2), (16, 3, 8, 2), (64, 4, 6, 3), (96, 1, 2, 1)])
def test_paged_attention_matches_contiguous_and_oracle(page_size, n_layers, n_q, batch):
    n_ctx = 3000
    mp = -(-n_ctx // page_size)
    n_pages = batch * mp + 5
    bt = _block_table(batch, mp, n_pages, page_size)
    g = torch.Generator().manual_seed(60 + page_size)
    q_seq = torch.arange(n_q, dtype=torch.int32) % batch
    idx = torch.stack([torch.sort(torch.randperm(n_ctx, generator=g)[:2048])[0] for _ in range(n_q)]).to(torch.int32)
    idx[0, 1900:] = -1                                              # a ragged row
    idx[-1, :8] = torch.arange(n_ctx - 8, n_ctx, dtype=torch.int32)  # last positions (last page)
    idx[-1] = torch.sort(torch.where(idx[-1] < 0, n_ctx, idx[-1]))[0]
    idx[-1] = torch.where(idx[-1] >= n_ctx, -1, idx[-1])
    wl = W.Workload("paged", batch, n_ctx, 1, 1, "bf16")
    layers_cpu, pools = [], []
    for l in range(n_layers):
        ql, qr = W.mla_queries(wl, 9, l)
        ql = ql[:1].repeat(n_q, 1, 1) + 0.25 * torch.randn((n_q, 64, 512), generator=g).to(torch.bfloat16)
        qr = qr[:1].repeat(n_q, 1, 1)
        kv = W.mla_cache(wl, 9, l)
        layers_cpu.append((ql, qr, kv))
        pools.append(_to_pool(kv, page_size, bt, n_pages, 100 + l))
    d = dev()
    contiguous = [tuple(t.to(d) for t in L) for L in layers_cpu]
    paged = [(ql.to(d), qr.to(d), p.to(d)) for (ql, qr, _), p in zip(layers_cpu, pools)]
    say(f"paged attention: page_size={page_size} layers={n_layers} n_q={n_q} batch={batch} pages={n_pages}")
    o_c = gsa.sparse_mla_attn_layers(contiguous, q_seq.to(d), idx.to(d), 1 / 16)
    o_p = gsa.sparse_mla_attn_paged(paged, bt.to(d), q_seq.to(d), idx.to(d), 1 / 16)
    torch.cuda.synchronize()
    for l, ((oc, sc), (op, sp), (ql, qr, _), pool) in enumerate(zip(o_c, o_p, layers_cpu, pools)):
        assert torch.equal(oc, op) and torch.equal(sc, sp), f"layer {l}: paged differs from contiguous"
        view = oracle.paged_cache_view(np32(pool), np32(bt), page_size)
        wo, ws = oracle.sparse_mla(np32(ql), np32(qr), view, np32(q_seq), np32(idx), 1 / 16)
        eo, el = max_abs(np32(op), wo), max_abs(np32(sp), ws)
        say(f"  layer {l}: out err {eo:.2e} lse err {el:.2e}")
        note(eo, el)
        assert eo <= ATOL_OUT and el <= ATOL_LSE


@pytest.mark.parametrize("page_size", [16, 100])
def test_paged_group_matches_contiguous(page_size):
    wl = W.Workload("paged_group", 3, 2500, 2, 4, "bf16")
    gi = W.group_inputs(wl, 2, n_layers=4)
    mp = -(-wl.n_ctx // page_size)
    n_pages = wl.batch * mp + 3
    bt = _block_table(wl.batch, mp, n_pages, page_size)
    d = dev()
    common = dict(q_pos=gi.q_pos.to(d), q_idx=gi.q_idx.to(d), w=gi.w.to(d), k_idx=gi.k_idx.to(d))
    layers = [tuple(t.to(d) for t in L) for L in gi.layers]
    paged = [(ql.to(d), qr.to(d), _to_pool(kv, page_size, bt, n_pages, 7 + l).to(d))
             for l, (ql, qr, kv) in enumerate(gi.layers)]
    idx_c = torch.full((wl.n_q, 2048), -7, dtype=torch.int32, device=d)
    idx_p = torch.full((wl.n_q, 2048), -7, dtype=torch.int32, device=d)
    say(f"paged group: page_size={page_size}, pages={n_pages}")
    o_c = gsa.indexshare_group(layers, gi.q_seq.to(d), idx_c, **common)
    o_p = gsa.indexshare_group(paged, gi.q_seq.to(d), idx_p, block_table=bt.to(d), **common)
    torch.cuda.synchronize()
    assert torch.equal(idx_c, idx_p)
    for (oc, sc), (op, sp) in zip(o_c, o_p):
        assert torch.equal(oc, op) and torch.equal(sc, sp)


def test_paged_stack_matches_contiguous():
    wl = W.Workload("paged_stack", 2, 3000, 3, 11, "bf16")
    n_layers, page_size = 11, 64
    src = oracle.shared_source(oracle.layer_pattern(n_layers))
    fulls = [l for l in range(n_layers) if src[l] == l]
    q_seq, q_pos = W.query_layout(wl)
    mp = -(-wl.n_ctx // page_size)
    n_pages = wl.batch * mp + 9
    bt = _block_table(wl.batch, mp, n_pages, page_size)
    d = dev()
    indexers = [(*(t.to(d) for t in W.indexer_queries(wl, 5, f)), W.indexer_keys(wl, 5, f).to(d), None, None)
                for f in fulls]
    mla_in = [(*W.mla_queries(wl, 5, l), W.mla_cache(wl, 5, l)) for l in range(n_layers)]
    layers = [tuple(t.to(d) for t in L) for L in mla_in]
    paged = [(ql.to(d), qr.to(d), _to_pool(kv, page_size, bt, n_pages, 30 + l).to(d))
             for l, (ql, qr, kv) in enumerate(mla_in)]
    buf_c = torch.full((len(fulls), wl.n_q, 2048), -7, dtype=torch.int32, device=d)
    buf_p = torch.full_like(buf_c, -7)
    say(f"paged stack: {n_layers} layers, page_size={page_size}")
    o_c = gsa.layer_stack(indexers, layers, q_seq.to(d), q_pos.to(d), buf_c)
    o_p = gsa.layer_stack(indexers, paged, q_seq.to(d), q_pos.to(d), buf_p, block_table=bt.to(d))
    torch.cuda.synchronize()
    assert torch.equal(buf_c, buf_p)
    for (oc, sc), (op, sp) in zip(o_c, o_p):
        assert torch.equal(oc, op) and torch.equal(sc, sp)
