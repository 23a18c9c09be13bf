"""gsa_indexshare_group_noalloc (the group call on the library's static scratch,
for callers that cannot allocate) against gsa_indexshare_group: two calls in a
row, the second on a smaller group, each identical to the workspace call."""
import ctypes

import numpy as np
import pytest
import torch

import long_context_sparse_02_amd as gsa
import oracle
import workloads as W
from gpu_util import ATOL_LSE, ATOL_OUT, dev, max_abs, np32, say, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gsa.lib()


def _group(wl, seed, noalloc, n_layers=4):
    """One group on the device; noalloc: through the static scratch, with every
    output and the score buffer passed in."""
    g = W.group_inputs(wl, seed, n_layers=n_layers)
    d = dev()
    layers = [tuple(t.to(d) for t in L) for L in g.layers]
    idx = torch.full((wl.n_q, 2048), -7, dtype=torch.int32, device=d)
    scores = torch.empty((wl.n_q, (wl.n_ctx + 3) // 4 * 4), dtype=torch.float32, device=d)
    outs = [(torch.full((wl.n_q, 64, 512), 7.0, device=d), torch.full((wl.n_q, 64), 7.0, device=d))
            for _ in layers]
    gsa.indexshare_group(layers, g.q_seq.to(d), idx, q_pos=g.q_pos.to(d), q_idx=g.q_idx.to(d), w=g.w.to(d),
                         k_idx=g.k_idx.to(d), scores=scores, outs=outs, noalloc=noalloc)
    torch.cuda.synchronize()
    return g, idx, outs


def test_noalloc_group_matches_the_workspace_call_twice():
    # first a group of 16 queries over 70,001 positions (one work-group per row
    # for the top-k, attention split across work-groups: partial results in the
    # scratch), then a smaller one of 3 queries over 20,000 positions (chunk lists
    # and their merge in the scratch, a different split)
    assert gsa.lib().gsa_noalloc_scratch_bytes() == 64 << 20
    for wl, seed in ((W.Workload("noalloc_a", 8, 70_001, 2, 4, "bf16"), 3),
                     (W.Workload("noalloc_b", 3, 20_000, 1, 4, "bf16"), 4)):
        say(f"no-alloc group: n_q={wl.n_q}, N={wl.n_ctx}")
        g, idx_n, outs_n = _group(wl, seed, noalloc=True)
        _, idx_w, outs_w = _group(wl, seed, noalloc=False)
        assert torch.equal(idx_n, idx_w)
        for (on, sn), (ow, sw) in zip(outs_n, outs_w):
            assert torch.equal(on, ow) and torch.equal(sn, sw)
        # and the oracle on the first query of each sequence
        want_idx = oracle.topk_select(
            oracle.indexer_score(np32(g.q_idx), np32(g.w), np32(g.k_idx), np32(g.q_seq), np32(g.q_pos)),
            np32(g.q_pos), 2048)
        assert np.array_equal(np32(idx_n), want_idx)
        for l, (ql, qr, kv) in enumerate(g.layers):
            o, s = oracle.sparse_mla(np32(ql), np32(qr), np32(kv), np32(g.q_seq), want_idx, 1 / 16)
            eo, el = max_abs(np32(outs_n[l][0]), o), max_abs(np32(outs_n[l][1]), s)
            note(eo, el)
            assert eo <= ATOL_OUT and el <= ATOL_LSE


def test_noalloc_group_rejects_what_the_scratch_cannot_hold():
    # 4096 queries over 131,072 positions need more than 64 MiB of top-k lists:
    # refused on the host, nothing enqueued
    L = gsa.lib()
    layers = (gsa._MlaLayer * 1)()
    layers[0] = gsa._MlaLayer(0x10000, 0x10000, 0x10000, 0x10000, None)
    d = gsa._GroupDesc()
    d.compute_index, d.dt = 1, 0
    d.q_idx_dev = d.w_dev = d.k_idx_dev = d.scores_dev = d.q_pos_dev = 0x10000
    d.q_seq_dev = d.index_buf_dev = 0x10000
    d.ld_scores = 131072
    d.n_q, d.batch, d.n_cap, d.k = 4096, 1, 131072, 2048
    d.n_layers, d.layers = 1, ctypes.cast(layers, ctypes.POINTER(gsa._MlaLayer))
    d.n_heads, d.scale = 64, 1 / 16
    assert L.gsa_indexshare_group_noalloc(ctypes.byref(d), None) == 3        # GSA_ERR_WORKSPACE
    assert b"static scratch" in L.gsa_last_error()
