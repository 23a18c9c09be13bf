"""Parity at the workloads' full sizes, in the launch configuration bench.py
times (its own input builder and call sequence), on one MI355X.

The oracle cannot recompute every output at these sizes, so:
  * for every query, properties that pin the selection at any size: the count
    is min(2048, pos + 1), indices ascending in [0, pos] with -1 after them,
    no unselected causal score above the smallest selected one, ties at that
    threshold kept at the lowest positions, and -inf past each query's position;
  * for sampled queries, the oracle recomputes the score row (bit-exact: the
    indexer inputs are integers), the top-2048 set (bit-exact) and each checked
    layer's attention output and lse (1e-2 max-abs) from host copies of the
    same device inputs.
"""
import numpy as np
import pytest
import torch

import bench
import long_context_sparse_02_amd as gsa
import oracle
import rounding
import workloads as W
from gpu_util import ATOL_LSE, ATOL_OUT, assert_scores_equal, dev, max_abs, np32, say, note

pytestmark = pytest.mark.gpu
SEED = 11


@pytest.fixture(autouse=True)
def _release_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def check_selection_properties(scores, idx, q_pos, n_ctx, rows_per_chunk=256):
    """Properties of idx [n_q, 2048] against the scores it was selected from."""
    n_q = idx.shape[0]
    for r0 in range(0, n_q, rows_per_chunk):
        r1 = min(n_q, r0 + rows_per_chunk)
        sc = scores[r0:r1, :n_ctx]
        ix = idx[r0:r1].long()
        pos = q_pos[r0:r1].long()[:, None]
        valid = ix >= 0
        n_valid = valid.sum(1, keepdim=True)
        assert torch.equal(n_valid, torch.clamp(pos + 1, max=2048)), "selection count"
        slot = torch.arange(2048, device=ix.device)[None]
        assert torch.equal(valid, slot < n_valid), "-1 padding only after the indices"
        assert bool(((ix <= pos) | ~valid).all()), "index beyond the query's position"
        inc = (ix[:, 1:] > ix[:, :-1]) | ~valid[:, 1:]
        assert bool(inc.all()), "indices not strictly ascending"
        col = torch.arange(n_ctx, device=sc.device)[None]
        causal = col <= pos
        assert bool(torch.isneginf(sc[~causal]).all()), "score past the position is not -inf"
        sel = torch.zeros_like(causal)
        sel.scatter_(1, ix.clamp(min=0), valid)
        ninf = torch.tensor(float("-inf"), device=sc.device)
        pinf = torch.tensor(float("inf"), device=sc.device)
        t_sel = torch.where(sel, sc, pinf).amin(1, keepdim=True)           # smallest selected
        unsel = causal & ~sel
        t_uns = torch.where(unsel, sc, ninf).amax(1, keepdim=True)         # largest unselected
        assert bool((t_uns <= t_sel).all()), "an unselected score exceeds a selected one"
        # ties at the threshold: every selected copy sits below every unselected copy
        big = torch.tensor(n_ctx, device=sc.device)
        last_sel = torch.where(sel & (sc == t_sel), col, -1).amax(1)
        first_uns = torch.where(unsel & (sc == t_sel), col, big).amin(1)
        assert bool((last_sel < first_uns).all()), "tie at the threshold not broken toward lower positions"


def check_sampled_queries(wl, inp, bufs, qis, mla_layers, full_ordinals):
    """Oracle recomputation for the sampled queries: score rows of the last full
    layer (the scores buffer holds the latest), every listed full layer's
    top-2048, and the listed attention layers."""
    last = len(inp["full_layers"]) - 1
    for qi in qis:
        b = int(inp["q_seq"][qi])
        pos = np.array([int(inp["q_pos"][qi])], np.int32)
        sel = {}
        for j in full_ordinals:
            qh, wh, kh = bench.host_indexer_inputs(wl, inp, j, qi, SEED)
            row = oracle.indexer_score(qh, wh, kh[None], np.zeros(1, np.int32), pos)
            sel[j] = oracle.topk_select(row, pos, 2048)[0]
            if j == last:
                assert_scores_equal(np32(bufs["scores"][qi, :wl.n_ctx]), row[0],
                                    f"{wl.name} query {qi} scores")
            got = np32(bufs["idx"][j, qi])
            assert np.array_equal(got, sel[j]), f"{wl.name} query {qi} full layer {inp['full_layers'][j]} indices"
        for l in mla_layers:
            j = inp["src"][l]
            if j not in sel:
                continue
            ql, qr, kv = inp["layers"][l]
            rows, local = bench.host_rows(kv, b, sel[j])
            o, s = oracle.sparse_mla(np32(ql[qi:qi + 1]), np32(qr[qi:qi + 1]), rows,
                                     np.zeros(1, np.int32), local, bench.SCALE)
            go, gs = bufs["outs"][l]
            eo, el = max_abs(np32(go[qi:qi + 1]), o), max_abs(np32(gs[qi:qi + 1]), s)
            note(eo, el)
            assert eo <= ATOL_OUT and el <= ATOL_LSE, f"{wl.name} query {qi} layer {l}: {eo:.2e} {el:.2e}"
        say(f"{wl.name}: query {qi} (seq {b}, pos {pos[0]}) matches the oracle")


def run_unit(name):
    wl = W.WORKLOADS[name]
    say(f"full size: {name} (n_q={wl.n_q}, N={wl.n_ctx}, layers={wl.n_layers}, {wl.indexer_dtype})")
    d = dev()
    inp = bench.build_inputs(wl, SEED, d)
    _, bufs, _ = bench.make_step(wl, inp, d)
    bench.make_boundary_step(wl, inp, bufs)()          # the boundary call bench.py times
    torch.cuda.synchronize()
    return wl, inp, bufs


@pytest.mark.parametrize("name", ["decode_b64_n131072", "decode_b64_n131072_kv8", "decode_b8_n1048576_fp8",
                                  "decode_b8_n1048576_fp8_kv8"])
def test_group_full_size(name):
    wl, inp, bufs = run_unit(name)
    check_selection_properties(bufs["scores"], bufs["idx"][0], inp["q_pos"], wl.n_ctx)
    qis = sorted({0, wl.n_q // 2, wl.n_q - 1})
    check_sampled_queries(wl, inp, bufs, qis, range(len(inp["layers"])), [0])


@pytest.mark.parametrize("name", ["prefill_q4096_n131072", "prefill_q4096_n131072_fp8"])
def test_prefill_full_size(name):
    wl, inp, bufs = run_unit(name)
    check_selection_properties(bufs["scores"], bufs["idx"][0], inp["q_pos"], wl.n_ctx)
    check_sampled_queries(wl, inp, bufs, [0, 1, 2047, 4094, 4095], [], [0])


def test_stack78_full_size():
    wl, inp, bufs = run_unit("stack78_b8_q8_n262144")
    n_full = len(inp["full_layers"])
    assert n_full == 21 and len(inp["layers"]) == 78
    # the scores buffer holds the last full layer's scores (layer 74)
    check_selection_properties(bufs["scores"], bufs["idx"][n_full - 1], inp["q_pos"], wl.n_ctx)
    for j in range(n_full):                                      # structure of every full layer's set
        ix = bufs["idx"][j]
        assert bool((ix >= 0).all()) and bool((ix[:, 1:] > ix[:, :-1]).all())
    check_sampled_queries(wl, inp, bufs, [0, wl.n_q - 1], [0, 1, 2, 3, 5, 6, 9, 41, 74, 77],
                          list(range(n_full)))


def test_prefill_rotated_fp8_full_size():
    # Hadamard-rotated fp8 indexer: the selection is exact for the scores the
    # kernel produced (all properties above); the sampled queries' scores are
    # within 1e-4 (1 + |s|) of the oracle's rotated-fp8 scores (rotated values
    # are not integers, so fp32 accumulation rounds), and their sets are the
    # oracle's except among positions that bound leaves open
    wl, inp, bufs = run_unit("prefill_q4096_n131072_fp8h")
    check_selection_properties(bufs["scores"], bufs["idx"][0], inp["q_pos"], wl.n_ctx)
    for qi in [0, 2047, 4095]:
        pos = np.array([int(inp["q_pos"][qi])], np.int32)
        qh, wh, kh = bench.host_indexer_inputs(wl, inp, 0, qi, SEED)
        row = oracle.indexer_score(qh, wh, kh[None], np.zeros(1, np.int32), pos)[0]
        got = np32(bufs["scores"][qi, :wl.n_ctx]).astype(np.float64)
        fin = np.isfinite(row)
        assert np.array_equal(np.isfinite(got), fin)
        assert np.all(np.abs(got[fin] - row[fin]) <= 1e-4 * (1 + np.abs(row[fin])))
        # the set differs from the oracle's only where the score bound leaves it open
        n_band = rounding.check_selection_within_bound(np32(bufs["idx"][0, qi]), row, 2048, 1e-4)
        say(f"{wl.name}: query {qi}: selection fixed by the bound except {n_band} positions at the threshold")


def test_decode_full_chunks_with_queries_inside_the_row():
    # 64 x 128K bf16 keys with one query per sequence: the launch takes 4096-key
    # chunks, which the one-query kernel collects whole in LDS before writing.
    # The queries sit inside their rows (at 0, at tile and chunk edges, in the
    # middle, at the end), so whole chunks and parts of chunks lie past them.
    wl = W.WORKLOADS["decode_b64_n131072"]
    d = dev()
    k = W.indexer_keys(wl, SEED, 0, device=d)
    q, w = W.indexer_queries(wl, SEED, 0, device=d)
    g = torch.Generator().manual_seed(5)
    pos = torch.randint(0, wl.n_ctx, (wl.n_q,), generator=g, dtype=torch.int32)
    special = [0, 1, 127, 128, 4095, 4096, 4097, 8191, 65535, wl.n_ctx - 1]
    pos[:len(special)] = torch.tensor(special, dtype=torch.int32)
    q_seq = torch.arange(wl.n_q, dtype=torch.int32, device=d)
    q_pos = pos.to(d)
    say(f"full chunks, queries inside the row: n_q={wl.n_q}, N={wl.n_ctx}, positions {special} and random")
    ld = wl.n_ctx
    scores = torch.full((wl.n_q, ld), 12345.0, device=d)
    gmax = torch.full((wl.n_q, gsa.group_max_ld(ld)), 777.0, device=d)
    gsa.indexer_score(q, w, k, q_seq, q_pos, scores=scores, group_max=gmax)
    torch.cuda.synchronize()
    # every row: -inf exactly past its position, finite up to it (scores >= 0 here)
    past = torch.arange(ld, device=d)[None, :] > q_pos[:, None].long()
    assert bool(torch.isneginf(scores[past]).all()), "a position past its query is not -inf"
    assert bool(torch.isfinite(scores[~past]).all()), "a causal position is not finite"
    for i in [0, 2, 3, 4, 5, 6, 8, 9, 33]:
        p = int(pos[i])
        row = oracle.indexer_score(np32(q[i:i + 1]), np32(w[i:i + 1]), np32(k[i:i + 1]),
                                   np.zeros(1, np.int32), np.array([p], np.int32))
        assert_scores_equal(np32(scores[i]), row[0], f"query {i} at {p}")
        assert_scores_equal(np32(gmax[i]), oracle.group_max(row, n_cols=ld)[0], f"query {i} at {p}: group maxima")
    say("full chunks, queries inside the row: sampled rows match the oracle")
