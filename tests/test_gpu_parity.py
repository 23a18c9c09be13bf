"""HIP path vs the CPU oracle on the same seeded inputs (small and ragged sizes).

Scores and indices must match bit for bit on integer-valued indexer inputs;
attention within 1e-2 max-abs. Every call goes through the C ABI."""
import numpy as np
import pytest
import torch

import long_context_sparse_02_amd as gsa
import oracle
import workloads as W
from gpu_util import ATOL_LSE, ATOL_OUT, assert_scores_equal, dev, max_abs, np32, say, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gsa.lib()


# ------------------------------------------------------------------ quantiser
def test_quantize_e4m3_matches_oracle():
    g = torch.Generator().manual_seed(11)
    ints = torch.randint(-4, 5, (300, 128), generator=g).float()
    normal = torch.randn((300, 128), generator=g) * torch.logspace(-30, 30, 300)[:, None]
    special = torch.zeros((4, 128))
    special[1, 5] = 3.0e38
    special[2] = torch.linspace(-1e-38, 1e-38, 128)
    special[3, ::2] = -0.0
    x = torch.cat([ints, normal, special]).to(torch.bfloat16)
    codes, scales = gsa.quantize_e4m3(x.to(dev()))
    torch.cuda.synchronize()
    oc, osc = oracle.quantize_blocks(np32(x))
    assert np.array_equal(np32(scales).astype(np.float64), osc[:, 0])
    assert np.array_equal(np32(codes), oc)


# ------------------------------------------------------------------ indexer score
def _score_case(wl, seed, ld=None, dtype="bf16", perm=None, with_max=True):
    q, w = W.indexer_queries(wl, seed, 0)
    k = W.indexer_keys(wl, seed, 0)
    q_seq, q_pos = W.query_layout(wl)
    if perm is not None:
        q, w, q_seq, q_pos = q[perm], w[perm], q_seq[perm], q_pos[perm]
    d = dev()
    ld = ld or (wl.n_ctx + 3) // 4 * 4
    scores = torch.full((wl.n_q, ld), 12345.0, device=d)
    gmax = torch.full((wl.n_q, gsa.group_max_ld(ld)), 777.0, device=d) if with_max else None
    if dtype == "fp8":
        qc, qs = gsa.quantize_e4m3(q.to(d))
        kc, ks = gsa.quantize_e4m3(k.to(d))
        gsa.indexer_score(qc, w.to(d), kc, q_seq.to(d), q_pos.to(d), q_scale=qs, k_scale=ks, scores=scores,
                          group_max=gmax)
    else:
        gsa.indexer_score(q.to(d), w.to(d), k.to(d), q_seq.to(d), q_pos.to(d), scores=scores, group_max=gmax)
    torch.cuda.synchronize()
    want = oracle.indexer_score(np32(q), np32(w), np32(k), np32(q_seq), np32(q_pos))
    got = np32(scores)
    for i in range(wl.n_q):
        assert_scores_equal(got[i, : wl.n_ctx], want[i], f"query {i}")
    assert np.all(got[:, wl.n_ctx:] == 12345.0), "columns past n_cap were written"
    if gmax is None:
        return got
    # group maxima: bit-exact (integer inputs), +0.0 for a zero maximum, untouched past n_cap
    ng = -(-wl.n_ctx // 32)
    gm_want = oracle.group_max(want, n_cols=wl.n_ctx)
    gm = np32(gmax)
    for i in range(wl.n_q):
        assert_scores_equal(gm[i, :ng], gm_want[i], f"query {i} group maxima")
    assert not np.any(np.signbit(gm[:, :ng]) & (gm[:, :ng] == 0)), "-0.0 group maximum"
    assert np.all(gm[:, ng:] == 777.0), "group maxima past n_cap were written"
    return got


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_score_tiny_group(dtype):
    _score_case(W.WORKLOADS["group_b1_n4096_q4"], 0, dtype=dtype)


@pytest.mark.parametrize("with_max", [True, False])
@pytest.mark.parametrize("q_per_seq", [1, 2, 3, 4, 8, 11, 16, 19, 37])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_score_ragged_and_query_blocks(q_per_seq, dtype, with_max):
    # 1-2 per sequence: one query per wave pair; 4-15: 4 or 8 queries per work-group;
    # 16+: 16 per work-group, with blocks that straddle two sequences (19, 37)
    # n_cap not a multiple of the 128-key tile; several sequences; ld padded;
    # with and without group maxima (the kernels issue different stores)
    wl = W.Workload("ragged", 3, 1000 + 37 * q_per_seq, q_per_seq, 1, dtype)
    _score_case(wl, q_per_seq, ld=(wl.n_ctx + 12 + 3) // 4 * 4, dtype=dtype, with_max=with_max)


@pytest.mark.parametrize("with_max", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("q_per_seq", [1, 4, 8, 16])
def test_score_many_tiles(q_per_seq, dtype, with_max):
    # long rows (many tiles per work-group, so the ring waits see every case)
    # through the one-query kernel and the multi-query kernel's two-query fast path,
    # with and without group maxima (each wait counts the stores issued since);
    # 8 or 16 queries per sequence stream their keys through the deeper ring
    wl = W.Workload("long_mq", 2, 20_000 + 7, q_per_seq, 1, dtype)
    _score_case(wl, 50 + q_per_seq, dtype=dtype, with_max=with_max)


@pytest.mark.parametrize("n_per", [5, 8, 10, 16, 20])
def test_score_unsorted_sequences_and_positions(n_per):
    # random sequence per query: every query block holds several short runs
    # (8 and 16 per sequence take the streaming multi-query kernel)
    wl = W.Workload("mixed", 4, 700, n_per, 1, "bf16")
    perm = torch.randperm(wl.n_q, generator=torch.Generator().manual_seed(3))
    q, w = W.indexer_queries(wl, 5, 0)
    k = W.indexer_keys(wl, 5, 0)
    q_seq = torch.randint(0, 4, (wl.n_q,), generator=torch.Generator().manual_seed(4), dtype=torch.int32)
    q_pos = torch.tensor(([0, 1, 127, 128, 129, 699, 300, 5, 64, 255, 256, 511, 512, 2, 3, 698, 640,
                           641, 10, 600] * 4)[: wl.n_q], dtype=torch.int32)
    d = dev()
    s = gsa.indexer_score(q.to(d), w.to(d), k.to(d), q_seq.to(d), q_pos.to(d))
    torch.cuda.synchronize()
    want = oracle.indexer_score(np32(q), np32(w), np32(k), np32(q_seq), np32(q_pos))
    for i in range(wl.n_q):
        assert_scores_equal(np32(s)[i, :700], want[i], f"query {i}")
    del perm


def test_score_one_query_rows_past_the_query():
    # one query per sequence at positions that leave partial tiles, whole tiles
    # and whole chunks after it: the one-query kernel writes those positions as
    # -inf (bf16 chunks this short collect the row in LDS and write it at the
    # chunk end; fp8 stores as it goes); full rows and group maxima bit-exact
    n_cap = 9000
    pos = [37, 1023, 1024, 5000, 8191, n_cap - 1]
    wl = W.Workload("past_query", len(pos), n_cap, 1, 1, "bf16")
    q, w = W.indexer_queries(wl, 61, 0)
    k = W.indexer_keys(wl, 61, 0)
    q_seq = torch.arange(len(pos), dtype=torch.int32)
    q_pos = torch.tensor(pos, dtype=torch.int32)
    want = oracle.indexer_score(np32(q), np32(w), np32(k), np32(q_seq), np32(q_pos))
    gm_want = oracle.group_max(want, n_cols=n_cap)
    d = dev()
    ld = (n_cap + 3) // 4 * 4 + 4
    for dtype in ("bf16", "fp8"):
        say(f"one-query rows past the query: {dtype}, positions {pos}")
        scores = torch.full((len(pos), ld), 12345.0, device=d)
        gmax = torch.full((len(pos), gsa.group_max_ld(ld)), 777.0, device=d)
        if dtype == "fp8":
            qc, qs = gsa.quantize_e4m3(q.to(d))
            kc, ks = gsa.quantize_e4m3(k.to(d))
            gsa.indexer_score(qc, w.to(d), kc, q_seq.to(d), q_pos.to(d), q_scale=qs, k_scale=ks,
                              scores=scores, group_max=gmax)
        else:
            gsa.indexer_score(q.to(d), w.to(d), k.to(d), q_seq.to(d), q_pos.to(d), scores=scores,
                              group_max=gmax)
        torch.cuda.synchronize()
        got, gm = np32(scores), np32(gmax)
        ng = -(-n_cap // 32)
        for i, p in enumerate(pos):
            assert_scores_equal(got[i, :n_cap], want[i], f"{dtype} query at {p}")
            assert np.all(np.isneginf(got[i, p + 1:n_cap])), f"{dtype} query at {p}: past positions"
            assert_scores_equal(gm[i, :ng], gm_want[i], f"{dtype} query at {p} group maxima")
        assert np.all(got[:, n_cap:] == 12345.0) and np.all(gm[:, ng:] == 777.0)


def test_score_persistent_fp8_grid_repeated_calls():
    # fp8 decode over 8 rows of 2^20 keys runs on the persistent grid: 256
    # work-groups taking 1024-key chunks from per-query counters that every
    # launch leaves at zero. Queries sit inside their rows (at 0, at chunk
    # edges, mid-row, at the end); the buffers start as NaN, so a chunk that no
    # work-group took shows; 70 calls use every counter slot at least once and
    # each must equal the first bit for bit; sampled rows are bit-exact against
    # the oracle, every row is -inf past its query, and every row's group
    # maxima are those of its scores.
    n_cap = 1 << 20
    pos = [0, 1023, 1024, 333_333, 524_287, 524_288, 1_000_000, n_cap - 1]
    wl = W.Workload("grid_fp8", len(pos), n_cap, 1, 1, "fp8")
    d = dev()
    q, w = W.indexer_queries(wl, 71, 0)
    k = W.indexer_keys(wl, 71, 0, device=d)
    sample = [0, 2, 5, 7]
    k_host = {b: np32(k[b]) for b in sample}
    q_seq = torch.arange(len(pos), dtype=torch.int32, device=d)
    q_pos = torch.tensor(pos, dtype=torch.int32, device=d)
    qc, qs = gsa.quantize_e4m3(q.to(d))
    kc, ks = gsa.quantize_e4m3(k)
    del k
    wd = w.to(d)
    scores = torch.empty((len(pos), n_cap), device=d)
    gmax = torch.empty((len(pos), gsa.group_max_ld(n_cap)), device=d)
    first = None
    for call in range(70):
        scores.fill_(float("nan"))
        gmax.fill_(float("nan"))
        gsa.indexer_score(qc, wd, kc, q_seq, q_pos, q_scale=qs, k_scale=ks, scores=scores, group_max=gmax)
        if first is None:
            first = (scores.clone(), gmax.clone())
            assert not bool(torch.isnan(first[0]).any()) and not bool(torch.isnan(first[1]).any())
        else:
            assert torch.equal(scores, first[0]) and torch.equal(gmax, first[1]), f"call {call}"
    torch.cuda.synchronize()
    got, gm = np32(first[0]), np32(first[1])
    for i, p in enumerate(pos):
        assert np.all(np.isneginf(got[i, p + 1:])), f"query at {p}: past positions"
        assert np.all(np.isfinite(got[i, :p + 1])), f"query at {p}: causal positions"
    assert_scores_equal(gm.ravel(), oracle.group_max(got).ravel(), "group maxima of the scores")
    for b in sample:
        say(f"persistent fp8 grid: oracle row {b} (query at {pos[b]})")
        want = oracle.indexer_score(np32(q[b:b + 1]), np32(w[b:b + 1]), k_host[b][None],
                                    np.zeros(1, np.int32), np.array([pos[b]], np.int32))[0]
        assert_scores_equal(got[b], want, f"row {b}")


@pytest.mark.parametrize("n_q,n_cap", [(1, 1 << 23), (256, 1 << 15), (32, 1 << 18)])
def test_score_persistent_fp8_grid_query_counts(n_q, n_cap):
    # the persistent grid at the ends of its range: one query (all 256
    # work-groups on one counter), 256 queries (one work-group each) and 32;
    # queries at random positions inside their rows, rows padded past n_cap,
    # buffers starting as NaN, two calls in a row equal (the second without
    # group maxima), sampled rows bit-exact against the oracle
    wl = W.Workload("grid_q%d" % n_q, n_q, n_cap, 1, 1, "fp8")
    d = dev()
    g = torch.Generator().manual_seed(73 + n_q)
    pos = torch.randint(0, n_cap, (n_q,), generator=g)
    pos[0] = n_cap - 1
    q, w = W.indexer_queries(wl, 74, 0)
    k = W.indexer_keys(wl, 74, 0, device=d)
    sample = sorted({0, n_q // 2, n_q - 1})
    k_host = {b: np32(k[b]) for b in sample}
    qc, qs = gsa.quantize_e4m3(q.to(d))
    kc, ks = gsa.quantize_e4m3(k)
    del k
    q_seq = torch.arange(n_q, dtype=torch.int32, device=d)
    q_pos = pos.to(torch.int32).to(d)
    # rows padded past n_cap (those columns must stay untouched); the second
    # call writes no group maxima
    ld = n_cap + 8
    outs = []
    for call in range(2):
        scores = torch.full((n_q, ld), float("nan"), device=d)
        gmax = torch.full((n_q, gsa.group_max_ld(ld)), float("nan"), device=d)
        gsa.indexer_score(qc, w.to(d), kc, q_seq, q_pos, q_scale=qs, k_scale=ks, scores=scores,
                          group_max=gmax if call == 0 else None)
        outs.append((scores, gmax))
    torch.cuda.synchronize()
    assert bool(torch.isnan(outs[0][0][:, n_cap:]).all()), "columns past n_cap written"
    assert bool(torch.isnan(outs[1][1]).all()), "group maxima written without a buffer"
    assert torch.equal(outs[0][0][:, :n_cap], outs[1][0][:, :n_cap])
    ng = n_cap // 32
    assert bool(torch.isnan(outs[0][1][:, ng:]).all())
    got, gm = np32(outs[0][0][:, :n_cap]), np32(outs[0][1][:, :ng])
    assert not np.isnan(got).any() and not np.isnan(gm).any()
    assert_scores_equal(gm.ravel(), oracle.group_max(got).ravel(), "group maxima of the scores")
    for b in sample:
        p = int(pos[b])
        assert np.all(np.isneginf(got[b, p + 1:])), f"query at {p}: past positions"
        want = oracle.indexer_score(np32(q[b:b + 1]), np32(w[b:b + 1]), k_host[b][None],
                                    np.zeros(1, np.int32), np.array([p], np.int32))[0]
        assert_scores_equal(got[b], want, f"row {b}")


def test_score_negative_weights_and_float_inputs():
    g = torch.Generator().manual_seed(9)
    q = (torch.randn((6, 32, 128), generator=g)).to(torch.bfloat16)
    k = (torch.randn((2, 900, 128), generator=g)).to(torch.bfloat16)
    w = torch.randn((6, 32), generator=g)
    q_seq = torch.tensor([0, 0, 0, 1, 1, 1], dtype=torch.int32)
    q_pos = torch.tensor([899, 450, 3, 899, 128, 0], dtype=torch.int32)
    d = dev()
    s = np32(gsa.indexer_score(q.to(d), w.to(d), k.to(d), q_seq.to(d), q_pos.to(d)))
    want = oracle.indexer_score(np32(q), np32(w), np32(k), np32(q_seq), np32(q_pos))
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(s[:, :900]), fin)
    # fp32 accumulation over 128 products then 32 heads, against float64
    err = np.abs(s[:, :900][fin] - want[fin])
    assert np.all(err <= 1e-4 * (1 + np.abs(want[fin]))), err.max()


# ------------------------------------------------------------------ top-k
@pytest.mark.parametrize("kind", W.SCORE_KINDS)
def test_topk_matches_oracle(kind):
    n = 40000                                          # 3 chunks, ragged tail
    pos = torch.tensor([39999, 20000, 16383, 16384, 2047, 2048, 2049, 0, 5000], dtype=torch.int32)
    s = W.score_matrix(kind, pos.numel(), n, seed=7)
    d = dev()
    idx = gsa.topk(s.to(d), pos.to(d))
    torch.cuda.synchronize()
    want = oracle.topk_select(np32(s), np32(pos), 2048)
    got = np32(idx)
    for i in range(pos.numel()):
        assert np.array_equal(got[i], want[i]), f"{kind} row {i} (pos {int(pos[i])})"


@pytest.mark.parametrize("kind", W.SCORE_KINDS)
@pytest.mark.parametrize("n", [64, 2048, 2052, 3000, 4092, 4096])
def test_topk_short_rows_match_oracle(kind, n):
    # rows of at most 4096 positions take the one-pass selection bounded by the
    # row's own smallest and largest key: every score kind (ties at the
    # threshold, all equal, signed zeros, a few values), rows shorter than,
    # equal to and just past 2048, rows ending anywhere in the buffer
    cand = [n - 1, 0, 1, 2046, 2047, 2048, 2049, n // 2, 4000]
    pos = torch.tensor(sorted({p for p in cand if 0 <= p < n}), dtype=torch.int32)
    s = W.score_matrix(kind, pos.numel(), n, seed=9 + n)
    d = dev()
    idx = gsa.topk(s.to(d), pos.to(d))
    torch.cuda.synchronize()
    want = oracle.topk_select(np32(s), np32(pos), 2048)
    got = np32(idx)
    for i in range(pos.numel()):
        assert np.array_equal(got[i], want[i]), f"{kind} n={n} row {i} (pos {int(pos[i])})"


def _topk_case(s, pos, label, with_max=True):
    """gsa.topk with the group maxima computed inside, and (with_max) with the
    oracle's maxima passed in; both against the oracle."""
    d = dev()
    want = oracle.topk_select(np32(s), np32(pos), 2048)
    runs = [("inside", None)]
    if with_max:
        ld = s.shape[1]
        gm = np.full((s.shape[0], gsa.group_max_ld(ld)), -np.inf, np.float32)
        gm[:, : -(-ld // 32)] = oracle.group_max(np32(s)).astype(np.float32)
        runs.append(("given", torch.from_numpy(gm).to(d)))
    for how, gm in runs:
        got = np32(gsa.topk(s.to(d), pos.to(d), group_max=gm))
        for i in range(pos.numel()):
            assert np.array_equal(got[i], want[i]), f"{label} ({how} maxima) row {i} (pos {int(pos[i])})"
    say(f"top-k {label}: {pos.numel()} rows match the oracle")


@pytest.mark.parametrize("kind", W.SCORE_KINDS)
def test_topk_bounded_rows_match_oracle(kind):
    # rows long enough for the group-maximum bound (>= 2048 full groups of 32)
    # and rows just short of it, in one call; 13 chunks with a ragged tail
    n = 200_004
    pos = torch.tensor([n - 1, 65535, 65534, 65536 + 31, 65536 + 32, 150_000, 16383, 2047, 0, 99_999],
                       dtype=torch.int32)
    s = W.score_matrix(kind, pos.numel(), n, seed=17)
    _topk_case(s, pos, f"{kind} n={n}")


def test_topk_many_rows_mixed_kinds():
    # >= 512 rows take the register-capped merge build; constant rows take its
    # round-based fallback (every score passes the bound, 5 lists of 2048)
    n, rows = 66_000, 520
    parts = [W.score_matrix(kind, rows, n, seed=31) for kind in ("all_equal", "int_ties", "few_values")]
    s = torch.stack([parts[i % 3][i] for i in range(rows)])
    g = torch.Generator().manual_seed(32)
    pos = torch.randint(60_000, n, (rows,), generator=g, dtype=torch.int32)
    pos[::7] = 65_535
    _topk_case(s, pos, f"{rows} mixed rows", with_max=False)


def test_topk_bound_with_one_huge_value_per_group():
    # every 32-group holds one large value: the bound is the k-th of them and
    # many equal scores sit exactly at it
    n = 131_072
    s = torch.zeros((3, n))
    s[:, ::32] = torch.arange(n // 32, dtype=torch.float32).remainder(50)[None] + 100
    s[1, 5::32] = 149.0
    pos = torch.tensor([n - 1, n - 1, 70_000], dtype=torch.int32)
    _topk_case(s, pos, "one large value per group")


def test_topk_one_million_row():
    n = 1 << 20
    s = W.score_matrix("int_ties", 2, n, seed=8)
    pos = torch.tensor([n - 1, n // 2 + 3], dtype=torch.int32)
    idx = np32(gsa.topk(s.to(dev()), pos.to(dev())))
    want = oracle.topk_select(np32(s), np32(pos), 2048)
    assert np.array_equal(idx, want)


@pytest.mark.parametrize("n", [(1 << 20) - 28, 600_004])
def test_topk_wide_rows_of_every_kind(n):
    # rows up to 2^20 positions (one work-group per row over up to 32K group
    # maxima; 2^20 - 28 leaves an odd number of maxima per row), each score
    # distribution in one call, rows long and short, ties at the bound
    rows = [W.score_matrix(kind, 1, n, seed=40 + i)[0] for i, kind in enumerate(W.SCORE_KINDS)]
    s = torch.stack(rows + rows[:3])
    pos = torch.tensor([n - 1, n - 2, n // 2, 65_535, 200_001, 70_000, 64_000, 3], dtype=torch.int32)
    _topk_case(s, pos, f"wide rows n={n}")


def test_topk_ld_padding_is_ignored():
    s = W.score_matrix("normal", 3, 5000, seed=2)
    s[:, 4990:] = 1e30                                 # beyond every q_pos: must not be selected
    pos = torch.tensor([4989, 3000, 100], dtype=torch.int32)
    idx = np32(gsa.topk(s.to(dev()), pos.to(dev())))
    assert np.array_equal(idx, oracle.topk_select(np32(s), np32(pos), 2048))


def test_topk_split_rows_workspace_of_any_contents():
    # launches of few rows split each row over several work-groups that hand
    # their candidates over through the workspace: the workspace may hold
    # anything beforehand (the arrival counters carry a launch tag) and is
    # reused call after call
    n = 300_000
    s = W.score_matrix("normal", 5, n, seed=51)
    pos = torch.tensor([n - 1, 250_000, 65_536 + 5, 100_000, n - 7], dtype=torch.int32)
    d = dev()
    want = oracle.topk_select(np32(s), np32(pos), 2048)
    sd, pd = s.to(d), pos.to(d)
    g = torch.Generator().manual_seed(52)
    ws = torch.randint(0, 256, (gsa.topk_workspace_bytes(5, n),), dtype=torch.uint8, generator=g).to(d)
    for rep in range(3):
        assert np.array_equal(np32(gsa.topk(sd, pd, workspace=ws)), want), f"random workspace, call {rep}"
    for fill in (255, 0):
        ws.fill_(fill)
        assert np.array_equal(np32(gsa.topk(sd, pd, workspace=ws)), want), f"workspace of {fill}s"
    say("top-k split rows: random, all-ones and zero workspaces, repeated calls")


def test_topk_split_rows_replayed_in_a_graph():
    # a captured launch keeps its tag: every replay must find the counters it
    # left (reset by the last arrival), with other launches on the same
    # workspace between the replays
    n = 200_000
    s = W.score_matrix("int_ties", 4, n, seed=53)
    s2 = W.score_matrix("normal", 4, n, seed=54)
    pos = torch.tensor([n - 1, 150_000, 70_000, n - 3], dtype=torch.int32)
    d = dev()
    sd, s2d, pd = s.to(d), s2.to(d), pos.to(d)
    want = oracle.topk_select(np32(s), np32(pos), 2048)
    want2 = oracle.topk_select(np32(s2), np32(pos), 2048)
    idx = torch.empty((4, 2048), dtype=torch.int32, device=d)
    ws = torch.empty(gsa.topk_workspace_bytes(4, n), dtype=torch.uint8, device=d)
    gsa.topk(sd, pd, idx=idx, workspace=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gsa.topk(sd, pd, idx=idx, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        idx.fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(np32(idx), want), f"replay {rep}"
        assert np.array_equal(np32(gsa.topk(s2d, pd, workspace=ws)), want2), f"eager call after replay {rep}"
    say("top-k split rows: 3 graph replays, each followed by an eager call on the same workspace")


def test_topk_split_rows_with_more_candidates_than_one_selection_takes():
    # every group's maximum is 1.0, so every group reaches the bound: one 1.0
    # per group fills each wave's part exactly and the shares together hold 16x
    # what the final selection takes; two per group overflow the parts; both go
    # to the fallback over the whole list
    n = 1 << 20
    s = torch.zeros((3, n))
    gi = torch.arange(n // 32)
    s[0, gi * 32 + gi % 32] = 1.0
    s[1, gi * 32] = 1.0
    s[1, gi * 32 + 31] = 1.0
    s[2] = W.score_matrix("normal", 1, n, seed=55)[0]
    pos = torch.tensor([n - 1, n - 1, 700_000], dtype=torch.int32)
    _topk_case(s, pos, "every group at the bound")


@pytest.mark.parametrize("n,rows", [(1 << 20, 3), (131_072, 40)])
def test_topk_split_rows_with_candidates_clustered_in_one_share(n, rows):
    # scores rising with the position (recent positions score higher, as in
    # attention): every candidate lies in the row's last share, far more than
    # its window of 4096 / shares; a few rows are i.i.d. for contrast
    g = torch.Generator().manual_seed(71)
    pos_f = torch.arange(n, dtype=torch.float32)
    s = pos_f[None, :] / 64.0 + torch.randint(0, 8, (rows, n), generator=g).float()
    s[1] = W.score_matrix("normal", 1, n, seed=72)[0]
    pos = torch.full((rows,), n - 1, dtype=torch.int32)
    pos[2] = n - 5000
    _topk_case(s, pos, f"clustered candidates n={n} rows={rows}")


def test_topk_four_shares_with_short_rows():
    # 40 rows: four shares per row; short rows (no bound, or fewer than 2048
    # candidates in all) beside full ones
    n, rows = 131_072, 40
    s = torch.stack([W.score_matrix(("normal", "int_ties", "few_values")[i % 3], 1, n, seed=80 + i)[0]
                     for i in range(rows)])
    pos = torch.full((rows,), n - 1, dtype=torch.int32)
    pos[0:8] = torch.tensor([0, 1, 100, 2046, 2047, 2048, 3000, 4095], dtype=torch.int32)
    pos[8:12] = torch.tensor([65_535, 65_536, 70_000, 100_000], dtype=torch.int32)
    _topk_case(s, pos, f"{rows} rows with short ones")


def test_topk_row_kernel_without_split():
    # 128..511 rows: one work-group per row, the default build
    n, rows = 70_000, 130
    parts = [W.score_matrix(kind, rows, n, seed=61) for kind in ("normal", "int_ties", "few_values")]
    s = torch.stack([parts[i % 3][i] for i in range(rows)])
    g = torch.Generator().manual_seed(62)
    pos = torch.randint(66_000, n, (rows,), generator=g, dtype=torch.int32)
    pos[::9] = n - 1
    _topk_case(s, pos, f"{rows} rows, one work-group each", with_max=False)


# ------------------------------------------------------------------ sparse MLA
def _mla_case(n_q, batch, n_ctx, seed, idx_fn=None):
    wl = W.Workload("mla", batch, n_ctx, n_q // batch, 1, "bf16")
    q_lat, q_rope = W.mla_queries(wl, seed, 0)
    kv = W.mla_cache(wl, seed, 0)
    q_seq, q_pos = W.query_layout(wl)
    g = torch.Generator().manual_seed(seed)
    if idx_fn is None:
        s = torch.randn((wl.n_q, n_ctx), generator=g)
        idx = torch.from_numpy(oracle.topk_select(s.numpy(), np32(q_pos), 2048))
    else:
        idx = idx_fn(wl, g)
    d = dev()
    out, lse = gsa.sparse_mla_attn(q_lat.to(d), q_rope.to(d), kv.to(d), q_seq.to(d), idx.to(d))
    torch.cuda.synchronize()
    o_want, l_want = oracle.sparse_mla(np32(q_lat), np32(q_rope), np32(kv), np32(q_seq), np32(idx), 1 / 16)
    eo, el = max_abs(np32(out), o_want), max_abs(np32(lse), l_want)
    say(f"mla n_q={n_q}: max|out-oracle|={eo:.2e} max|lse-oracle|={el:.2e}")
    note(eo, el)
    assert eo <= ATOL_OUT and el <= ATOL_LSE
    return out, lse


@pytest.mark.parametrize("n_q,batch", [(4, 1), (8, 2), (64, 4), (256, 2)])   # splits 32, 32, 4, 1
def test_mla_matches_oracle(n_q, batch):
    _mla_case(n_q, batch, 5000, seed=n_q)


def test_mla_scattered_invalid_indices_and_empty_rows():
    def idx_fn(wl, g):
        idx = torch.randint(0, wl.n_ctx, (wl.n_q, 2048), generator=g, dtype=torch.int32)
        drop = torch.rand((wl.n_q, 2048), generator=g) < 0.3
        idx[drop] = -1
        idx[1] = -1                                    # a query with nothing to attend
        idx[2, :] = -1
        idx[2, 777] = 42                               # a single valid row
        return idx
    out, lse = _mla_case(4, 1, 3000, seed=21, idx_fn=idx_fn)
    assert torch.all(out[1] == 0) and torch.all(torch.isneginf(lse[1]))


def test_mla_out_of_range_indices_are_skipped_like_minus_one():
    # entries past the cache (n_ctx, 2^30, 2^31 - 1) or below -1 are skipped by the
    # gather exactly as -1 is: the same bits as the call with those entries set to -1
    wl = W.Workload("mla_oob", 1, 3000, 4, 1, "bf16")
    q_lat, q_rope = W.mla_queries(wl, 23, 0)
    kv = W.mla_cache(wl, 23, 0)
    q_seq, _ = W.query_layout(wl)
    g = torch.Generator().manual_seed(23)
    idx = torch.randint(0, 3000, (4, 2048), generator=g, dtype=torch.int32)
    bad = torch.rand((4, 2048), generator=g) < 0.25
    junk = torch.tensor([3000, 3001, 1 << 30, (1 << 31) - 1, -2, -(1 << 31)], dtype=torch.int32)
    idx_bad = idx.clone()
    idx_bad[bad] = junk[torch.randint(0, len(junk), (int(bad.sum()),), generator=g)]
    idx_bad[3] = 5000                                     # a row with nothing in range
    idx_clean = torch.where((idx_bad >= 0) & (idx_bad < 3000), idx_bad, torch.full_like(idx_bad, -1))
    d = dev()
    a = gsa.sparse_mla_attn(q_lat.to(d), q_rope.to(d), kv.to(d), q_seq.to(d), idx_bad.to(d))
    b = gsa.sparse_mla_attn(q_lat.to(d), q_rope.to(d), kv.to(d), q_seq.to(d), idx_clean.to(d))
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.all(a[0][3] == 0) and torch.all(torch.isneginf(a[1][3]))
    o_want, l_want = oracle.sparse_mla(np32(q_lat), np32(q_rope), np32(kv), np32(q_seq), np32(idx_clean), 1 / 16)
    eo, el = max_abs(np32(a[0]), o_want), max_abs(np32(a[1]), l_want)
    note(eo, el)
    assert eo <= ATOL_OUT and el <= ATOL_LSE


def test_mla_short_prefix_equals_dense():
    # prefix <= 2048: top-k keeps every position, so sparse attention is dense attention
    def idx_fn(wl, g):
        pos = torch.tensor([0, 1, 700, 2047])
        idx = torch.full((4, 2048), -1, dtype=torch.int32)
        for i, p in enumerate(pos):
            idx[i, : p + 1] = torch.arange(p + 1)
        return idx
    _mla_case(4, 1, 2048, seed=5, idx_fn=idx_fn)


# ------------------------------------------------------------------ IndexShare group
def _group_case(wl, seed, dtype="bf16"):
    g = W.group_inputs(wl, seed, n_layers=4)
    d = dev()
    layers = [tuple(t.to(d) for t in L) for L in g.layers]
    idx = torch.full((wl.n_q, 2048), -7, dtype=torch.int32, device=d)
    kw = {}
    q_idx, k_idx = g.q_idx.to(d), g.k_idx.to(d)
    if dtype == "fp8":
        q_idx, kw["q_scale"] = gsa.quantize_e4m3(q_idx)
        k_idx, kw["k_scale"] = gsa.quantize_e4m3(k_idx)
    outs = gsa.indexshare_group(layers, g.q_seq.to(d), idx, q_pos=g.q_pos.to(d), q_idx=q_idx,
                                w=g.w.to(d), k_idx=k_idx, **kw)
    torch.cuda.synchronize()
    sc, oidx, oouts = oracle.indexshare_group(
        np32(g.q_idx), np32(g.w), np32(g.k_idx), np32(g.q_seq), np32(g.q_pos),
        [tuple(np32(t) for t in L) for L in g.layers])
    assert np.array_equal(np32(idx), oidx)
    for l, ((o, s), (wo, ws)) in enumerate(zip(outs, oouts)):
        eo, el = max_abs(np32(o), wo), max_abs(np32(s), ws)
        say(f"group layer {l}: max|out|err={eo:.2e} lse err={el:.2e}")
        note(eo, el)
        assert eo <= ATOL_OUT and el <= ATOL_LSE
    return idx, outs


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_group_tiny(dtype):
    _group_case(W.WORKLOADS["group_b1_n4096_q4"], 0, dtype)


def test_group_s_only_call_reuses_buffer_and_is_deterministic():
    # an S-only call over the F layer's buffer reproduces the group's S layers (to the
    # attention tolerance: a call over fewer layers may split rows differently), and
    # repeating the same call gives the same bits
    wl = W.WORKLOADS["group_b1_n4096_q4"]
    idx, outs = _group_case(wl, 1)
    g = W.group_inputs(wl, 1, n_layers=4)
    d = dev()
    layers = [tuple(t.to(d) for t in L) for L in g.layers[1:]]
    outs2 = gsa.indexshare_group(layers, g.q_seq.to(d), idx, compute_index=False)
    outs3 = gsa.indexshare_group(layers, g.q_seq.to(d), idx, compute_index=False)
    torch.cuda.synchronize()
    for (o1, s1), (o2, s2), (o3, s3) in zip(outs[1:], outs2, outs3):
        assert max_abs(np32(o1), np32(o2)) <= ATOL_OUT and max_abs(np32(s1), np32(s2)) <= ATOL_LSE
        assert torch.equal(o2, o3) and torch.equal(s2, s3)


def test_group_index_tag_written_then_checked():
    # the F call records what its buffer holds; an S-only call naming the same
    # epoch and full layer runs (same bits as the unchecked call), any other
    # epoch or layer is refused before anything is enqueued
    wl = W.WORKLOADS["group_b1_n4096_q4"]
    g = W.group_inputs(wl, 2, n_layers=4)
    d = dev()
    layers = [tuple(t.to(d) for t in L) for L in g.layers]
    idx = torch.full((wl.n_q, 2048), -7, dtype=torch.int32, device=d)
    tag = gsa.IndexTag()
    gsa.indexshare_group(layers[:1], g.q_seq.to(d), idx, q_pos=g.q_pos.to(d), q_idx=g.q_idx.to(d),
                         w=g.w.to(d), k_idx=g.k_idx.to(d), index_epoch=1234, index_layer=6, index_tag=tag)
    assert (tag.index_buf_dev, tag.epoch, tag.full_layer, tag.n_q, tag.k, tag.n_cap) == \
        (idx.data_ptr(), 1234, 6, wl.n_q, 2048, wl.n_ctx)
    checked = gsa.indexshare_group(layers[1:], g.q_seq.to(d), idx, compute_index=False,
                                   index_epoch=1234, index_layer=6, index_tag=tag)
    plain = gsa.indexshare_group(layers[1:], g.q_seq.to(d), idx, compute_index=False)
    torch.cuda.synchronize()
    for (o1, s1), (o2, s2) in zip(checked, plain):
        assert torch.equal(o1, o2) and torch.equal(s1, s2)
    before = [o.clone() for o, _ in checked]
    for kw in (dict(index_epoch=1235, index_layer=6), dict(index_epoch=1234, index_layer=10)):
        with pytest.raises(gsa.GsaError, match="GSA_ERR_STALE_INDEX"):
            gsa.indexshare_group(layers[1:], g.q_seq.to(d), idx, compute_index=False, index_tag=tag,
                                 outs=checked, **kw)
    torch.cuda.synchronize()
    assert all(torch.equal(o, b) for (o, _), b in zip(checked, before))   # nothing ran


@pytest.mark.parametrize("n_layers,n_q,batch", [(3, 2, 1), (4, 8, 8), (9, 5, 2)])
def test_sparse_mla_layers_launch_matches_oracle(n_layers, n_q, batch):
    # one launch over several layers sharing the index buffer (9 layers: two launches);
    # the split per query depends on layers x queries, so every case splits differently
    wl = W.Workload("mla_layers", batch, 3000, n_q // batch if n_q % batch == 0 else 1, n_layers, "bf16")
    q_seq = torch.arange(n_q, dtype=torch.int32) % batch
    q_pos = torch.full((n_q,), 2999, dtype=torch.int32)
    g = torch.Generator().manual_seed(40 + n_layers)
    idx = torch.stack([torch.sort(torch.randperm(3000, generator=g)[:2048])[0] for _ in range(n_q)]).to(torch.int32)
    idx[0, 2000:] = -1                                      # a ragged row
    d = dev()
    layers_cpu = []
    for l in range(n_layers):
        ql, qr = W.mla_queries(W.Workload("x", batch, 3000, 1, 1, "bf16"), 7, l)
        ql, qr = ql[:1].repeat(n_q, 1, 1), qr[:1].repeat(n_q, 1, 1)
        ql = ql + 0.25 * torch.randn(ql.shape, generator=g).to(torch.bfloat16)
        layers_cpu.append((ql, qr, W.mla_cache(W.Workload("x", batch, 3000, 1, 1, "bf16"), 7, l)))
    layers = [tuple(t.to(d) for t in L) for L in layers_cpu]
    outs = gsa.sparse_mla_attn_layers(layers, q_seq.to(d), idx.to(d), 1 / 16)
    torch.cuda.synchronize()
    for l, ((o, s), (ql, qr, kv)) in enumerate(zip(outs, layers_cpu)):
        wo, ws = oracle.sparse_mla(np32(ql), np32(qr), np32(kv), np32(q_seq), np32(idx), 1 / 16)
        eo, el = max_abs(np32(o), wo), max_abs(np32(s), ws)
        say(f"layers launch {n_layers}x{n_q}: layer {l} out err {eo:.2e} lse err {el:.2e}")
        note(eo, el)
        assert eo <= ATOL_OUT and el <= ATOL_LSE
    del q_pos


def test_mla_row_pair_layout_rescales_and_edge_rows():
    # 4 layers x 32 queries: 128 (query, layer) units, each query split into 2
    # slices of 1024 rows, which takes the row-pair layout (each wave of a pair
    # scores 16 of a block's 32 rows). The RoPE half of the cache rows grows with
    # the position (up to 11x), so rows taken in ascending order raise the running
    # max block after block: on the CPU, 1.6 later rescales per head on average,
    # some moving in both row halves at once; descending order puts the largest
    # rows first. Edge rows: every index -1; a single valid index; one row half of
    # every block empty (the first, or the second).
    n_layers, n_q, batch, n_ctx = 4, 32, 2, 5000
    wl = W.Workload("mla_rp", batch, n_ctx, n_q // batch, n_layers, "bf16")
    q_seq = torch.arange(n_q, dtype=torch.int32) % batch
    g = torch.Generator().manual_seed(91)
    idx = torch.stack([torch.sort(torch.randperm(n_ctx, generator=g)[:2048])[0] for _ in range(n_q)]).to(torch.int32)
    idx[1] = torch.flip(idx[1], [0])
    idx[2] = -1
    idx[3] = -1
    idx[3, 1500] = 4321
    second_half = (torch.arange(2048) // 16) % 2 == 1
    idx[4, second_half] = -1
    idx[5, ~second_half] = -1
    grow = 1.0 + torch.arange(n_ctx, dtype=torch.float32) / 500.0
    layers_cpu = []
    for l in range(n_layers):
        ql, qr = W.mla_queries(wl, 9, l)
        kv = W.mla_cache(wl, 9, l).float()
        kv[..., 512:] *= grow[None, :, None]
        layers_cpu.append((ql, qr, kv.to(torch.bfloat16)))
    d = dev()
    layers = [tuple(t.to(d) for t in L) for L in layers_cpu]
    outs = gsa.sparse_mla_attn_layers(layers, q_seq.to(d), idx.to(d), 1 / 16)
    torch.cuda.synchronize()
    for l, ((o, s), (ql, qr, kv)) in enumerate(zip(outs, layers_cpu)):
        wo, ws = oracle.sparse_mla(np32(ql), np32(qr), np32(kv), np32(q_seq), np32(idx), 1 / 16)
        eo, el = max_abs(np32(o), wo), max_abs(np32(s), ws)
        # These scores are large, so the softmax is peaked and few rows carry each
        # output: the 1e-2 bar of the unit-scale cases no longer bounds the error.
        # Bound from the arithmetic instead: out = sum_j p_j v_j / l with l the exact
        # fp32 sum and P rounded to bf16 (unit roundoff 2^-8), so the error is at
        # most 2^-8 max|v|; the 2 slices' partials are fp16 with a power-of-two
        # scale per (head, latent half), adding at most 2^-11 max|v|.
        tol = 1.05 * (2.0 ** -8 + 2.0 ** -11) * float(kv[..., :512].float().abs().max())
        say(f"row-pair layout: layer {l} out err {eo:.2e} (bound {tol:.2e}) lse err {el:.2e}")
        note(eo, el, bar=tol)
        assert eo <= tol and el <= ATOL_LSE
        assert torch.all(o[2] == 0) and torch.all(torch.isneginf(s[2]))
