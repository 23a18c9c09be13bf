"""Pins for the oracle's indexer score and top-K selection (CPU only)."""
import itertools

import numpy as np
import pytest

import oracle
import workloads as W


def _brute_score(q, w, k, q_seq, q_pos, n):
    """Pure-Python integer loops over (query, position, head, dim)."""
    n_q, n_h, n_d = len(q), len(q[0]), len(q[0][0])
    out = [[None] * n for _ in range(n_q)]
    for i in range(n_q):
        for s in range(n):
            if s > q_pos[i]:
                out[i][s] = float("-inf")
                continue
            tot = 0
            for h in range(n_h):
                dot = 0
                for d in range(n_d):
                    dot += int(q[i][h][d]) * int(k[q_seq[i]][s][d])
                tot += int(w[i][h]) * max(0, dot)
            out[i][s] = float(tot)
    return out


def test_score_matches_integer_brute_force():
    rng = np.random.default_rng(1)
    n_q, n_h, n_d, b, n = 5, 4, 8, 2, 11
    q = rng.integers(-4, 5, (n_q, n_h, n_d))
    k = rng.integers(-4, 5, (b, n, n_d))
    w = rng.integers(1, 5, (n_q, n_h))
    q_seq = np.array([0, 0, 1, 1, 1])
    q_pos = np.array([10, 3, 0, 7, 10])
    got = oracle.indexer_score(q, w, k, q_seq, q_pos)
    want = np.array(_brute_score(q.tolist(), w.tolist(), k.tolist(), q_seq.tolist(), q_pos.tolist(), n))
    assert np.array_equal(got, want)


def test_score_negative_weights_and_relu():
    # negative w and negative dots: ReLU applies to the dot, w multiplies after
    q = np.array([[[1.0, 0.0], [0.0, 1.0]]])
    k = np.array([[[2.0, -3.0], [-1.0, 5.0]]])
    w = np.array([[-2.0, 3.0]])
    got = oracle.indexer_score(q, w, k, [0], [1])
    # s=0: head0 dot=2 -> -4 ; head1 dot=-3 -> 0  => -4
    # s=1: head0 dot=-1 -> 0 ; head1 dot=5 -> 15  => 15
    assert got.tolist() == [[-4.0, 15.0]]


def test_score_closed_forms():
    n, h, d = 64, W.INDEX_HEADS, W.INDEX_DIM
    w = np.arange(1, h + 1, dtype=np.float64)[None, :]
    ones = oracle.indexer_score(np.ones((1, h, d)), w, np.ones((1, n, d)), [0], [n - 1])
    assert np.all(ones == d * w.sum())
    zeros = oracle.indexer_score(np.zeros((1, h, d)), w, np.ones((1, n, d)), [0], [n - 1])
    assert np.all(zeros == 0.0)
    # one-hot: q[h] = e_{h}, k[s] = 3 e_{s mod h}: only head s mod h fires, with dot 3
    q = np.zeros((1, h, d))
    q[0, np.arange(h), np.arange(h)] = 1.0
    k = np.zeros((1, n, d))
    k[0, np.arange(n), np.arange(n) % h] = 3.0
    got = oracle.indexer_score(q, w, k, [0], [n - 1])[0]
    assert np.array_equal(got, 3.0 * w[0, np.arange(n) % h])


def test_score_causal_mask():
    q = np.ones((3, 2, 4))
    k = np.ones((1, 6, 4))
    got = oracle.indexer_score(q, np.ones((3, 2)), k, [0, 0, 0], [0, 2, 5])
    for i, p in enumerate([0, 2, 5]):
        assert np.all(np.isfinite(got[i, : p + 1]))
        assert np.all(got[i, p + 1:] == -np.inf)


def _brute_topk(row, p, k):
    cand = sorted(range(p + 1), key=lambda s: (-row[s], s))[:k]
    cand = sorted(cand)
    return cand + [-1] * (k - len(cand))


@pytest.mark.parametrize("k", [1, 4, 16])
def test_topk_matches_full_sort_tiny(k):
    rng = np.random.default_rng(k)
    for trial in range(20):
        n = int(rng.integers(1, 65))
        row = rng.integers(-3, 4, n).astype(np.float32)      # dense ties
        p = int(rng.integers(0, n))
        got = oracle.topk_select(row[None], [p], k)[0].tolist()
        assert got == _brute_topk(row.tolist(), p, k)


@pytest.mark.parametrize("n", [2047, 2048, 2049, 4096])
def test_topk_matches_full_sort_real_k(n):
    rng = np.random.default_rng(n)
    row = np.round(rng.normal(0, 30, n)).astype(np.float32)
    got = oracle.topk_select(row[None], [n - 1], 2048)[0].tolist()
    assert got == _brute_topk(row.tolist(), n - 1, 2048)


def _check_topk_invariants(row, p, idx, k):
    sel = idx[idx >= 0]
    assert sel.size == min(k, p + 1)
    assert np.all(idx[: sel.size] >= 0) and np.all(idx[sel.size:] == -1)
    assert np.all(np.diff(sel) > 0) and sel.max() <= p
    if sel.size < p + 1:
        valid = row[: p + 1]
        mask = np.zeros(p + 1, bool)
        mask[sel] = True
        thr = valid[mask].min()
        assert thr >= valid[~mask].max()
        # at the threshold, every unselected position lies above every selected one
        sel_t = np.nonzero(mask & (valid == thr))[0]
        uns_t = np.nonzero(~mask & (valid == thr))[0]
        if uns_t.size and sel_t.size:
            assert uns_t.min() > sel_t.max()


@pytest.mark.parametrize("kind", W.SCORE_KINDS)
def test_topk_invariants(kind):
    s = W.score_matrix(kind, 4, 6000, seed=3).numpy()
    pos = np.array([5999, 4000, 2048, 100])
    idx = oracle.topk_select(s, pos, 2048)
    for i in range(4):
        _check_topk_invariants(s[i], pos[i], idx[i], 2048)


def test_topk_all_equal_is_prefix():
    s = np.full((2, 10000), 7.0, np.float32)
    idx = oracle.topk_select(s, [9999, 5000], 2048)
    assert np.array_equal(idx[0], np.arange(2048)) and np.array_equal(idx[1], np.arange(2048))


def test_topk_short_prefix_selects_everything():
    s = np.random.default_rng(0).normal(size=(3, 3000)).astype(np.float32)
    idx = oracle.topk_select(s, [0, 2, 2047], 2048)
    assert idx[0, 0] == 0 and np.all(idx[0, 1:] == -1)
    assert idx[1, :3].tolist() == [0, 1, 2] and np.all(idx[1, 3:] == -1)
    assert np.array_equal(idx[2], np.arange(2048))


def test_signed_zero_ties_with_positive_zero():
    row = np.array([-0.0, 0.0, -0.0, 0.0, -1.0], np.float32)
    assert oracle.topk_select(row[None], [4], 2)[0].tolist() == [0, 1]


def test_skip_topk_offset_is_moot():
    """index_skip_topk_offset = 3 (GLM-5.2 架构深度拆解 §2.1): the first 3 tokens take
    the full path. With fewer than K positions a full layer keeps every position,
    exactly what a shared layer reuses, so no special case is needed."""
    wl = W.Workload("t", 1, 8, 3, 1, "bf16")
    q, w = W.indexer_queries(wl, 0, 0)
    k = W.indexer_keys(wl, 0, 0)
    for pos in range(3):
        sc = oracle.indexer_score(q.float().numpy()[:1], w.numpy()[:1], k.float().numpy(), [0], [pos])
        idx = oracle.topk_select(sc, [pos], 2048)[0]
        assert idx[: pos + 1].tolist() == list(range(pos + 1)) and np.all(idx[pos + 1:] == -1)


def test_score_on_tiny_group_is_integer_and_fp32_exact():
    wl = W.WORKLOADS["group_b1_n4096_q4"]
    g = W.group_inputs(wl, seed=0, n_layers=0)
    sc = oracle.indexer_score(g.q_idx.float().numpy(), g.w.numpy(), g.k_idx.float().numpy(),
                              g.q_seq.numpy(), g.q_pos.numpy())
    fin = sc[np.isfinite(sc)]
    assert np.all(fin == np.round(fin)) and np.abs(fin).max() < 2 ** 24
    assert np.array_equal(fin.astype(np.float32).astype(np.float64), fin)


# ---------------------------------------------------------------- group maxima
def test_group_max_worked_example():
    row = np.array([[1.0, -0.0, 3.0, 2.0, -np.inf, -np.inf, -5.0, 7.0, -0.0, -1.0]])
    got = oracle.group_max(row, group=4)
    assert got.tolist() == [[3.0, 7.0, 0.0]]                    # last run: 2 columns
    assert not np.signbit(got[0, 2])                            # -0.0 reported as +0.0
    assert oracle.group_max(row, n_cols=5, group=4).tolist() == [[3.0, -np.inf]]


@pytest.mark.parametrize("n", [1, 31, 32, 33, 1000])
def test_group_max_is_attained_and_bounds_its_group(n):
    rng = np.random.default_rng(n)
    s = rng.integers(-50, 50, size=(3, n)).astype(np.float64)
    gm = oracle.group_max(s)
    assert gm.shape == (3, -(-n // 32))
    for i in range(3):
        for g in range(gm.shape[1]):
            blk = s[i, 32 * g: 32 * g + 32]
            assert gm[i, g] in blk and np.all(blk <= gm[i, g])
        assert gm[i].max() == s[i].max()


def test_kth_group_max_bounds_the_kth_score():
    # the fact the GPU top-k relies on: the k-th largest group maximum is <= the
    # k-th largest score, so no selected score is below it
    rng = np.random.default_rng(3)
    for _ in range(20):
        n, k = int(rng.integers(64, 3000)), int(rng.integers(1, 60))
        s = rng.integers(0, 40, size=(1, n)).astype(np.float64)
        gm = oracle.group_max(s, group=int(rng.integers(1, 40)))
        if gm.shape[1] < k:
            continue
        assert np.sort(gm[0])[::-1][k - 1] <= np.sort(s[0])[::-1][k - 1]


def test_selection_bound_check_accepts_perturbed_scores_and_rejects_wrong_sets():
    # the check the rotated-fp8 GPU tests use: a selection made from scores
    # within tau (1 + |s|) of the oracle's passes it; swapping a clearly
    # selected position for a clearly unselected one fails it
    import rounding
    rng = np.random.default_rng(4)
    n, k, tau = 20000, 2048, 1e-4
    want = rng.standard_normal(n) * 3.0
    want[-100:] = -np.inf                                   # masked tail
    want[500:540] = np.sort(want[~np.isinf(want)])[-k]      # ties at the threshold
    pos = np.array([n - 101], np.int32)
    noisy = want + tau * (1.0 + np.abs(np.where(np.isinf(want), 0.0, want))) * rng.uniform(-1, 1, n)
    sel = oracle.topk_select(noisy[None], pos, k)[0]
    n_band = rounding.check_selection_within_bound(sel, want, k, tau)
    assert n_band >= 40
    order = np.argsort(-np.where(np.isinf(want), -1e30, want))
    bad = sel.copy()
    bad[bad == order[0]] = order[-200]                      # best position out, a poor one in
    with pytest.raises(AssertionError):
        rounding.check_selection_within_bound(bad, want, k, tau)
    # rows with at most k causal positions select them all
    short = want.copy()
    short[100:] = -np.inf
    assert rounding.check_selection_within_bound(np.arange(100), short, k, tau) == 0
