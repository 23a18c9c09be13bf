"""Absorbed sparse MLA over the selected positions of one layer. Oracle only.

Pages: "GLM-5.2 总览" tbl-glm52-config (64 heads; QK head dim 256 = 192 NoPE +
64 RoPE; KV latent 512; each token's cache row is the 512-dim latent plus the
64-dim RoPE key, 1152 B in BF16) and its sub-document index (decode runs in
latent space via the absorb trick); "GLM-5.2 架构深度拆解" CH2 §2.2 (attention
runs only over the 2048 selected tokens, the same cost in F and S layers);
"GLM-5→5.1→5.2…" §10 (each layer gathers the selected entries from its own
K/V cache).

For query i, head h, selected positions s_j = idx[i, j] >= 0 of sequence b:

    z_j   = scale * (<q_lat[i,h], c[b,s_j]> + <q_rope[i,h], kr[b,s_j]>)
    p     = softmax_j(z)
    out   = sum_j p_j * c[b, s_j]          (512-dim; V is the latent itself)
    lse   = log sum_j exp(z_j)

Readings (pages silent): scale = 1/sqrt(256); the W_UV up-projection after the
latent output is outside the path; a query with no valid index gives out = 0
and lse = -inf.
"""
from __future__ import annotations

import numpy as np


def sparse_mla(q_lat, q_rope, kv, q_seq, idx, scale: float, d_latent: int = 512):
    """q_lat [n_q, H, Dc], q_rope [n_q, H, Dr], kv [B, N, Dc + Dr], idx [n_q, K].

    Returns (out float64 [n_q, H, Dc], lse float64 [n_q, H])."""
    q_lat = np.asarray(q_lat, dtype=np.float64)
    q_rope = np.asarray(q_rope, dtype=np.float64)
    q_seq = np.asarray(q_seq, dtype=np.int64)
    idx = np.asarray(idx, dtype=np.int64)
    n_q, n_h, _ = q_lat.shape
    out = np.zeros((n_q, n_h, d_latent), dtype=np.float64)
    lse = np.full((n_q, n_h), -np.inf, dtype=np.float64)
    for i in range(n_q):
        sel = idx[i][idx[i] >= 0]
        if sel.size == 0:
            continue
        rows = np.asarray(kv[int(q_seq[i])][sel], dtype=np.float64)   # [k, Dc + Dr]
        c = rows[:, :d_latent]
        kr = rows[:, d_latent:]
        z = scale * (q_lat[i] @ c.T + q_rope[i] @ kr.T)               # [H, k]
        m = z.max(axis=1, keepdims=True)
        e = np.exp(z - m)
        denom = e.sum(axis=1, keepdims=True)
        out[i] = (e @ c) / denom
        lse[i] = (m + np.log(denom))[:, 0]
    return out, lse


def paged_cache_view(pool, block_table, page_size: int):
    """The per-sequence cache [B, max_pages * page_size, D] that a paged pool
    stands for: position s of sequence b lives in pool row
    block_table[b, s // page_size] * page_size + s % page_size.

    pool [n_pages * page_size, D] (or [n_pages, page_size, D]); block_table
    int [B, max_pages]. Pages whose table entry is not a pool page (e.g. -1 for
    a page not yet allocated) read as NaN, so that attending to them shows.

    Pages: "GLM-5→5.1→5.2…" §10 (each layer gathers the selected positions'
    rows from its own cache); "GLM-5.2 架构深度拆解" CH4 §4.4 (PagedAttention as
    the paging used with the 512-d latent cache). The layout is a reading (the
    pages give none): fixed-size pages named by a per-sequence table."""
    pool = np.asarray(pool, dtype=np.float64)
    pool = pool.reshape(-1, pool.shape[-1])
    bt = np.asarray(block_table, dtype=np.int64)
    n_pages = pool.shape[0] // page_size
    B, max_pages = bt.shape
    view = np.full((B, max_pages * page_size, pool.shape[1]), np.nan)
    for b in range(B):
        for j in range(max_pages):
            p = int(bt[b, j])
            if 0 <= p < n_pages:
                view[b, j * page_size:(j + 1) * page_size] = pool[p * page_size:(p + 1) * page_size]
    return view
