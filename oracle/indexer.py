"""Lightning-indexer score of a full (F) layer. Oracle only.

Pages: "GLM-5.2 架构深度拆解" CH2 §2.2 — in an F layer every query scores all
historical tokens with a 32-head, 128-dim indexer before the top-2048 pick;
"GLM-5.2 总览" tbl-glm52-config (32 heads x 128 dims) and its sub-document
index (the indexer has a ReLU); "GLM-5.2架构与基准" §2 (a lightning indexer
picks the top-k tokens per query).

What is computed, for query i in sequence b = q_seq[i] at position p = q_pos[i]:

    score[i, s] = sum_h w[i, h] * max(0, sum_d q[i, h, d] * k[b, s, d])   s <= p
    score[i, s] = -inf                                                   s >  p

Readings (pages silent):
  * one key per position is shared by all indexer heads, weighted per
    (query, head) by w;
  * no extra scale factor (a positive scalar cannot change the selection);
  * the query sees its own position (s <= p): the decode cache already holds
    the current token.
"""
from __future__ import annotations

import numpy as np


def indexer_score(q_idx, w, k_idx, q_seq, q_pos, n_cols=None) -> np.ndarray:
    """q_idx [n_q, H, D], w [n_q, H], k_idx [B, N, D], q_seq/q_pos [n_q].

    Returns float64 [n_q, n_cols] (n_cols defaults to N)."""
    q = np.asarray(q_idx, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    q_seq = np.asarray(q_seq, dtype=np.int64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    n_q = q.shape[0]
    n = k_idx.shape[1] if n_cols is None else n_cols
    out = np.full((n_q, n), -np.inf, dtype=np.float64)
    for i in range(n_q):
        length = int(q_pos[i]) + 1
        keys = np.asarray(k_idx[int(q_seq[i]), :length], dtype=np.float64)   # [L, D]
        dots = q[i] @ keys.T                                                # [H, L]
        out[i, :length] = (w[i][:, None] * np.maximum(dots, 0.0)).sum(axis=0)
    return out
