"""Causal top-K selection (K = 2048). Oracle only.

Pages: "GLM-5.2 架构深度拆解" CH2 §2.2 and §1.1 (index_topk = 2048): the F layer
keeps the 2048 highest-scoring positions as the sparse set of that layer's
attention; "GLM-5.2 总览" tbl-glm52-config (top-K = 2048).

For query i with position p, among positions s = 0..p:
  * keep the min(K, p + 1) positions with the largest scores;
  * ties are broken toward the lower position (order by (-score, s));
  * return the kept positions in ascending order, padded with -1 to K.

Readings (pages silent): the tie rule, the ascending output order, and the
-1 padding when fewer than K positions exist. With them the selected set is
unique. Scores compare as the floats they are (so -0.0 ties with +0.0).
"""
from __future__ import annotations

import numpy as np


def topk_select(scores, q_pos, k: int = 2048) -> np.ndarray:
    scores = np.asarray(scores)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    n_q = scores.shape[0]
    out = np.full((n_q, k), -1, dtype=np.int32)
    for i in range(n_q):
        length = int(q_pos[i]) + 1
        s = scores[i, :length]
        pos = np.arange(length)
        order = np.lexsort((pos, -s))          # primary key -score, then position
        kept = np.sort(order[: min(k, length)])
        out[i, : kept.size] = kept
    return out


def group_max(scores, n_cols=None, group: int = 32) -> np.ndarray:
    """The largest score of every run of `group` consecutive columns of each row
    (columns [group*g, group*g + group) below n_cols; the last run may be
    shorter), with -0.0 reported as +0.0.

    Not a quantity of the pages: the library's score call can also return these
    maxima, which its top-k uses to pass over scores that cannot be selected.
    The oracle states them so that this output can be checked."""
    scores = np.asarray(scores, dtype=np.float64)
    n_q, n = scores.shape
    n_cols = n if n_cols is None else int(n_cols)
    n_groups = -(-n_cols // group)
    out = np.empty((n_q, n_groups), dtype=np.float64)
    for g in range(n_groups):
        out[:, g] = scores[:, group * g: min(group * g + group, n_cols)].max(axis=1)
    return out + 0.0                                   # -0.0 + 0.0 = +0.0
