"""Lightning Indexer scores (oracle; test infrastructure only).

[P1] section 混合注意力機制 introduces a light indexer that picks the important
compressed blocks for each query; [P1] section FP4 量化 runs its QK path in FP4.
The pages give no formula. This build reads it as a low-dimensional dot product
per indexer head, passed through ReLU and mixed with per-query head weights:

    I[t, j] = sum_h  w[t, h] * max(0, <q_I[t, h, :], k_I[j, :]>)

with no scale and no positional rotation. q_I, w and k_I are inputs (their
projections need trained weights, which are not part of this path).
"""
import numpy as np


def _pos(q_pos0, b):
    return int(q_pos0) if np.ndim(q_pos0) == 0 else int(np.asarray(q_pos0)[b])


def index_scores(q_i, w_i, k_i):
    """Scores of one query against n entries.

    q_i: [H_I, d_I], w_i: [H_I], k_i: [n, d_I] (float64). Returns [n].
    """
    q_i = np.asarray(q_i, dtype=np.float64)
    w_i = np.asarray(w_i, dtype=np.float64)
    k_i = np.asarray(k_i, dtype=np.float64)
    dots = k_i @ q_i.T                      # [n, H_I]
    return np.maximum(dots, 0.0) @ w_i      # [n]


def index_scores_batch(q_i, w_i, k_i, q_pos0, m):
    """Scores for a batch, with -inf where an entry is not yet visible.

    q_i [B, Lq, H_I, d_I], w_i [B, Lq, H_I], k_i [B, N, d_I] (float64).
    Returns [B, Lq, N]; query row i is at absolute position q_pos0 + i and
    sees entries j < (q_pos0 + i + 1) // m. q_pos0 is one position for the
    batch or one per sequence ([B]).
    """
    q_i = np.asarray(q_i, dtype=np.float64)
    B, Lq = q_i.shape[:2]
    N = k_i.shape[1]
    out = np.full((B, Lq, N), -np.inf)
    for b in range(B):
        for i in range(Lq):
            n = (_pos(q_pos0, b) + i + 1) // m
            assert n <= N, "indexer key cache does not hold every visible entry"
            out[b, i, :n] = index_scores(q_i[b, i], w_i[b, i], k_i[b, :n])
    return out
