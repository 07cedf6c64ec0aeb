"""Per-query top-k selection (oracle; test infrastructure only).

[P1] section 混合注意力機制: each query attends only k compressed entries
(k = 512..1024) chosen by the indexer. Tie-breaking, output order and padding
are not on the pages; this build fixes them:

  * the order key is (-score, j): larger score first, equal scores by lower j;
    -0.0 and +0.0 are the same score;
  * the first min(k, n) entries of that order are selected, n = visible entries;
  * they are emitted in ascending j, and the rest of the k slots hold -1.
"""
import numpy as np

from .formats import round_bf16


def topk_select(scores, k):
    """scores: [n] finite floats of the visible entries. Returns int64 [k]."""
    s = np.asarray(scores, dtype=np.float64)
    assert np.all(np.isfinite(s)), "scores must be finite"
    s = np.where(s == 0.0, 0.0, s)          # -0 -> +0
    n = s.shape[0]
    j = np.arange(n)
    order = np.lexsort((j, -s))             # primary -s, secondary j
    take = min(k, n)
    sel = np.sort(order[:take])
    out = np.full(k, -1, dtype=np.int64)
    out[:take] = sel
    return out


def topk_batch(scores, k, q_pos0, m):
    """scores [B, Lq, N] -> idx [B, Lq, k]; query row i sees j < (q_pos0+i+1)//m
    (q_pos0 one position for the batch or one per sequence, [B])."""
    B, Lq, N = scores.shape
    out = np.full((B, Lq, k), -1, dtype=np.int64)
    for b in range(B):
        for i in range(Lq):
            n = ((int(q_pos0) if np.ndim(q_pos0) == 0 else int(np.asarray(q_pos0)[b])) + i + 1) // m
            assert n <= N, "score row does not hold every visible entry"
            out[b, i] = topk_select(scores[b, i, :n], k)
    return out


def topk_batch_bf16(scores, k, q_pos0, m):
    """[P1] section FP4 量化: the indexer scores rounded from FP32 to BF16.
    The top-k of the rounded scores (nearest even) under the same rule, so
    entries whose scores round alike are ordered by index."""
    s = np.asarray(scores, dtype=np.float64)
    fin = np.isfinite(s)
    r = np.where(fin, round_bf16(np.where(fin, s, 0.0)), s)
    return topk_batch(r, k, q_pos0, m)
