"""Compressed attention with window branch and attention sink (oracle; test
infrastructure only).

[P1] section 混合注意力機制:
  * CSA: each query attends the k compressed entries its indexer selected;
  * HCA: each query attends every compressed entry (dense), with m' = 128;
  * engineering highlights: RoPE on the last 64 dims, a sliding-window branch
    over raw recent tokens for local detail, and an attention sink so that a
    query's attention weights need not add up to one.
[P5] section 3 混合注意力机制 repeats CSA (compress then sparse) and HCA (very
high compression, dense).

Readings taken here (the pages give no formula):
  * one shared KV head, H query heads; logits are <RoPE(q, t), key> / sqrt(D);
  * compressed keys are stored already rotated (at their block's last token);
    raw window keys are rotated at their own position s;
  * the window is the W raw tokens s = t-W+1 .. t (clipped at 0), t included;
    window rows and compressed entries share one softmax; rows that cover the
    same tokens are not de-duplicated;
  * the sink is one unscaled logit z_h per head that joins the softmax
    denominator with a zero value; absent sink = -inf;
  * with no source and no sink the output is 0 and lse is -inf.

Per-sequence positions and the state cache (see state.py): q_pos0 may be one
position for the batch or one per sequence ([B]); query row i of sequence b
is at q_pos0[b] + i. With ring=True the raw rows are a ring of R = T_raw
slots, position s in slot s % R, and raw_pos0 is not used.

Returned lse = M + ln(e^(z-M) + sum e^(l-M)), M = max(z, max l).
"""
import math

import numpy as np

from .rope import apply_rope
from .compress import n_visible


def attend_one(q, t, keys, vals, win_k_raw, win_pos, win_v, sink):
    """One query token, all heads.

    q: [H, D] (pre-RoPE); keys/vals: [n, D] compressed rows (keys rotated);
    win_k_raw/win_v: [w, D] raw rows at absolute positions win_pos [w];
    sink: [H] or None. Returns (o [H, D], lse [H]).
    """
    q = np.asarray(q, dtype=np.float64)
    H, D = q.shape
    qr = apply_rope(q, t)
    wk = apply_rope(win_k_raw, np.asarray(win_pos)) if len(win_pos) else np.zeros((0, D))
    K = np.concatenate([np.asarray(keys, dtype=np.float64).reshape(-1, D), wk], axis=0)
    V = np.concatenate([np.asarray(vals, dtype=np.float64).reshape(-1, D),
                        np.asarray(win_v, dtype=np.float64).reshape(-1, D)], axis=0)
    logits = qr @ K.T / math.sqrt(D)                          # [H, n+w]
    z = np.full(H, -np.inf) if sink is None else np.asarray(sink, dtype=np.float64)
    if logits.shape[1] == 0 and sink is None:
        return np.zeros((H, D)), np.full(H, -np.inf)
    lmax = logits.max(axis=1) if logits.shape[1] else np.full(H, -np.inf)
    M = np.maximum(z, lmax)
    p = np.exp(logits - M[:, None])
    den = p.sum(axis=1) + np.exp(z - M)
    o = (p @ V) / den[:, None]
    lse = M + np.log(den)
    return o, lse


def _window(t, W, raw_pos0, T_raw, ring=False):
    """Absolute positions of the window of a query at t, and their raw rows."""
    lo = max(0, t - W + 1)
    pos = np.arange(lo, t + 1) if W > 0 else np.arange(0)
    if ring:
        assert len(pos) <= T_raw, "window longer than the ring"
        return pos, pos % T_raw
    if len(pos):
        assert pos[0] >= raw_pos0 and pos[-1] - raw_pos0 < T_raw, "raw window not covered"
    return pos, pos - raw_pos0


def seq_pos(q_pos0, b):
    """Position of query row 0 of sequence b (one for all, or per sequence)."""
    return int(q_pos0) if np.ndim(q_pos0) == 0 else int(np.asarray(q_pos0)[b])


def csa_sparse_attn(q, q_pos0, k_c, v_c, idx, k_raw, v_raw, raw_pos0, W, sink, ring=False):
    """CSA attention for a batch.

    q [B, Lq, H, D]; k_c, v_c [B, N, D]; idx [B, Lq, k] (-1 = unused slot);
    k_raw, v_raw [B, T_raw, D] at absolute positions raw_pos0 ..; sink [H] or
    None. Query row i is at absolute position q_pos0 + i.
    Returns out [B, Lq, H, D], lse [B, Lq, H] (float64).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Lq, H, D = q.shape
    out = np.zeros((B, Lq, H, D))
    lse = np.zeros((B, Lq, H))
    T_raw = k_raw.shape[1]
    for b in range(B):
        for i in range(Lq):
            t = seq_pos(q_pos0, b) + i
            sel = np.asarray(idx[b, i])
            sel = sel[sel >= 0]
            pos, rows = _window(t, W, raw_pos0, T_raw, ring)
            out[b, i], lse[b, i] = attend_one(
                q[b, i], t, k_c[b][sel], v_c[b][sel],
                k_raw[b][rows], pos, v_raw[b][rows], sink)
    return out, lse


def hca_dense_attn(q, q_pos0, m, k_c, v_c, k_raw, v_raw, raw_pos0, W, sink, ring=False):
    """HCA attention for a batch: every visible compressed entry j < (t+1)//m,
    plus the window and the sink. Shapes as in csa_sparse_attn."""
    q = np.asarray(q, dtype=np.float64)
    B, Lq, H, D = q.shape
    out = np.zeros((B, Lq, H, D))
    lse = np.zeros((B, Lq, H))
    T_raw = k_raw.shape[1]
    for b in range(B):
        for i in range(Lq):
            t = seq_pos(q_pos0, b) + i
            n = n_visible(t, m)
            assert n <= k_c.shape[1], "compressed cache does not hold every visible entry"
            pos, rows = _window(t, W, raw_pos0, T_raw, ring)
            out[b, i], lse[b, i] = attend_one(
                q[b, i], t, k_c[b][:n], v_c[b][:n],
                k_raw[b][rows], pos, v_raw[b][rows], sink)
    return out, lse
