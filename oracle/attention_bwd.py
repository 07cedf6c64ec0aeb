"""Backward pass of the compressed attention (oracle; test infrastructure
only).

[P1] section 確定性內核: for training, the attention backward is made
deterministic (no split-KV; a fixed accumulation order), and every token's
output does not depend on its batch position. This module computes the exact
gradients of attention.py's forward (one softmax over the selected compressed
rows, the window rows and the sink) in float64, written out from the forward's
formula:

  qr = RoPE(q, t);  k_r = stored compressed key, or RoPE(k_raw[s], s);
  l_hr = <qr_h, k_r> / sqrt(D);  M_h = max(z_h, max_r l_hr);
  den_h = e^(z_h - M_h) + sum_r e^(l_hr - M_h);  P_hr = e^(l_hr - M_h) / den_h;
  Pz_h = e^(z_h - M_h) / den_h;  o_h = sum_r P_hr v_r.

Given dO (the gradient of a loss with respect to o):

  dP_hr = <dO_h, v_r>;  Dl_h = <dO_h, o_h>;  dS_hr = P_hr (dP_hr - Dl_h);
  d qr_h = sum_r dS_hr k_r / sqrt(D)   -> dq = RoPE(d qr, -t) (the transpose of
                                          a rotation is the opposite rotation);
  d k_r  = sum_h dS_hr qr_h / sqrt(D)  -> compressed keys as stored; window rows
                                          dk_raw[s] = RoPE(d k_r, -s);
  d v_r  = sum_h P_hr dO_h;
  d z_h  = -Pz_h Dl_h.

Rows used by several queries (a compressed entry selected by many queries of
a sequence, a raw row in many windows) add their gradients; so do the sinks
over all queries. Pinned against central finite differences of the forward.
"""
import math

import numpy as np

from .rope import apply_rope
from .compress import n_visible
from .attention import _window, seq_pos


def attend_one_bwd(q, t, keys, vals, win_k_raw, win_pos, win_v, sink, dout):
    """Gradients for one query token (all heads).

    Arguments as attention.attend_one plus dout [H, D]. Returns
    (dq [H, D], dkeys [n, D], dvals [n, D], dwin_k_raw [w, D], dwin_v [w, D],
    dsink [H]).
    """
    q = np.asarray(q, dtype=np.float64)
    H, D = q.shape
    keys = np.asarray(keys, dtype=np.float64).reshape(-1, D)
    vals = np.asarray(vals, dtype=np.float64).reshape(-1, D)
    wkr = np.asarray(win_k_raw, dtype=np.float64).reshape(-1, D)
    wv = np.asarray(win_v, dtype=np.float64).reshape(-1, D)
    dout = np.asarray(dout, dtype=np.float64)
    n, w = keys.shape[0], wkr.shape[0]
    qr = apply_rope(q, t)
    wk = apply_rope(wkr, np.asarray(win_pos)) if w else np.zeros((0, D))
    K = np.concatenate([keys, wk], axis=0)
    V = np.concatenate([vals, wv], axis=0)
    z = np.full(H, -np.inf) if sink is None else np.asarray(sink, dtype=np.float64)
    S = K.shape[0]
    if S == 0 and sink is None:
        return (np.zeros((H, D)), keys * 0, vals * 0, wkr * 0, wv * 0, np.zeros(H))
    logits = qr @ K.T / math.sqrt(D)                               # [H, S]
    lmax = logits.max(axis=1) if S else np.full(H, -np.inf)
    M = np.maximum(z, lmax)
    e = np.exp(logits - M[:, None])
    ez = np.exp(z - M)
    den = e.sum(axis=1) + ez
    P = e / den[:, None]
    Pz = ez / den
    o = P @ V
    dP = dout @ V.T                                                # [H, S]
    Dl = (dout * o).sum(axis=1)                                    # [H]
    dS = P * (dP - Dl[:, None])
    dqr = dS @ K / math.sqrt(D)
    dK = dS.T @ qr / math.sqrt(D)                                  # [S, D]
    dV = P.T @ dout
    dq = apply_rope(dqr, -t)
    dwk_raw = apply_rope(dK[n:], -np.asarray(win_pos)) if w else np.zeros((0, D))
    dsink = -Pz * Dl if sink is not None else np.zeros(H)
    return dq, dK[:n], dV[:n], dwk_raw, dV[n:], dsink


def _accumulate(q, q_pos0, k_c, v_c, rows_of, k_raw, v_raw, raw_pos0, W, sink, dout):
    q = np.asarray(q, dtype=np.float64)
    B, Lq, H, D = q.shape
    dq = np.zeros((B, Lq, H, D))
    dk_c = np.zeros(np.shape(k_c))
    dv_c = np.zeros(np.shape(v_c))
    dk_raw = np.zeros(np.shape(k_raw))
    dv_raw = np.zeros(np.shape(v_raw))
    dsink = np.zeros(H)
    T_raw = np.shape(k_raw)[1]
    for b in range(B):
        for i in range(Lq):
            t = seq_pos(q_pos0, b) + i
            sel = rows_of(b, i, t)
            pos, rr = _window(t, W, raw_pos0, T_raw)
            g = attend_one_bwd(q[b, i], t, k_c[b][sel], v_c[b][sel], k_raw[b][rr], pos, v_raw[b][rr], sink,
                               dout[b, i])
            dq[b, i] = g[0]
            np.add.at(dk_c[b], sel, g[1])
            np.add.at(dv_c[b], sel, g[2])
            np.add.at(dk_raw[b], rr, g[3])
            np.add.at(dv_raw[b], rr, g[4])
            dsink += g[5]
    return dq, dk_c, dv_c, dk_raw, dv_raw, dsink


def csa_sparse_attn_bwd(q, q_pos0, k_c, v_c, idx, k_raw, v_raw, raw_pos0, W, sink, dout):
    """Gradients of attention.csa_sparse_attn for dout [B, Lq, H, D]: returns
    (dq, dk_c, dv_c, dk_raw, dv_raw, dsink) shaped like their inputs (dsink
    [H], zero without a sink)."""
    idx = np.asarray(idx)

    def rows_of(b, i, t):
        s = idx[b, i]
        return s[s >= 0]
    return _accumulate(q, q_pos0, np.asarray(k_c, dtype=np.float64), np.asarray(v_c, dtype=np.float64), rows_of,
                       np.asarray(k_raw, dtype=np.float64), np.asarray(v_raw, dtype=np.float64), raw_pos0, W, sink,
                       np.asarray(dout, dtype=np.float64))


def hca_dense_attn_bwd(q, q_pos0, m, k_c, v_c, k_raw, v_raw, raw_pos0, W, sink, dout):
    """Gradients of attention.hca_dense_attn (every visible entry)."""
    def rows_of(b, i, t):
        return np.arange(n_visible(t, m))
    return _accumulate(q, q_pos0, np.asarray(k_c, dtype=np.float64), np.asarray(v_c, dtype=np.float64), rows_of,
                       np.asarray(k_raw, dtype=np.float64), np.asarray(v_raw, dtype=np.float64), raw_pos0, W, sink,
                       np.asarray(dout, dtype=np.float64))
