"""KV compressor (oracle; test infrastructure only).

[P1] section 混合注意力機制: CSA folds the KV of every m = 4 consecutive tokens
into one entry, so the sequence shrinks to 1/m; HCA does the same with
m' = 128 and attends densely. [P3] section 01 says both compress the KV cache
along the sequence dimension. The pages do not define the folding; this build
takes a softmax-gated weighted sum over each block:

  for block j covering absolute positions s = j*m .. j*m+m-1:
      g_s   = <w_gate, K_raw[s]>           (one scalar gate per token, pre-RoPE K)
      alpha = softmax over the m gates     (max-subtracted)
      K_c[j] = RoPE( sum_s alpha_s K_raw[s],  p_j = j*m + m - 1 )
      V_c[j] = sum_s alpha_s V_raw[s]

Readings: blocks are aligned to absolute multiples of m (the caller's first
position pos0 must be a multiple of m); only complete blocks produce an entry
(the state cache of [P1] section 框架層優化 holds tokens not yet compressed);
the compressed key is rotated at the position of its block's last token, the
first position at which the entry exists (with m = 1 this is the raw position).
"""
import numpy as np

from .rope import apply_rope


def compress(k_raw, v_raw, w_gate, m, pos0=0, x_raw=None):
    """Compress raw rows of one sequence.

    k_raw, v_raw: [T, D] float64 (pre-RoPE keys, values) at absolute positions
    pos0 .. pos0+T-1. w_gate: [D]. Returns (k_c, v_c), each [T // m, D]; row i
    is the block whose absolute index is pos0 // m + i.

    x_raw: optional [T, d] rows of another per-token tensor (the indexer's raw
    keys) folded with the same block weights alpha and not rotated (the
    indexer has no positional rotation); then (k_c, v_c, x_c) is returned.
    """
    k_raw = np.asarray(k_raw, dtype=np.float64)
    v_raw = np.asarray(v_raw, dtype=np.float64)
    w_gate = np.asarray(w_gate, dtype=np.float64)
    assert pos0 % m == 0, "blocks are aligned to absolute multiples of m"
    T, D = k_raw.shape
    nb = T // m
    k_c = np.zeros((nb, D))
    v_c = np.zeros((nb, D))
    if x_raw is not None:
        x_raw = np.asarray(x_raw, dtype=np.float64)
        x_c = np.zeros((nb, x_raw.shape[1]))
    for i in range(nb):
        ks = k_raw[i * m:(i + 1) * m]
        vs = v_raw[i * m:(i + 1) * m]
        g = ks @ w_gate
        e = np.exp(g - g.max())
        alpha = e / e.sum()
        j = pos0 // m + i
        k_c[i] = apply_rope(alpha @ ks, j * m + m - 1)
        v_c[i] = alpha @ vs
        if x_raw is not None:
            x_c[i] = alpha @ x_raw[i * m:(i + 1) * m]
    if x_raw is not None:
        return k_c, v_c, x_c
    return k_c, v_c


def n_visible(t, m):
    """Number of compressed entries a query at absolute position t may see.

    Entry j exists once its last token j*m+m-1 has been seen: j*m+m-1 <= t.
    """
    return (t + 1) // m
