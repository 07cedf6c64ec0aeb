"""Decode state cache and incremental compression (oracle; test
infrastructure only).

[P1] section 框架層優化 (heterogeneous KV cache management) keeps two caches
apart: a state cache holding the sliding-window tokens together with the
tokens whose block is not complete yet, and the classic KV cache of
compressed entries; [P3] section 01, 异构缓存设计, names the same
heterogeneous KV cache layout for inference. [P1] section 混合注意力機制 makes an entry exist once its
block of m tokens is complete (the compressor folds whole blocks only).

Readings taken here (the pages give no layout or step order):
  * the state cache of a sequence is a ring of R raw rows (K, V and the
    indexer's raw key); the token at absolute position s lives in slot s % R,
    so R >= max(m, W + Lq - 1) keeps a block and every query's window
    resident;
  * one decode step appends the token at position pos[b] of each sequence b;
    when pos[b] + 1 is a multiple of m the step also compresses the block
    that token completes, entry j = (pos[b] + 1) // m - 1, from the block's m
    rows (compress() of the batch compressor, same gate, same RoPE position);
    an entry with j >= N_cap is not written;
  * the indexer key of the entry is the same alpha-weighted fold of the raw
    indexer keys, unrotated, stored in the indexer's format (the encoders of
    formats.py round it for fp8 / fp4).
"""
import numpy as np

from .compress import compress


def ring_rows(ring, positions):
    """Rows of a [R, D] ring for absolute positions (array)."""
    R = ring.shape[0]
    return ring[np.asarray(positions, dtype=np.int64) % R]


def state_append(pos, k_new, v_new, k_ring, v_ring, w_gate, m, k_c, v_c,
                 ki_new=None, ki_ring=None, ki_c=None):
    """One decode step for a batch, in place on float64 arrays.

    pos [B] int; k_new, v_new [B, D]; k_ring, v_ring [B, R, D]; k_c, v_c
    [B, N_cap, D]; optional ki_new [B, d], ki_ring [B, R, d], ki_c [B, N_cap, d].
    Returns the list of (b, j) entries written.
    """
    B, R, D = k_ring.shape
    N_cap = k_c.shape[1]
    assert R >= m, "the ring must hold a whole block"
    written = []
    for b in range(B):
        t = int(pos[b])
        k_ring[b, t % R] = k_new[b]
        v_ring[b, t % R] = v_new[b]
        if ki_ring is not None:
            ki_ring[b, t % R] = ki_new[b]
        if (t + 1) % m != 0:
            continue
        j = (t + 1) // m - 1
        if j >= N_cap:
            continue
        blk = np.arange(t - m + 1, t + 1)
        kr, vr = ring_rows(k_ring[b], blk), ring_rows(v_ring[b], blk)
        if ki_ring is not None:
            kc, vc, xc = compress(kr, vr, w_gate, m, pos0=j * m, x_raw=ring_rows(ki_ring[b], blk))
            ki_c[b, j] = xc[0]
        else:
            kc, vc = compress(kr, vr, w_gate, m, pos0=j * m)
        k_c[b, j] = kc[0]
        v_c[b, j] = vc[0]
        written.append((b, j))
    return written
