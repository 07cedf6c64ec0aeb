"""Partial rotary position embedding (oracle; test infrastructure only).

[P1] section 混合注意力機制 (engineering highlights) says RoPE is applied to the
last 64 dimensions only, to keep relative-position information. The pages give
no base, pairing or scaling, so this build reads it as:

  * rotated dims: D-64 .. D-1 of a D-dim vector; dims 0 .. D-65 untouched;
  * pairs are interleaved: (D-64+2i, D-64+2i+1) for i = 0..31;
  * frequency theta_i = 10000 ** (-i/32) (the common base, no scaling);
  * the pair at position p is rotated by the angle p * theta_i:
        (x0, x1) -> (x0 cos a - x1 sin a, x0 sin a + x1 cos a).

Everything is float64 and p is an exact integer.
"""
import numpy as np

ROPE_DIMS = 64
ROPE_BASE = 10000.0


def inv_freq():
    """theta_i for i = 0..31."""
    i = np.arange(ROPE_DIMS // 2, dtype=np.float64)
    return ROPE_BASE ** (-i / (ROPE_DIMS // 2))


def apply_rope(x, pos):
    """Rotate the last 64 dims of x[..., D] by position(s) pos.

    pos is a scalar or an integer array broadcastable to x.shape[:-1].
    Returns a new float64 array.
    """
    x = np.array(x, dtype=np.float64, copy=True)
    D = x.shape[-1]
    assert D >= ROPE_DIMS
    p = np.asarray(pos, dtype=np.float64)[..., None]          # [..., 1]
    ang = p * inv_freq()                                      # [..., 32]
    c, s = np.cos(ang), np.sin(ang)
    x0 = x[..., D - ROPE_DIMS + 0::2].copy()
    x1 = x[..., D - ROPE_DIMS + 1::2].copy()
    x[..., D - ROPE_DIMS + 0::2] = x0 * c - x1 * s
    x[..., D - ROPE_DIMS + 1::2] = x0 * s + x1 * c
    return x
